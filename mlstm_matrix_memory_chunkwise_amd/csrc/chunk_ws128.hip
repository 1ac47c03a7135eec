// Fused chunkwise mLSTM forward at chunk 128, bf16 MFMA, d_qk 256: a state
// group and a score group of waves, pipelined by one chunk.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form" inside
// chunks of 128 tokens, the state of "Associative Matrix Cell State" carried
// between chunks, the running maximum of section 2 "The Normalizer State and
// Numerical Stabilization".  The chunk algebra is the one of chunk_mfma.hip:
//   u_j = i~_j - b_j,  M_i = max(m_s, max_{j<=i} u_j),  m_i = b_i + M_i
//   D_ij = exp(u_j - M_i),  g_i = exp(m_s - M_i),  w_j = exp(u_j - M_L)
//   h_i = sigmoid(o~_i) (.) (g_i q_i^T C~_s + sum_j D_ij (q_i.k_j) v_j)
//         / max(|g_i q_i.n~_s + sum_j D_ij (q_i.k_j)|, exp(-m_i))
//   C~ <- g_L C~ + K^T diag(w) V,  n~ <- g_L n~ + K^T w.
//
// A workgroup (8 waves) owns one (head, 64 value columns) pair and walks the
// chunks in order, one wave of each role per SIMD:
// * state waves 0..3 (16 value columns each) keep C~ in registers and, per
//   32-row d_qk slice ("stage", eight per chunk), run the readout C~^T Q^T
//   (C~ as a high/remainder bf16 pair), the update K^T (w V), and a quarter
//   of the normaliser increment K^T w (w as three bf16 terms, so the sum
//   keeps about 24 bits); at the end of a chunk they leave the scaled
//   readout in LDS.  They also issue every global->LDS load, D stages ahead,
//   with compile-time vmcnt waits.
// * score waves 4..7: wave 4 + V owns query tiles V and 7 - V (nine causal
//   16x16 score tiles per wave) and accumulates S^T = K Q^T and q.n~ over
//   the stages of chunk c.  At the chunk's last stage it forms P = S (.) D
//   and the row sums in registers (its second query tile at the first stage
//   of the next chunk): the MFMA output of S^T, with the keys of
//   a 32-key step taken in the order (4g..4g+3, 16+4g..16+4g+3), is the B
//   operand of P V as it stands (the value fragments are read in the same
//   key order), so P never goes through LDS.  During the first stages of
//   chunk c + 1 the wave finishes chunk c: P V onto the scaled readout, the
//   denominators, the output gate (float32 o~ copied global -> LDS at
//   stage 1 into the wave's part of the scaled-readout buffer, which is free
//   until stage 7; bfloat16 o~ read straight into registers at the chunk's
//   last stage) and h.  Waves 5 and 6 also fold the normaliser
//   increments into n~, half of the rows each, at stages where they are
//   idle; wave 7 runs the gate scan of the next chunk.
// The finishing work of one chunk (vector ALU) thus overlaps the MFMA work
// of the next on every SIMD.
//
// LDS (~149 KB): a ring of four [128 x 32] q/k slice pairs (64 KB), two
// value tiles (the score waves read chunk c's during chunk c + 1 while chunk
// c + 2's lands), the scaled readout (32 KB), the gates by chunk mod 3 and n~
// by chunk parity.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int NTH = 512;
constexpr int TV = 64;              // value columns per workgroup
constexpr int L = 128;              // chunk
constexpr int NT = L / 16;          // 16-token tiles
constexpr int NKS = L / 32;         // 32-token k-steps
constexpr int DQK = 256;
constexpr int AS = 32;              // d_qk rows per stage
constexpr int NS = DQK / AS;        // stages per chunk
constexpr int NCT = DQK / 16;       // 16-row C~ tiles per state wave
constexpr int QKT = L * AS * 2;     // bytes of one [128 x 32] bf16 slice
constexpr int VTB = L * TV * 2;     // bytes of the [128 x 64] value tile
constexpr int D = 3;                // stages in flight
constexpr int NSLOT = D + 1;
constexpr int NB_QK = 2 * QKT / 1024 / 4;   // 1 KB loads per loading wave per stage
constexpr int NB_V = VTB / 1024 / 4;        // ... per value tile
constexpr int NB_G = 1;                     // 256 B gate loads per loading wave per chunk
constexpr int O_STAGE = 7;          // stage of chunk c at which chunk c's o~ is read
constexpr int SCAN_WAVE = 7;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte offset of element (row, col) of a [rows x 32] bf16 slice with 64-byte
// rows whose 16-byte chunks are XOR-swizzled by (row / 2) mod 4: the 16 rows
// of an MFMA fragment cover every bank once.
__device__ __forceinline__ int swz4(int row, int col) {
  return row * 64 + 16 * ((col >> 3) ^ ((row >> 1) & 3)) + 2 * (col & 7);
}

__device__ __forceinline__ float rl63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Wait at the top of stage slice s for that stage's loads (folds to one
// s_waitcnt once the stage loop is unrolled).
__device__ __forceinline__ void wait_stage8(int s) {
  switch (s) {
    case 0: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(0)>(); break;
    case 1: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(1)>(); break;
    case 2: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(2)>(); break;
    case 3: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(3)>(); break;
    case 4: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(4)>(); break;
    case 5: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(5)>(); break;
    case 6: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(6)>(); break;
    default: wait_vm<loads_after_stage<NS, D, NB_QK, NB_V, NB_G>(7)>(); break;
  }
}

// Loads issued by one loading wave after those of stage x + 1, counted at the
// top of stage x (slice s) before that stage's own issue: the stage loads of
// x + 2 .. x + D - 1 and the gate loads at the tops of stages x + 1 - D ..
// x - 1 that open a chunk.
template <int NS_, int D_, int NBQK, int NBV, int NBX>
__host__ __device__ constexpr int loads_after_next_stage(int s) {
  int n = 0;
  for (int k = 2; k < D_; ++k) n += NBQK + (((s + k) % NS_) == 0 ? NBV : 0);
  for (int j = 1; j < D_; ++j) n += (((s - j) % NS_ + NS_) % NS_ == 0) ? NBX : 0;
  return n;
}
__device__ __forceinline__ void wait_next_stage8(int s) {
  switch (s) {
    case 0: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(0)>(); break;
    case 1: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(1)>(); break;
    case 2: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(2)>(); break;
    case 3: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(3)>(); break;
    case 4: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(4)>(); break;
    case 5: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(5)>(); break;
    case 6: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(6)>(); break;
    default: wait_vm<loads_after_next_stage<NS, D, NB_QK, NB_V, NB_G>(7)>(); break;
  }
}

template <int OM>
__global__ __launch_bounds__(NTH, 1) void chunk_ws128_kernel(SeqArgs a) {
  __shared__ __align__(1024) char sRing[NSLOT][2][QKT];   // [slot][q|k]
  __shared__ __align__(1024) char sV[2][VTB];             // value tile by chunk parity
  __shared__ __align__(16) float sR[4][NT][64][4];        // scaled readout [col tile][query tile]
  __shared__ __align__(16) float sGate[3][6][L];          // u, M, g, exp(-m), w / sig', w by chunk mod 3
  __shared__ __align__(16) bf16_t sWs[3][4][L];           // w as three bf16 terms and a zero row
  __shared__ __align__(16) float sN[2][DQK];              // n~ at the chunk start, by parity
  __shared__ __align__(16) bf16_t sNs[2][4][DQK];         // ... as three bf16 terms and a zero row
  __shared__ __align__(16) float sNp[2][DQK];             // K^T w of the chunk, two partial sums
  __shared__ __align__(256) float sGin[2][2][L];          // raw gates [chunk parity][i~ | f~]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const bool state_wave = wave < 4;
  const int cg = wave & 3;
  const int kr = l16 >> 2, kq = l16 & 3;

  // ---- workgroup -> (head, value tile); a head's tiles share one XCD
  const int nvt = static_cast<int>(a.dv / TV);
  const int64_t nhead = a.B * a.H;
  int64_t head;
  int vt;
  {
    const int64_t w = blockIdx.x;
    if (nhead % 8 == 0) {
      const int64_t grp = w / (8 * nvt), r = w % (8 * nvt);
      vt = static_cast<int>(r / 8);
      head = grp * 8 + r % 8;
    } else {
      head = w / nvt;
      vt = static_cast<int>(w % nvt);
    }
  }
  const int dv = static_cast<int>(a.dv);
  const int64_t Ts = a.Ts;
  const int nchunks = static_cast<int>(a.T / L);

  const bf16_t* gq = static_cast<const bf16_t*>(a.q) + head * Ts * DQK;
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * Ts * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * Ts * dv + vt * TV;
  const float* gi = a.i_pre + head * Ts;
  const float* gf = a.f_pre + head * Ts;

  if (tid < DQK) {
    const float n0 = a.C0 ? a.n0[head * DQK + tid] : 0.0f;
    sN[0][tid] = n0;
    split3_bf16(n0, sNs[0][0][tid], sNs[0][1][tid], sNs[0][2][tid]);
    sNs[0][3][tid] = 0;
    sNs[1][3][tid] = 0;
  }
  if (tid < 3 * L) sWs[tid / L][3][tid % L] = 0;
  float m_s = a.C0 ? a.m0[head] : 0.0f;

  // ---- loads, issued by the state waves (lw = 0..3).  Lane l of a 1 KB
  // slice load writes row 16 G + l/4, physical chunk l%4 of its tile, which
  // holds logical chunk (l%4) ^ ((row/2)%4); a value-tile load writes row
  // 8 G + l/8 with the 8-chunk swizzle of swz().
  const int lw = cg;
  int qk_off[NB_QK];
#pragma unroll
  for (int m = 0; m < NB_QK; ++m) {
    const int Gr = (lw * NB_QK + m) & 7;
    const int row = 16 * Gr + (lane >> 2);
    qk_off[m] = row * DQK + 8 * ((lane & 3) ^ ((row >> 1) & 3));
  }
  int v_off[NB_V];
#pragma unroll
  for (int m = 0; m < NB_V; ++m) {
    const int row = 8 * (lw * NB_V + m) + (lane >> 3);
    v_off[m] = row * dv + 8 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  auto issue_stage = [&](int x) {
    const int cx = x / NS, sx = x % NS;
    const int cc = cx < nchunks ? cx : nchunks - 1;   // past the end: harmless re-read
    char* slot = sRing[x % NSLOT][0];
    const int64_t base = static_cast<int64_t>(cc) * L * DQK + sx * AS;
#pragma unroll
    for (int m = 0; m < NB_QK; ++m) {
      const int G = lw * NB_QK + m;
      const int mat = G >> 3;
      dma16_s((mat ? gk : gq) + base, static_cast<uint32_t>(2 * qk_off[m]),
              lds_addr(slot + mat * QKT + (G & 7) * 1024));
    }
    if (sx == 0) {
      // (a past-the-end value tile lands in the slot of chunk nchunks - 2,
      // whose last reader finished before this stage's barrier)
#pragma unroll
      for (int m = 0; m < NB_V; ++m)
        dma16_nt_s(gv + static_cast<int64_t>(cc) * L * dv, static_cast<uint32_t>(2 * v_off[m]),
                   lds_addr(sV[cx & 1] + (lw * NB_V + m) * 1024));
    }
  };
  // each loading wave brings one quarter of the gates of chunk c + 2
  const float* gsrc = (lw & 1) ? gf : gi;
  const int ghalf = 64 * (lw >> 1);
  auto issue_gates = [&](int c) {
    const int cn = (c + 2 < nchunks) ? c + 2 : nchunks - 1;
    dma4(gsrc + static_cast<int64_t>(cn) * L + ghalf + lane, lds_addr(&sGin[c & 1][lw & 1][ghalf]));
  };

  // Gate scan of one chunk (raw gates gin) into sGate[gb] / sWs[gb], in four
  // parts; ms and sg are m and the state scale before the chunk.  The last
  // part yields m and the state scale after it.
  struct GScan {
    float xi[2], lf[2], bc[2], u[2], Mx[2], ML, bL;
  };
  auto scan_part = [&](int part, int gin, int gb, float ms, float sg, GScan& x, float& m_after,
                       float& sg_after) {
    if (part == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x.xi[h] = sGin[gin][0][lane + 64 * h];
        x.lf[h] = log_forget_fast(sGin[gin][1][lane + 64 * h], a.fgate_exp);
      }
    } else if (part == 1) {
      x.bc[0] = scan_add(x.lf[0]);
      x.bc[1] = scan_add(x.lf[1]) + rl63(x.bc[0]);
#pragma unroll
      for (int h = 0; h < 2; ++h) x.u[h] = x.xi[h] - x.bc[h];
    } else if (part == 2) {
      x.Mx[0] = fmaxf(ms, scan_max(x.u[0]));
      x.Mx[1] = fmaxf(rl63(x.Mx[0]), scan_max(x.u[1]));
      x.ML = rl63(x.Mx[1]);
      x.bL = rl63(x.bc[1]);
    } else {
      float gv_[2], wv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        gv_[h] = __expf(ms - x.Mx[h]);
        wv[h] = __expf(x.u[h] - x.ML);
      }
      const float gLn = rl63(gv_[1]);
      const float sg_new = gLn * sg < 0x1p-64f ? 1.0f : gLn * sg;
      const float rsg = __builtin_amdgcn_rcpf(sg_new);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        sGate[gb][0][j] = x.u[h];
        sGate[gb][1][j] = x.Mx[h];
        sGate[gb][2][j] = gv_[h];
        sGate[gb][3][j] = __expf(-(x.bc[h] + x.Mx[h]));
        sGate[gb][4][j] = wv[h] * rsg;
        sGate[gb][5][j] = wv[h];
        split3_bf16(wv[h], sWs[gb][0][j], sWs[gb][1][j], sWs[gb][2][j]);
      }
      m_after = x.bL + x.ML;
      sg_after = sg_new;
    }
  };

  // ---- prologue: stages 0 .. D-1 and the gates of chunks 0, 1 in flight,
  // chunk 0's gates scanned
  if (state_wave) {
#pragma unroll
    for (int x = 0; x < D; ++x) issue_stage(x);
    dma4(gsrc + ghalf + lane, lds_addr(&sGin[0][lw & 1][ghalf]));
    dma4(gsrc + (nchunks > 1 ? L : 0) + ghalf + lane, lds_addr(&sGin[1][lw & 1][ghalf]));
    wait_vm<0>();
  }
  __syncthreads();
  float m_n1 = 0.0f, sg1 = 1.0f;   // scan wave: m and state scale after the current chunk
  if (wave == SCAN_WAVE) {
    GScan x;
#pragma unroll
    for (int part = 0; part < 4; ++part) scan_part(part, 0, 0, m_s, 1.0f, x, m_n1, sg1);
  }
  __syncthreads();

  if (state_wave) {
    const int W = cg;
    const int b0w = vt * TV + W * 16;
    // C~ of this wave's 16 columns: tile t holds rows 32 (t/2) + 8 g + 4 (t%2) + e
    f32x4 cacc[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) cacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.C0) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
          cacc[t][e] = a.C0[(head * DQK + arow) * dv + b0w + l16];
        }
      }
    }
    // Wait for these loads here: the compiler does not see the asm loads of
    // the ring, and with the C~ loads still counted as pending in the loop it
    // places waits at the first use of each row tile whose counts, once the
    // ring's loads are in flight, would wait for those too (down to vmcnt(0)
    // at the last stage of every chunk).
    wait_vm<0>();
    float sig = 1.0f;   // C~ = sig * cacc
    f32x4 outT[NT];
    bf16x8 wVf[NKS];
    // the normaliser partial of this wave: row tile nj of every slice, the
    // k-steps nk and nk + 2
    const int nj = W & 1, nk = W >> 1;
    int gb = 0;
    // Q fragments of the first half of the query tiles of the next stage,
    // read at the end of the stage before (the loading waves wait for the
    // loads of stage x + 1 at the top of stage x, so that stage's barrier
    // publishes them)
    uint4 QfN[NT / 2];
#pragma unroll
    for (int it = 0; it < NT / 2; ++it) QfN[it] = lds_ld16(sRing[0][0], swz4(it * 16 + l16, 8 * g));
    for (int c = 0; c < nchunks; ++c) {
      float gL = 0.0f, sig_new = 0.0f;
      bool renorm = false;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int x = c * NS + s;
        if (x + 1 >= D) wait_next_stage8(s);
        __syncthreads();
        issue_stage(x + D);
        if (s == 0) issue_gates(c);
        const char* Qb = sRing[x % NSLOT][0];
        const char* Kb = sRing[x % NSLOT][1];
        if (s == 0) {
          gL = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sGate[gb][2][L - 1])));
          renorm = gL * sig < 0x1p-64f;
          sig_new = renorm ? 1.0f : gL * sig;
          // w V (w / sig' from the scan) as the update's B operand: lane
          // (g, c) holds tokens 32 ks + 8 g + 0..7 of column 16 W + c
          const char* Vb = sV[c & 1];
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int col = W * 16 + 4 * kq;
            const uint2 lo = lds_tr(Vb, swz(32 * ks + 8 * g + kr, col));
            const uint2 hi = lds_tr(Vb, swz(32 * ks + 8 * g + 4 + kr, col));
            const float4 w0 = *reinterpret_cast<const float4*>(&sGate[gb][4][32 * ks + 8 * g]);
            const float4 w1 = *reinterpret_cast<const float4*>(&sGate[gb][4][32 * ks + 8 * g + 4]);
            float xw[8];
            xw[0] = bf_lo(lo.x) * w0.x; xw[1] = bf_hi(lo.x) * w0.y;
            xw[2] = bf_lo(lo.y) * w0.z; xw[3] = bf_hi(lo.y) * w0.w;
            xw[4] = bf_lo(hi.x) * w1.x; xw[5] = bf_hi(hi.x) * w1.y;
            xw[6] = bf_lo(hi.y) * w1.z; xw[7] = bf_hi(hi.y) * w1.w;
            wVf[ks] = cvt8(xw);
          }
#pragma unroll
          for (int it = 0; it < NT; ++it) outT[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // readout of the slice's rows (C~ as a high/remainder bf16 pair:
        // bf16 alone costs up to ~2% of h where the carried and in-chunk
        // terms cancel) on the Q fragments of every query tile
        bf16x8 Ahi, Alo;
        {
          float ca[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ca[e] = cacc[2 * s][e];
            ca[4 + e] = cacc[2 * s + 1][e];
          }
          cvt8_split(ca, Ahi, Alo);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint4 Qf[NT / 2];
#pragma unroll
          for (int it = 0; it < NT / 2; ++it)
            Qf[it] = h2 == 0 ? QfN[it] : lds_ld16(Qb, swz4((4 * h2 + it) * 16 + l16, 8 * g));
#pragma unroll
          for (int it = 0; it < NT / 2; ++it)
            outT[4 * h2 + it] = mfma16x16x32(Ahi, as_bf16x8(Qf[it]), outT[4 * h2 + it]);
#pragma unroll
          for (int it = 0; it < NT / 2; ++it)
            outT[4 * h2 + it] = mfma16x16x32(Alo, as_bf16x8(Qf[it]), outT[4 * h2 + it]);
        }
        // then their update on the K^T fragments of the slice's two row tiles
        // (lane c of tile j holds d_qk row 8 (c/4) + 4 j + c%4 of the slice)
        bf16x8 Kt[NKS][2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = 8 * kq + 4 * j;
            Kt[ks][j] = join(lds_tr(Kb, swz4(32 * ks + 8 * g + kr, col)),
                             lds_tr(Kb, swz4(32 * ks + 8 * g + 4 + kr, col)));
          }
        }
        if (renorm) {
          const float f = gL * sig;
          cacc[2 * s] *= f;
          cacc[2 * s + 1] *= f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int j = 0; j < 2; ++j) cacc[2 * s + j] = mfma16x16x32(Kt[ks][j], wVf[ks], cacc[2 * s + j]);
        }
        // normaliser increment: A rows 4r + e hold term e of w (row 4r + 3
        // zero), B = the K^T fragment, so D[4r + e][c] is term e of
        // sum_j w_j K[j][row c]
        {
          // (the K^T fragments of k-steps nk, nk + 2 and row tile nj, read
          // again from LDS rather than selected among registers)
          const int ncol = 8 * kq + 4 * nj;
          const bf16x8 B0 = join(lds_tr(Kb, swz4(32 * nk + 8 * g + kr, ncol)),
                                 lds_tr(Kb, swz4(32 * nk + 8 * g + 4 + kr, ncol)));
          const bf16x8 B1 = join(lds_tr(Kb, swz4(32 * (nk + 2) + 8 * g + kr, ncol)),
                                 lds_tr(Kb, swz4(32 * (nk + 2) + 8 * g + 4 + kr, ncol)));
          const uint4 W0 = *reinterpret_cast<const uint4*>(&sWs[gb][l16 & 3][32 * nk + 8 * g]);
          const uint4 W1 = *reinterpret_cast<const uint4*>(&sWs[gb][l16 & 3][32 * (nk + 2) + 8 * g]);
          f32x4 ni = mfma16x16x32(as_bf16x8(W0), B0, f32x4{0.f, 0.f, 0.f, 0.f});
          ni = mfma16x16x32(as_bf16x8(W1), B1, ni);
          if (g == 0) sNp[nk][32 * s + 8 * kr + 4 * nj + kq] = (ni[0] + ni[1]) + ni[2];
        }
        if (s == NS - 1) {
#pragma unroll
          for (int it = 0; it < NT; ++it)
            *reinterpret_cast<f32x4*>(&sR[W][it][lane][0]) = outT[it] * (sGate[gb][2][it * 16 + l16] * sig);
        }
        {
          const char* QbN = sRing[(x + 1) % NSLOT][0];
#pragma unroll
          for (int it = 0; it < NT / 2; ++it) QfN[it] = lds_ld16(QbN, swz4(it * 16 + l16, 8 * g));
        }
      }
      sig = sig_new;
      gb = (gb == 2) ? 0 : gb + 1;
    }
    // no load may still be in flight when the workgroup ends
    wait_vm<0>();
    __syncthreads();   // (the score waves' drain barrier)
    if (a.C1) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
          a.C1[(head * DQK + arow) * dv + b0w + l16] = cacc[t][e] * sig;
        }
      }
    }
  } else {
    for_wave<4>(cg, [&](auto Vc) {
      constexpr int V = decltype(Vc)::value;
      constexpr int QA = V, QB = NT - 1 - V;          // query tiles of this wave
      constexpr int KA = QA / 2 + 1, KB = QB / 2 + 1;  // their 32-key steps in P V
      f32x4 sa[QA + 1], sb[QB + 1];   // S^T tiles (key jt, query QA / QB)
      f32x4 qna, qnb;                 // q.n~ as three terms
      bf16x8 Pa[KA], Pb[KB];          // P of the chunk being finished (B operands)
      float rsa = 0.f, rsb = 0.f, qva = 0.f, qvb = 0.f;
      f32x4 oa[4], ob[4];             // numerators, value column tiles 0..3
      f32x4 ofa[4], ofb[4];           // o~ (float32)
      u32x2 oba[4], obb[4];           // o~ (bfloat16)
      bf16_t* const hbase = static_cast<bf16_t*>(a.h) + head * Ts * dv + vt * TV + 4 * g;

      // o~ (float32) of chunk c - 1 reaches the wave through LDS: a global ->
      // LDS copy at stage 1 of chunk c into this wave's 8 KB of the scaled
      // readout buffer, which is dead between its read at stage 0 and its
      // rewrite at stage 7.  Whole 256-byte rows per copy (direct 16-byte
      // loads in the h layout touched 16 half lines per instruction); row r
      // holds its 16-byte chunk j at slot j ^ (r % 16), so that the reads of
      // the h layout (16 rows, one chunk each) meet every bank once.
      char* const sOw = reinterpret_cast<char*>(&sR[0][0][0][0]) + V * 8192;
      auto issue_o = [&](int cp) {
        const float* ob_ = static_cast<const float*>(a.o_pre) + head * Ts * dv + vt * TV;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int r = 4 * m + (lane >> 4);            // rows 0..15: tile QA, 16..31: tile QB
          const int rr = r & 15;
          const int qt = (r < 16) ? QA : QB;
          const int lc = (lane & 15) ^ rr;              // the row's 16-byte chunk in this slot
          dma16_nt(ob_ + (static_cast<int64_t>(cp) * L + qt * 16 + rr) * dv + 4 * lc,
                   lds_addr(sOw + m * 1024));
        }
      };
      auto load_o = [&](int cp) {
        if constexpr (OM == O_F32) {
          const float* ob_ = static_cast<const float*>(a.o_pre) + head * Ts * dv + vt * TV + 4 * g;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            ofa[ct] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                ob_ + (static_cast<int64_t>(cp) * L + QA * 16 + l16) * dv + 16 * ct));
            ofb[ct] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                ob_ + (static_cast<int64_t>(cp) * L + QB * 16 + l16) * dv + 16 * ct));
          }
        } else if constexpr (OM == O_BF16) {
          const bf16_t* ob_ = static_cast<const bf16_t*>(a.o_pre) + head * Ts * dv + vt * TV + 4 * g;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            oba[ct] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
                ob_ + (static_cast<int64_t>(cp) * L + QA * 16 + l16) * dv + 16 * ct));
            obb[ct] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
                ob_ + (static_cast<int64_t>(cp) * L + QB * 16 + l16) * dv + 16 * ct));
          }
        }
      };
      // P V steps k0 .. k1 - 1 of both query tiles onto their numerators.  The
      // value fragment of step ks, column tile ct: lane (g, c) holds column
      // 16 ct + c for keys 32 ks + 4 g + 0..3 and 32 ks + 16 + 4 g + 0..3,
      // the key order of the P operands.
      auto pv_steps = [&](int k0, int k1, const char* Vb) {
#pragma unroll
        for (int ks = k0; ks < k1; ++ks) {
          bf16x8 Vf[4];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            Vf[ct] = join(lds_tr(Vb, swz(32 * ks + 4 * g + kr, 16 * ct + 4 * kq)),
                          lds_tr(Vb, swz(32 * ks + 16 + 4 * g + kr, 16 * ct + 4 * kq)));
          if (ks < KA) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) oa[ct] = mfma16x16x32(Vf[ct], Pa[ks < KA ? ks : 0], oa[ct]);
          }
          if (ks < KB) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ob[ct] = mfma16x16x32(Vf[ct], Pb[ks < KB ? ks : 0], ob[ct]);
          }
        }
      };
      // h of query tile qt of chunk cp from its numerators, row sum and q.n~
      auto h_tile = [&](int qt, const f32x4* o, const f32x4* of, const u32x2* obf, float rs, float qv,
                        int cp, int gbx, uint32_t* hk, int tb, bool o_lds) {
        const int i = qt * 16 + l16;
        const float gi_ = sGate[gbx][2][i];
        const float den = fmaxf(fabsf(gi_ * qv + rs), sGate[gbx][3][i]);
        bf16_t* dst = hbase + (static_cast<int64_t>(cp) * L + i) * dv;
        // h = o~-gate * num / den = num / (den (1 + exp(-o~))): one
        // reciprocal per element
        const float inv = __builtin_amdgcn_rcpf(den);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          float hv[4];
          if constexpr (OM == O_NONE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = o[ct][e] * inv;
          } else {
            float ov[4];
            if constexpr (OM == O_F32) {
              if (o_lds) {
                const f32x4 o4 = *reinterpret_cast<const f32x4*>(
                    sOw + (tb + l16) * 256 + 16 * ((4 * ct + g) ^ l16));
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = o4[e];
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = of[ct][e];
              }
            } else {
              ov[0] = bf_lo(obf[ct][0]); ov[1] = bf_hi(obf[ct][0]);
              ov[2] = bf_lo(obf[ct][1]); ov[3] = bf_hi(obf[ct][1]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hv[e] = o[ct][e] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, __expf(-ov[e]), den));
          }
          hk[2 * ct] = cvt2(hv[0], hv[1]);
          hk[2 * ct + 1] = cvt2(hv[2], hv[3]);
          st8_nt(dst + 16 * ct, hk[2 * ct], hk[2 * ct + 1]);
        }
      };
      // A store reads its data registers after it issues, so the compiler
      // waits for the store to complete before those registers are written
      // again.  Keeping the stored words live through the following stage
      // moves that wait one stage later, when the store has long completed.
      uint32_t hkA[8], hkB[8];
      auto keep = [](const uint32_t* hk) {
        asm volatile("" :: "v"(hk[0]), "v"(hk[1]), "v"(hk[2]), "v"(hk[3]), "v"(hk[4]), "v"(hk[5]),
                     "v"(hk[6]), "v"(hk[7]));
      };
      // P = S (.) D of query tile qt (accumulators acc[0..qt]) as B operands
      // of P V, its float32 row sum (before rounding) and q.n~
      auto form_p = [&](auto& acc, auto qtc, bf16x8* P, float& rs, float& qv, const f32x4& qn, int gbx) {
        constexpr int qt = decltype(qtc)::value;
        const int i = qt * 16 + l16;
        const float Mi = sGate[gbx][1][i];
        const float dM = sGate[gbx][1][L - 1] - Mi;
        float pe[qt + 2][4];
        float r = 0.0f;
        // D_ij = exp(u_j - M_i) = w_j exp(M_L - M_i), with w_j = exp(u_j - M_L)
        // from the gate scan: two multiplies per element instead of an
        // exponential.  While M_L - M_i <= 64 no factor overflows, and a w_j
        // that underflows belongs to a weight below e^-23 of the row's
        // largest (which is 1); a tile with a larger jump of the running
        // maximum inside the chunk takes the direct form (a wave-wide vote).
        if (__ballot(dM > 64.0f) == 0) {
          const float bi = __expf(dM);
#pragma unroll
          for (int jt = 0; jt <= qt; ++jt) {
            const float4 wj = *reinterpret_cast<const float4*>(&sGate[gbx][5][jt * 16 + 4 * g]);
            const float wjv[4] = {wj.x, wj.y, wj.z, wj.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = (acc[jt][e] * bi) * wjv[e];
              pe[jt][e] = (jt < qt || 4 * g + e <= l16) ? pv : 0.0f;
            }
            r += (pe[jt][0] + pe[jt][1]) + (pe[jt][2] + pe[jt][3]);
          }
        } else {
#pragma unroll
          for (int jt = 0; jt <= qt; ++jt) {
            const float4 uj = *reinterpret_cast<const float4*>(&sGate[gbx][0][jt * 16 + 4 * g]);
            const float ujv[4] = {uj.x, uj.y, uj.z, uj.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = acc[jt][e] * __expf(ujv[e] - Mi);
              pe[jt][e] = (jt < qt || 4 * g + e <= l16) ? pv : 0.0f;
            }
            r += (pe[jt][0] + pe[jt][1]) + (pe[jt][2] + pe[jt][3]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[qt + 1][e] = 0.0f;   // above the diagonal
#pragma unroll
        for (int ks = 0; ks <= qt / 2; ++ks) {
          const int j1 = (2 * ks + 1 <= qt) ? 2 * ks + 1 : qt + 1;
          P[ks] = __builtin_bit_cast(bf16x8, make_uint4(cvt2(pe[2 * ks][0], pe[2 * ks][1]),
                                                        cvt2(pe[2 * ks][2], pe[2 * ks][3]),
                                                        cvt2(pe[j1][0], pe[j1][1]),
                                                        cvt2(pe[j1][2], pe[j1][3])));
        }
        rs = sum_groups(r);
        qv = (qn[0] + qn[1]) + qn[2];
      };
      // n~ rows 128 hf .. 128 hf + 127 (slices 4 hf .. 4 hf + 3) after chunk
      // cf: g_L n~ + the two partial sums
      auto fold_n = [&](int cf, int hf, int gbf) {
        const int p = cf & 1;
        const float gLf = sGate[gbf][2][L - 1];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 128 * hf + 64 * r + lane;
          const float nv = gLf * sN[p][row] + (sNp[0][row] + sNp[1][row]);
          sN[p ^ 1][row] = nv;
          split3_bf16(nv, sNs[p ^ 1][0][row], sNs[p ^ 1][1][row], sNs[p ^ 1][2][row]);
        }
      };

      int gb = 0, gbp = 2;   // gate buffers of chunks c, c - 1
      float m_n2 = 0.0f, sg2 = 1.0f;
      GScan gsc;
      for (int c = 0; c < nchunks; ++c) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int x = c * NS + s;
          __syncthreads();
          const char* Qb = sRing[x % NSLOT][0];
          const char* Kb = sRing[x % NSLOT][1];
          if (s == 0) {
            // P of the previous chunk's second query tile (its scores stay
            // in sb until here)
            if (c > 0) form_p(sb, wave_c<QB>{}, Pb, rsb, qvb, qnb, gbp);
#pragma unroll
            for (int jt = 0; jt <= QA; ++jt) sa[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jt = 0; jt <= QB; ++jt) sb[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            qna = f32x4{0.f, 0.f, 0.f, 0.f};
            qnb = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          // the o~ loads (issued a chunk ago) complete here, on every path,
          // before the h stores: once stores are in flight, the compiler's
          // in-order wait for a late o~ load would also wait for those stores
          if (s == 5) wait_vm<0>();
          // scores and q.n~ of chunk c over the slice
          uint4 Kf[QB + 1];
#pragma unroll
          for (int jt = 0; jt <= QB; ++jt) Kf[jt] = lds_ld16(Kb, swz4(jt * 16 + l16, 8 * g));
          const uint4 QfA = lds_ld16(Qb, swz4(QA * 16 + l16, 8 * g));
          const uint4 QfB = lds_ld16(Qb, swz4(QB * 16 + l16, 8 * g));
          const uint4 Nx = *reinterpret_cast<const uint4*>(&sNs[c & 1][l16 & 3][32 * s + 8 * g]);
#pragma unroll
          for (int jt = 0; jt <= QA; ++jt) sa[jt] = mfma16x16x32(as_bf16x8(Kf[jt]), as_bf16x8(QfA), sa[jt]);
#pragma unroll
          for (int jt = 0; jt <= QB; ++jt) sb[jt] = mfma16x16x32(as_bf16x8(Kf[jt]), as_bf16x8(QfB), sb[jt]);
          qna = mfma16x16x32(as_bf16x8(Nx), as_bf16x8(QfA), qna);
          qnb = mfma16x16x32(as_bf16x8(Nx), as_bf16x8(QfB), qnb);
          // finishing of chunk c - 1, spread over the stages: P V one key
          // step per stage from stage 1 on (onto the scaled readout the state
          // waves left at its last stage; its value tile is overwritten from
          // stage 5 on), h at stages 5, 6
          if (c > 0) {
            const char* Vb = sV[(c - 1) & 1];
            if (s == 0) {
#pragma unroll
              for (int ct = 0; ct < 4; ++ct) {
                oa[ct] = *reinterpret_cast<const f32x4*>(&sR[ct][QA][lane][0]);
                ob[ct] = *reinterpret_cast<const f32x4*>(&sR[ct][QB][lane][0]);
              }
            }
            if (s >= 1 && s <= KB) pv_steps(s - 1, s, Vb);
            if constexpr (OM == O_F32) {
              if (s == 1) issue_o(c - 1);
            }
            if (s == 5) h_tile(QA, oa, ofa, oba, rsa, qva, c - 1, gbp, hkA, 0, true);
            if (s == 6) h_tile(QB, ob, ofb, obb, rsb, qvb, c - 1, gbp, hkB, 16, true);
          }
          if constexpr (OM == O_BF16) {
            if (s == O_STAGE) load_o(c);
          }
          // n~: the increments of slices 0..3 of chunk c are folded at stage 4
          // (wave 6), those of slices 4..7 of chunk c - 1 at stage 2 of
          // chunk c (wave 5), each before the next chunk's q.n~ reads the
          // rows and before the state waves rewrite their partial sums; a
          // fold is a chain of LDS round trips, so it sits at a stage where
          // its wave has no other work
          if (V == 2 && s == 4) fold_n(c, 0, gb);
          if (V == 1 && s == 2 && c > 0) fold_n(c - 1, 1, gbp);
          // gate scan of chunk c + 1
          if (V == SCAN_WAVE - 4) {
            if (s == 2) {
              scan_part(0, (c + 1) & 1, gb == 2 ? 0 : gb + 1, m_n1, sg1, gsc, m_n2, sg2);
              scan_part(1, (c + 1) & 1, gb == 2 ? 0 : gb + 1, m_n1, sg1, gsc, m_n2, sg2);
            }
            if (s == 3) scan_part(2, (c + 1) & 1, gb == 2 ? 0 : gb + 1, m_n1, sg1, gsc, m_n2, sg2);
            if (s == 4) scan_part(3, (c + 1) & 1, gb == 2 ? 0 : gb + 1, m_n1, sg1, gsc, m_n2, sg2);
          }
          if (s == NS - 1) form_p(sa, wave_c<QA>{}, Pa, rsa, qva, qna, gb);
          if (c > 0 && s == 6) keep(hkA);
          if (c > 0 && s == 7) keep(hkB);
        }
        m_s = m_n1;
        m_n1 = m_n2;
        sg1 = sg2;
        gbp = gb;
        gb = (gb == 2) ? 0 : gb + 1;
      }
      // ---- drain: the last chunk
      __syncthreads();
      form_p(sb, wave_c<QB>{}, Pb, rsb, qvb, qnb, gbp);
      {
        const char* Vb = sV[(nchunks - 1) & 1];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          oa[ct] = *reinterpret_cast<const f32x4*>(&sR[ct][QA][lane][0]);
          ob[ct] = *reinterpret_cast<const f32x4*>(&sR[ct][QB][lane][0]);
        }
        // (the last chunk's o~ straight into registers: the buffer above
        // holds its scaled readout until this point)
        if constexpr (OM == O_F32) load_o(nchunks - 1);
        pv_steps(0, KB, Vb);
        h_tile(QA, oa, ofa, oba, rsa, qva, nchunks - 1, gbp, hkA, 0, false);
        h_tile(QB, ob, ofb, obb, rsb, qvb, nchunks - 1, gbp, hkB, 16, false);
      }
      if (V == 1) {
        fold_n(nchunks - 1, 1, gbp);
        if (a.C1 && vt == 0) {
          const int p = nchunks & 1;
#pragma unroll
          for (int r = 0; r < DQK / 64; ++r) a.n1[head * DQK + 64 * r + lane] = sN[p][64 * r + lane];
        }
      }
      if (V == SCAN_WAVE - 4 && a.C1 && vt == 0 && lane == 0) a.m1[head] = m_s;
    });
  }
}

}  // namespace

bool chunk_ws128_supported(const SeqArgs& a, int64_t chunk) {
  return a.qkv_bf16 && a.dqk == DQK && a.dv % TV == 0 && chunk == L && a.T % L == 0 && a.T >= L;
}

hipError_t launch_chunk_ws128(const SeqArgs& a, hipStream_t stream) {
  const unsigned nwg = static_cast<unsigned>(a.B * a.H * (a.dv / TV));
  switch (a.o_mode) {
    case O_F32: chunk_ws128_kernel<O_F32><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    case O_BF16: chunk_ws128_kernel<O_BF16><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    default: chunk_ws128_kernel<O_NONE><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace mlstm
