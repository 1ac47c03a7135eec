// Fused chunkwise mLSTM forward on bf16 MFMA (gfx950), one launch.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form" (decay
// matrix S, H = ((Q K^T) (.) S) V) applied inside chunks of L tokens, with the
// state of "Associative Matrix Cell State" carried from chunk to chunk, and the
// running maximum of section 2 "The Normalizer State and Numerical
// Stabilization".  For a chunk after token s with carried (C~_s, n~_s, m_s)
// and chunk-local cumulative log forget gates b_i:
//   u_j = i~_j - b_j,  M_i = max(m_s, max_{j<=i} u_j),  m_i = b_i + M_i
//   D_ij = exp(u_j - M_i) (j <= i),  g_i = exp(m_s - M_i),  w_j = exp(u_j - M_L)
//   num_i = g_i q_i^T C~_s + sum_j D_ij (q_i . k_j) v_j
//   den_i = max(|g_i q_i . n~_s + sum_j D_ij (q_i . k_j)|, exp(-m_i))
//   h_i = sigmoid(o~_i) (.) num_i / den_i
//   C~ <- g_L C~_s + K^T diag(w) V,  n~ <- g_L n~_s + K^T w,  m <- m_L.
// m depends on the gates only, so every weight is <= 1 and no online
// rescaling is needed (unlike softmax attention).
//
// Design (MI355X, CDNA4):
// * One workgroup (4 waves) per (head, 64 value columns).  It walks the chunks
//   in order and keeps its [d_qk x 64] slice of C~ in float32 registers (each
//   wave: 16 columns x all d_qk rows) for the whole sequence; the state never
//   round-trips through HBM between chunks.  The workgroups of one head sit on
//   one XCD (block id = head mod 8), so their shared q/k reads hit one L2.
// * Four contractions per chunk on v_mfma_f32_16x16x32_bf16 (fp32 accumulate):
//   S^T = K Q^T (causal 16x16 tiles), the readout C~^T Q^T, P V, and the state
//   update K^T (w V).  The state update's output rows are permuted so that a
//   lane holds 8 consecutive d_qk rows of C~: the readout then takes C~ from
//   its accumulator registers with no data movement.
// * Every load inside the chunk loop goes global -> LDS directly
//   (global_load_lds_dwordx4 / _dword): q/k in 64-wide d_qk slices ("stages")
//   into a ring of D+1 slots with D stages in flight, the value tile and the
//   o~ tile once per chunk, and the gate preactivations.  The loads are issued
//   from inline asm, so the compiler sees no vector-memory load in the loop and
//   inserts no waits of its own; each wait is an explicit s_waitcnt vmcnt(n)
//   whose n (the loads this wave issued after the awaited one) is a
//   compile-time constant, because every load is issued unconditionally
//   (clamped to valid addresses past the end of the sequence).
// * All tiles stay row-major in LDS (128-byte rows, 16-byte chunks XOR-swizzled
//   by row).  Operands that contract over tokens (K^T for the state update,
//   V^T for P V and the update) are read with ds_read_b64_tr_b16, the gfx950
//   LDS transpose read, instead of keeping transposed copies.
// * The denominator uses the float32 decay-weighted row sums (before P is
//   rounded to bf16) and the float32 n~.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int NW = 4;       // waves per workgroup
constexpr int NTH = 256;    // threads per workgroup
constexpr int TV = 64;      // value columns per workgroup (16 per wave)
constexpr int AS = 64;      // d_qk slice width (one stage)

template <int DQK, int L, int OM>
struct CK {
  static constexpr int NT = L / 16;                // 16-token tiles per chunk
  static constexpr int NKS = L / 32;               // 32-token MFMA k-steps
  static constexpr int NS = DQK / AS;              // stages (d_qk slices) per chunk
  static constexpr int NCT = DQK / 16;             // 16-row C~ tiles
  static constexpr int TILE = L * 128;             // bytes of one [L x 64] bf16 tile
  static constexpr int DPREF = (L == 128) ? 1 : 4;
  // look-ahead: at most one chunk, so that nothing issued for a later chunk is
  // awaited before it is needed
  static constexpr int D = DPREF < NS ? DPREF : NS;
  static constexpr int NSLOT = D + 1;
  static constexpr int VSLOT = (D <= NS - 1) ? 1 : 2;   // value tile slots
  static constexpr int OROW = (OM == O_BF16) ? 128 : 256;   // bytes per o~ tile row
  static constexpr int OTILE = (OM == O_NONE) ? 16 : L * OROW;
  static constexpr int PROW = L + 8;               // padded row of P (bf16)
  static constexpr int NTILES = NT * (NT + 1) / 2; // causal 16x16 score tiles
  static constexpr int TPW = (NTILES + NW - 1) / NW;
  static constexpr int NQN = (NT + NW - 1) / NW;
  static constexpr int NB_QK = L / 16;             // 1 KB loads per wave per stage (q + k)
  static constexpr int NB_V = L / 32;              // 1 KB loads per wave per value tile
  static constexpr int NB_O = (OM == O_NONE) ? 0 : L * OROW / 1024 / NW;   // per o~ tile
  static constexpr int GH = (L > 64) ? 2 : 1;      // 64-token halves of the gates
  static constexpr int NB_G = 2 * GH;              // 256 B gate loads per wave per chunk
  static constexpr int NB_X = NB_O + NB_G;         // per-chunk loads after the opening stage
  static_assert(DQK % AS == 0 && NS <= NW, "d_qk must be 64, 128, 192 or 256");
  static_assert(L % 32 == 0 && L <= 128, "chunk must be 32, 64 or 128");
};

template <int DQK, int L, int OM>
__global__ __launch_bounds__(NTH, 1) void chunk_mfma_kernel(SeqArgs a) {
  using C = CK<DQK, L, OM>;
  __shared__ __align__(1024) char sRing[C::NSLOT][2][C::TILE];  // [slot][q|k]
  __shared__ __align__(1024) char sV[C::VSLOT][C::TILE];
  __shared__ __align__(1024) char sO[C::OTILE];                 // o~ tile of the chunk
  // raw gates [chunk parity][i~ | f~]; every wave loads the same values here
  // (identical writes) so that all waves issue the same number of loads
  __shared__ __align__(256) float sGin[2][2][64 * C::GH];
  __shared__ __align__(16) bf16_t sP[L * C::PROW];
  __shared__ __align__(16) float sGate[2][5][L];  // u, M, g, w, exp(-m) by chunk parity
  __shared__ float sRs[NW][L];
  __shared__ float sQn[L];
  __shared__ __align__(16) float sN[DQK];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // ---- workgroup -> (head, value tile)
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
  const int64_t T = a.T, Ts = a.Ts;   // tokens per head; token stride between heads
  const int nchunks = static_cast<int>(T / L);
  const int b0w = vt * TV + wave * 16;

  const bf16_t* gq = static_cast<const bf16_t*>(a.q) + head * Ts * DQK;
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * Ts * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * Ts * dv + vt * TV;
  const float* gi = a.i_pre + head * Ts;
  const float* gf = a.f_pre + head * Ts;
  bf16_t* gh = static_cast<bf16_t*>(a.h) + head * Ts * dv;

  // ---- state
  f32x4 cacc[C::NCT];
#pragma unroll
  for (int t = 0; t < C::NCT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
      cacc[t][e] = a.C0 ? a.C0[(head * DQK + arow) * dv + b0w + l16] : 0.0f;
    }
  }
  if (tid < DQK) sN[tid] = a.C0 ? a.n0[head * DQK + tid] : 0.0f;
  float m_s = a.C0 ? a.m0[head] : 0.0f;

  // ---- stage loads (global -> LDS).  Lane l of a 1 KB load writes bytes
  // 16l..16l+15 of its destination: row 8G + l/8 of the tile, physical chunk
  // l%8, which holds logical chunk (l%8) ^ ((row/2)%8).
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  // per-lane element offsets of this wave's stage loads inside one chunk/slice
  int qk_off[C::NB_QK], v_off[C::NB_V];
#pragma unroll
  for (int m = 0; m < C::NB_QK; ++m) {
    const int Gr = (wave * C::NB_QK + m) % (L / 8);
    const int row = 8 * Gr + ld_r;
    qk_off[m] = row * DQK + 8 * (ld_pc ^ ((row >> 1) & 7));
  }
#pragma unroll
  for (int m = 0; m < C::NB_V; ++m) {
    const int row = 8 * (wave * C::NB_V + m) + ld_r;
    v_off[m] = row * dv + 8 * (ld_pc ^ ((row >> 1) & 7));
  }
  auto issue_stage = [&](int x) {
    const int cx = x / C::NS, sx = x % C::NS;
    const int cc = cx < nchunks ? cx : nchunks - 1;    // past the end: harmless re-read
    char* slot = sRing[x % C::NSLOT][0];
    const int64_t base = static_cast<int64_t>(cc) * L * DQK + sx * AS;
#pragma unroll
    for (int m = 0; m < C::NB_QK; ++m) {
      const int G = wave * C::NB_QK + m;               // 0 .. L/4-1
      const int mat = G / (L / 8);                      // 0 = q, 1 = k
      const int Gr = G % (L / 8);
      dma16((mat ? gk : gq) + base + qk_off[m], lds_addr(slot + mat * C::TILE + Gr * 1024));
    }
    if (sx == 0) {
      const int64_t vbase = static_cast<int64_t>(cc) * L * dv;
#pragma unroll
      for (int m = 0; m < C::NB_V; ++m)
        dma16(gv + vbase + v_off[m], lds_addr(sV[cx % C::VSLOT] + (wave * C::NB_V + m) * 1024));
    }
  };
  // Per-chunk loads: the o~ tile of chunk c (rows of 64 values; 16-byte
  // chunks swizzled by row) and this wave's copy of the gates of chunk c + 2
  // (two chunks ahead, so that waiting for them never waits for a stage).
  auto issue_chunk_extras = [&](int c) {
    if (OM != O_NONE) {
      constexpr int RPI = 1024 / C::OROW;               // o~ rows per 1 KB load
      constexpr int NCH = C::OROW / 16;                 // 16-byte chunks per row
#pragma unroll
      for (int m = 0; m < C::NB_O; ++m) {
        const int G = wave * C::NB_O + m;
        const int row = RPI * G + lane / NCH;
        const int pc = lane % NCH;
        const int lc = (OM == O_F32) ? (pc ^ (row & 15)) : (pc ^ ((row >> 1) & 7));
        const int64_t r = head * Ts + static_cast<int64_t>(c) * L + row;
        const char* src = (OM == O_F32)
            ? reinterpret_cast<const char*>(static_cast<const float*>(a.o_pre) + r * dv + vt * TV + 4 * lc)
            : reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.o_pre) + r * dv + vt * TV + 8 * lc);
        dma16(src, lds_addr(sO + G * 1024));
      }
    }
    const int cn = (c + 2 < nchunks) ? c + 2 : nchunks - 1;
#pragma unroll
    for (int h2 = 0; h2 < C::GH; ++h2) {
      const int64_t j = static_cast<int64_t>(cn) * L + (lane + 64 * h2) % L;
      dma4(gi + j, lds_addr(&sGin[c & 1][0][64 * h2]));
      dma4(gf + j, lds_addr(&sGin[c & 1][1][64 * h2]));
    }
  };

  // Gate scan of one chunk (its gates in the staging buffer of parity `par`)
  // given the carried m; run by wave 0, which publishes the per-token
  // values.  Returns the m after the chunk's last token.
  auto scan_gates = [&](int par, float ms) {
    float pgi[2], pgf[2], lf[2], bcum[2], u[2], Mx[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      pgi[h2] = (h2 < C::GH) ? sGin[par][0][lane + 64 * h2] : 0.0f;
      pgf[h2] = (h2 < C::GH) ? sGin[par][1][lane + 64 * h2] : 0.0f;
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int j = lane + 64 * h2;
      lf[h2] = (j < L && (h2 == 0 || L > 64)) ? log_forget(pgf[h2], a.fgate_exp) : 0.0f;
    }
    bcum[0] = wave_incl_sum(lf[0], lane);
    u[0] = (lane < L) ? pgi[0] - bcum[0] : -INFINITY;
    Mx[0] = fmaxf(ms, wave_incl_max(u[0], lane));
    if (L > 64) {
      bcum[1] = wave_incl_sum(lf[1], lane) + __shfl(bcum[0], 63, 64);
      u[1] = pgi[1] - bcum[1];
      Mx[1] = fmaxf(__shfl(Mx[0], 63, 64), wave_incl_max(u[1], lane));
    } else {
      bcum[1] = u[1] = Mx[1] = 0.0f;
    }
    const float Mlast = __shfl(L > 64 ? Mx[1] : Mx[0], (L - 1) & 63, 64);
    const float blast = __shfl(L > 64 ? bcum[1] : bcum[0], (L - 1) & 63, 64);
    {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = lane + 64 * h2;
        if (j < L) {
          sGate[par][0][j] = u[h2];
          sGate[par][1][j] = Mx[h2];
          sGate[par][2][j] = __expf(ms - Mx[h2]);
          sGate[par][3][j] = __expf(u[h2] - Mlast);
          sGate[par][4][j] = __expf(-(bcum[h2] + Mx[h2]));
        }
      }
    }
    return blast + Mlast;
  };

  // ---- prologue: stages 0 .. D-1 in flight, gates of chunk 0 scanned
#pragma unroll
  for (int x = 0; x < C::D; ++x) issue_stage(x);
#pragma unroll
  for (int h2 = 0; h2 < C::GH; ++h2) {
    const int j0 = (lane + 64 * h2) % L;
    const int j1 = (nchunks > 1 ? L : 0) + j0;
    dma4(gi + j0, lds_addr(&sGin[0][0][64 * h2]));
    dma4(gf + j0, lds_addr(&sGin[0][1][64 * h2]));
    dma4(gi + j1, lds_addr(&sGin[1][0][64 * h2]));
    dma4(gf + j1, lds_addr(&sGin[1][1][64 * h2]));
  }
  wait_vm<0>();
  float m_next = 0.0f;                 // m after the current chunk (wave 0)
  if (wave == 0) m_next = scan_gates(0, m_s);
  __syncthreads();   // chunk 0's gate values are read by every wave below
  // C~ = sig * cacc: the decay g_L of each chunk is folded into sig (a scalar)
  // instead of rescaling every accumulator; see the state update below.
  float sig = 1.0f;

  f32x4 outT[C::NT];
  f32x4 sacc[C::TPW];
  bf16x8 Vf[C::NKS];
  bf16x8 wVf[C::NKS];
  float nn[C::NS];
  float qnp[C::NQN];

  for (int c = 0; c < nchunks; ++c) {
    const int par = c & 1;
    const float gL = sGate[par][2][L - 1];
    // Lazy scaling: C~_new = g_L C~ + K^T(wV) = sig' (cacc + K^T((w / sig') V))
    // with sig' = g_L sig.  When sig' gets tiny the chunk instead applies
    // g_L sig to the accumulators (after their readout) and resets sig' = 1.
    const bool renorm = gL * sig < 0x1p-64f;
    const float sig_new = renorm ? 1.0f : gL * sig;
    const float wscale = 1.0f / sig_new;

#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const int x = c * C::NS + s;
      // ---- wait for this stage's LDS loads, then make them visible
      if (x < C::D) wait_vm<0>();
      else wait_stage<C::NS, C::D, C::NB_QK, C::NB_V, C::NB_X>(s);
      __syncthreads();
      issue_stage(x + C::D);
      if (s == 0) issue_chunk_extras(c);
      const char* Qb = sRing[x % C::NSLOT][0];
      const char* Kb = sRing[x % C::NSLOT][1];

      if (s == 0) {
        // V^T fragments of this wave's 16 columns: lane (g, c) gets the
        // values of column c for tokens 32ks + 8g + 0..7
        const char* Vb = sV[c % C::VSLOT];
        const int vr = l16 >> 2, vq = l16 & 3;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          const int col = wave * 16 + 4 * vq;
          const uint2 lo = lds_tr(Vb, swz(32 * ks + 8 * g + vr, col));
          const uint2 hi = lds_tr(Vb, swz(32 * ks + 8 * g + 4 + vr, col));
          Vf[ks] = join(lo, hi);
          const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g + 4]);
          float xw[8];
          xw[0] = bf_lo(lo.x) * (w0.x * wscale); xw[1] = bf_hi(lo.x) * (w0.y * wscale);
          xw[2] = bf_lo(lo.y) * (w0.z * wscale); xw[3] = bf_hi(lo.y) * (w0.w * wscale);
          xw[4] = bf_lo(hi.x) * (w1.x * wscale); xw[5] = bf_hi(hi.x) * (w1.y * wscale);
          xw[6] = bf_lo(hi.y) * (w1.z * wscale); xw[7] = bf_hi(hi.y) * (w1.w * wscale);
          wVf[ks] = cvt8(xw);
        }
#pragma unroll
        for (int it = 0; it < C::NT; ++it) outT[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < C::TPW; ++k) sacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < C::NQN; ++k) qnp[k] = 0.0f;
      }

      // ---- readout, n~ . q and score tiles for the slice's two 32-row k-steps
#pragma unroll
      for (int p = 0; p < AS / 32; ++p) {
        const int P = s * (AS / 32) + p;   // C~ tile pair
        float ca[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ca[e] = cacc[2 * P][e];
          ca[4 + e] = cacc[2 * P + 1][e];
        }
        // C~ as a (high, remainder) pair of bf16 operands (see cvt8_split)
        bf16x8 A_hi, A_lo;
        cvt8_split(ca, A_hi, A_lo);
        uint4 Qf[C::NT];
#pragma unroll
        for (int it = 0; it < C::NT; ++it) {
          Qf[it] = lds_ld16(Qb, swz(it * 16 + l16, 32 * p + 8 * g));
          outT[it] = mfma16x16x32(A_hi, as_bf16x8(Qf[it]), outT[it]);
          outT[it] = mfma16x16x32(A_lo, as_bf16x8(Qf[it]), outT[it]);
        }
        for_wave<NW>(wave, [&](auto Wc) {
          constexpr int W = decltype(Wc)::value;
          // n~ . q for the query tiles of this wave, and its causal score tiles
          const float4 n0v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g]);
          const float4 n1v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g + 4]);
#pragma unroll
          for (int it = 0; it < C::NT; ++it) {
            if (it % NW == W) {
              qnp[it / NW] += bf_lo(Qf[it].x) * n0v.x + bf_hi(Qf[it].x) * n0v.y +
                              bf_lo(Qf[it].y) * n0v.z + bf_hi(Qf[it].y) * n0v.w +
                              bf_lo(Qf[it].z) * n1v.x + bf_hi(Qf[it].z) * n1v.y +
                              bf_lo(Qf[it].w) * n1v.z + bf_hi(Qf[it].w) * n1v.w;
            }
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
              const int n = it * (it + 1) / 2 + jt;
              if (n % NW == W) {
                const uint4 Kf = lds_ld16(Kb, swz(jt * 16 + l16, 32 * p + 8 * g));
                sacc[n / NW] = mfma16x16x32(as_bf16x8(Kf), as_bf16x8(Qf[it]), sacc[n / NW]);
              }
            }
          }
        });
      }

      // ---- state update of the slice's rows (after their readout above).
      // A fragment of C~ tile t: lane (g, c) holds k_j[a] for tokens
      // 32ks+8g+0..7 and d_qk row a = 32(t/2) + 8(c/4) + 4(t%2) + c%4.
      float npart = 0.0f;
      if (renorm) {
        const float f = gL * sig;
#pragma unroll
        for (int tl = 0; tl < AS / 16; ++tl) cacc[s * (AS / 16) + tl] *= f;
      }
      const int kr = l16 >> 2, kq = l16 & 3;
      for_wave<NW>(wave, [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
          for (int tl = 0; tl < AS / 16; ++tl) {
            const int col = 32 * (tl >> 1) + 8 * kq + 4 * (tl & 1);
            const uint2 lo = lds_tr(Kb, swz(32 * ks + 8 * g + kr, col));
            const uint2 hi = lds_tr(Kb, swz(32 * ks + 8 * g + 4 + kr, col));
            const int t = s * (AS / 16) + tl;
            cacc[t] = mfma16x16x32(join(lo, hi), wVf[ks], cacc[t]);
            if (tl == W) {
              // n~ rows of tile W: sum_j w_j k_j[a] over this lane's 8 tokens
              const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g]);
              const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g + 4]);
              npart += bf_lo(lo.x) * w0.x + bf_hi(lo.x) * w0.y + bf_lo(lo.y) * w0.z + bf_hi(lo.y) * w0.w +
                       bf_lo(hi.x) * w1.x + bf_hi(hi.x) * w1.y + bf_lo(hi.y) * w1.z + bf_hi(hi.y) * w1.w;
            }
          }
        }
      });
      npart += __shfl_xor(npart, 16, 64);
      npart += __shfl_xor(npart, 32, 64);
      nn[s] = npart;
    }

    // ================= end of chunk: this chunk's o~ and the next chunk's
    // gates have landed (each wave waits for its own loads; the barrier below
    // publishes the o~ tile), then the epilogue
    wait_vm<C::NB_G + loads_after_chunk_extras<C::NS, C::D, C::NB_QK, C::NB_V>()>();
    const float m_cur = m_next;
    if (wave == 0) m_next = scan_gates(par ^ 1, m_cur);

    float rsp[C::NT];
#pragma unroll
    for (int it = 0; it < C::NT; ++it) rsp[it] = 0.0f;
    for_wave<NW>(wave, [&](auto Wc) {
     constexpr int W = decltype(Wc)::value;
#pragma unroll
     for (int it = 0; it < C::NT; ++it) {
#pragma unroll
      for (int jt = 0; jt <= it; ++jt) {
        const int n = it * (it + 1) / 2 + jt;
        if (n % NW == W) {
          const int i = it * 16 + l16;
          const float Mi = sGate[par][1][i];
          const float4 uj = *reinterpret_cast<const float4*>(&sGate[par][0][jt * 16 + 4 * g]);
          const float ujv[4] = {uj.x, uj.y, uj.z, uj.w};
          float pe[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = jt * 16 + 4 * g + e;
            const float pv = sacc[n / NW][e] * __expf(ujv[e] - Mi);
            pe[e] = (jt < it || j <= i) ? pv : 0.0f;
          }
          rsp[it] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
          *reinterpret_cast<uint2*>(sP + i * C::PROW + jt * 16 + 4 * g) =
              make_uint2(cvt2(pe[0], pe[1]), cvt2(pe[2], pe[3]));
          // P V runs in 32-token k-steps: the tile right of an even diagonal
          // tile lies in the same step and must read as zero (j > i)
          if (jt == it && (it & 1) == 0)
            *reinterpret_cast<uint2*>(sP + i * C::PROW + (jt + 1) * 16 + 4 * g) = make_uint2(0u, 0u);
        }
      }
     }
#pragma unroll
     for (int it = 0; it < C::NT; ++it) {
       float r = rsp[it];
       r += __shfl_xor(r, 16, 64);
       r += __shfl_xor(r, 32, 64);
       if (g == 0) sRs[W][it * 16 + l16] = r;
       if (it % NW == W) {
         float qv = qnp[it / NW];
         qv += __shfl_xor(qv, 16, 64);
         qv += __shfl_xor(qv, 32, 64);
         if (g == 0) sQn[it * 16 + l16] = qv;
       }
     }
    });
    __syncthreads();
    // n~ for the next chunk: wave w owns the rows of tile w of every slice
    if (g == 0) {
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int arow = s * AS + 32 * (wave >> 1) + 8 * (l16 >> 2) + 4 * (wave & 1) + (l16 & 3);
        sN[arow] = gL * sN[arow] + nn[s];
      }
    }

#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
      const int i = it * 16 + l16;
      const float gi_ = sGate[par][2][i];
      f32x4 o = outT[it] * (gi_ * sig);   // the readout saw C~_s / sig
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        if (32 * ks <= it * 16 + 15) {
          const uint4 Pf = *reinterpret_cast<const uint4*>(sP + i * C::PROW + 32 * ks + 8 * g);
          o = mfma16x16x32(Vf[ks], as_bf16x8(Pf), o);
        }
      }
      const float rs = (sRs[0][i] + sRs[1][i]) + (sRs[2][i] + sRs[3][i]);
      const float den = fmaxf(fabsf(gi_ * sQn[i] + rs), sGate[par][4][i]);
      const float inv = __builtin_amdgcn_rcpf(den);
      float hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = o[e] * inv;
      if (OM != O_NONE) {
        float ov[4];
        if (OM == O_F32) {
          const float4 o4 = *reinterpret_cast<const float4*>(
              sO + i * 256 + 16 * ((wave * 4 + g) ^ (i & 15)));
          ov[0] = o4.x; ov[1] = o4.y; ov[2] = o4.z; ov[3] = o4.w;
        } else {
          const uint2 o2 = *reinterpret_cast<const uint2*>(sO + swz(i, wave * 16 + 4 * g));
          ov[0] = bf_lo(o2.x); ov[1] = bf_hi(o2.x); ov[2] = bf_lo(o2.y); ov[3] = bf_hi(o2.y);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] *= __builtin_amdgcn_rcpf(1.0f + __expf(-ov[e]));
      }
      *reinterpret_cast<uint2*>(gh + (static_cast<int64_t>(c) * L + i) * dv + b0w + 4 * g) =
          make_uint2(cvt2(hv[0], hv[1]), cvt2(hv[2], hv[3]));
    }
    m_s = m_cur;
    sig = sig_new;
  }
  // no LDS load may still be in flight when the workgroup ends
  wait_vm<0>();
  __syncthreads();

  // ---- final state
  if (a.C1) {
#pragma unroll
    for (int t = 0; t < C::NCT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
        a.C1[(head * DQK + arow) * dv + b0w + l16] = cacc[t][e] * sig;
      }
    }
    if (vt == 0) {
      if (tid < DQK) a.n1[head * DQK + tid] = sN[tid];
      if (tid == 0) a.m1[head] = m_s;
    }
  }
}

template <int DQK, int L, int OM>
hipError_t launch_shape(const SeqArgs& a, hipStream_t stream) {
  const unsigned nwg = static_cast<unsigned>(a.B * a.H * (a.dv / TV));
  chunk_mfma_kernel<DQK, L, OM><<<dim3(nwg), dim3(NTH), 0, stream>>>(a);
  return hipGetLastError();
}

template <int DQK, int OM>
hipError_t launch_L(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  switch (chunk) {
    case 32: return launch_shape<DQK, 32, OM>(a, stream);
    case 64: return launch_shape<DQK, 64, OM>(a, stream);
    default:
      if constexpr (DQK >= 128) return launch_shape<DQK, 128, OM>(a, stream);
      return hipErrorInvalidValue;
  }
}

template <int OM>
hipError_t launch_D(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  switch (a.dqk) {
    case 64: return launch_L<64, OM>(a, chunk, stream);
    case 128: return launch_L<128, OM>(a, chunk, stream);
    default: return launch_L<256, OM>(a, chunk, stream);
  }
}

}  // namespace

bool chunk_mfma_supported(const SeqArgs& a, int64_t chunk) {
  // chunk 128 with d_qk 64 would need more LDS than a CU has (one look-ahead
  // stage cannot share its value slot); it takes the VALU kernel instead
  return a.qkv_bf16 && (a.dqk == 64 || a.dqk == 128 || a.dqk == 256) && a.dv % TV == 0 &&
         (chunk == 32 || chunk == 64 || (chunk == 128 && a.dqk >= 128)) && a.T % chunk == 0;
}

size_t chunk_mfma_workspace(const SeqArgs&, int64_t) { return 0; }

hipError_t launch_chunk_mfma(const SeqArgs& a, int64_t chunk, void*, hipStream_t stream) {
  if (chunk_ws_supported(a, chunk)) return launch_chunk_ws(a, stream);
  if (chunk_ws128_supported(a, chunk)) return launch_chunk_ws128(a, stream);
  if (chunk_mfma8_supported(a, chunk)) return launch_chunk_mfma8(a, stream);
  switch (a.o_mode) {
    case O_F32: return launch_D<O_F32>(a, chunk, stream);
    case O_BF16: return launch_D<O_BF16>(a, chunk, stream);
    default: return launch_D<O_NONE>(a, chunk, stream);
  }
}

}  // namespace mlstm
