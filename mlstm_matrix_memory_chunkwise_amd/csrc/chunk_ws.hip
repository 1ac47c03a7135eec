// Fused chunkwise mLSTM forward, bf16 MFMA, chunk 64, d_qk 256: a state group
// and an intra-chunk group of waves, software-pipelined by one chunk.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form" inside
// chunks of 64 tokens, the state of "Associative Matrix Cell State" carried
// between chunks, the running maximum of section 2 "The Normalizer State and
// Numerical Stabilization".  The chunk algebra is the one of chunk_mfma.hip:
//   u_j = i~_j - b_j,  M_i = max(m_s, max_{j<=i} u_j),  m_i = b_i + M_i
//   D_ij = exp(u_j - M_i),  g_i = exp(m_s - M_i),  w_j = exp(u_j - M_L)
//   h_i = sigmoid(o~_i) (.) (g_i q_i^T C~_s + sum_j D_ij (q_i.k_j) v_j)
//         / max(|g_i q_i.n~_s + sum_j D_ij (q_i.k_j)|, exp(-m_i))
//   C~ <- g_L C~ + K^T diag(w) V,  n~ <- g_L n~ + K^T w.
//
// Of the chunk's work only the state update feeds the next chunk; the score
// tiles, P, P V and the output do not.  The workgroup (8 waves, one (head, 64
// value columns) pair) therefore splits by role, one wave of each role per
// SIMD:
// * state waves 0..3 (16 value columns each) keep C~ in registers and, per
//   64-row d_qk slice ("stage"), run the readout C~^T Q^T, the update
//   K^T (w V) and their share of the causal transposed score tiles
//   S^T = K Q^T on MFMA (wave W: key tile W against query tiles W..3, with
//   (key 0, query 3) moved from wave 0 to wave 3, so 3, 3, 2, 2 tiles; the
//   wave index is a compile-time constant in each wave's copy of the loop);
//   at the end of a chunk they leave the scaled readout g_i sig C~^T q_i and
//   P = S (.) D in LDS (query tiles 2, 3 in one of two buffers by chunk
//   parity, since the intra waves still read the previous chunk's);
// * intra waves 4..7 compute q.n~ and the n~ increment K^T w (MFMAs with
//   the vector split into three bf16 terms), issue and await every
//   global->LDS load, and, during the stages of chunk c, finish chunk c-1:
//   P V of query tiles 0, 1 at stage 1, their h and P V of tiles 2, 3 at
//   stage 2, the denominators of tiles 2, 3 at stage 3 and their h at stage
//   0 of chunk c+1.
// The VALU-heavy finishing of one chunk thus overlaps the MFMA-heavy state
// work of the next on every SIMD, and no wave waits for a chunk epilogue.
// h leaves through a small LDS staging tile: each intra wave computes 16 of
// the 64 columns, and written directly every 128-byte row of h would reach
// memory as four 32-byte pieces from four waves (measured: a third more
// write traffic than h itself).  Staged, a row is written by one wave as
// eight 16-byte lane stores, one stage after it was computed.
//
// Inside a stage the state waves work in two halves of 32 d_qk rows: the
// Q/K fragments of a half are read one half ahead (those of a stage's first
// half during the previous stage, whose barrier already published the
// slot), and the high/remainder bf16 pair of the next half's C~ rows is
// formed between the current half's MFMAs.  On a SIMD, vector-ALU and MFMA
// work do not overlap (measured), so the chunk costs the sum of both roles'
// instructions: the score tiles above the diagonal are not computed, and
// the gate scan runs on the wave with the fewest tiles.
//
// Loads are global->LDS DMAs issued from asm, with compile-time vmcnt
// waits; q/k come in 64-wide d_qk slices through a ring of D+1 slots, v once
// per chunk, the o~ tile once per chunk into one of two slots, the gates two
// chunks ahead.  At the top of stage x the loading waves wait for the loads
// of stage x + 1 (the state waves' read-ahead), issued D - 1 stages earlier.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int NW = 8;
constexpr int NTH = 512;
constexpr int TV = 64;         // value columns per workgroup
constexpr int AS = 64;         // d_qk slice (stage) width
constexpr int L = 64;          // chunk
constexpr int NT = L / 16;     // 16-token tiles
constexpr int NKS = L / 32;    // 32-token k-steps
constexpr int TILE = L * 128;  // one [64 x 64] bf16 tile
constexpr int PROW = L + 8;
constexpr int DQK = 256;
constexpr int NS = DQK / AS;   // stages per chunk
constexpr int NCT = DQK / 16;  // 16-row C~ tiles per state wave
constexpr int D = 3;           // stages in flight
constexpr int NSLOT = D + 1;
// One role (NWL waves) issues and awaits all global->LDS loads (issuing
// stalls while the address units are busy); the barrier after each wait
// publishes the landed data to the other role.  The intra waves take them:
// the state waves have the longer stages and the higher register count.
constexpr bool STATE_LOADS = false;
constexpr int NWL = 4;
constexpr int NB_QK = 2 * TILE / 1024 / NWL;   // 1 KB loads per loading wave per stage
constexpr int NB_V = TILE / 1024 / NWL;
constexpr int NB_G = 2;

// Loads issued after those of stage x + 1 when the loading wave waits at the
// top of stage x (slice s), before it issues stage x + D: the stage groups
// x + 2 .. x + D - 1 and the per-chunk loads issued at the tops of stages
// x + 1 - D .. x - 1.
template <int NBX>
__host__ __device__ constexpr int loads_after_next(int s) {
  int n = 0;
  for (int k = 2; k < D; ++k) n += NB_QK + (((s + k) % NS) == 0 ? NB_V : 0);
  for (int k = 1; k <= D - 1; ++k) n += (((s - k) % NS + NS) % NS == 0) ? NBX : 0;
  return n;
}
static_assert(NS == 4 && D <= NS - 1, "one value slot needs the look-ahead inside a chunk");

template <int OM>
struct CO {
  static constexpr int OROW = (OM == O_BF16) ? 128 : 256;
  static constexpr int OTILE = (OM == O_NONE) ? 16 : L * OROW;
  static constexpr int NB_O = (OM == O_NONE) ? 0 : L * OROW / 1024 / NWL;
  static constexpr int NB_X = NB_O + NB_G;
};

template <int OM>
__global__ __launch_bounds__(NTH, 1) void chunk_ws_kernel(SeqArgs a) {
  using C = CO<OM>;
  __shared__ __align__(1024) char sRing[NSLOT][2][TILE];   // [slot][q|k]
  __shared__ __align__(1024) char sV[TILE];
  __shared__ __align__(1024) char sO[2][C::OTILE];         // o~ by chunk parity
  __shared__ __align__(16) float sR[4][NT][64][4];         // scaled readout
  // P: query tiles 0, 1 in rows 0..31, tiles 2, 3 by chunk parity in rows
  // 32..63 and 64..95
  __shared__ __align__(16) bf16_t sP[(L + 32) * PROW];
  // per chunk mod 3: u, M, g, exp(-m), w / sig'
  __shared__ __align__(16) float sGate[3][5][L];
  __shared__ float sQn[L];
  __shared__ __align__(16) float sN[DQK];
  // n~ and w (per chunk mod 3) as three bf16 terms (high, middle, low) and a
  // row of zeros: the A operands of the normaliser MFMAs
  __shared__ __align__(16) bf16_t sNs[4][DQK];
  __shared__ __align__(16) bf16_t sWs[3][4][L];
  __shared__ __align__(256) float sGin[2][2][64];
  // h of two query tiles (32 rows x the 64 columns), staged so that each
  // row leaves in one 128-byte piece
  __shared__ __align__(16) char sH[32 * 128];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const bool state_wave = wave < 4;
  const int cg = wave & 3;   // column group of either role

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
  const int b0w = vt * TV + cg * 16;

  const bf16_t* gq = static_cast<const bf16_t*>(a.q) + head * Ts * DQK;
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * Ts * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * Ts * dv + vt * TV;
  const float* gi = a.i_pre + head * Ts;
  const float* gf = a.f_pre + head * Ts;
  bf16_t* gh = static_cast<bf16_t*>(a.h) + head * Ts * dv + b0w + 4 * g;

  if (tid < DQK) {
    const float n0 = a.C0 ? a.n0[head * DQK + tid] : 0.0f;
    sN[tid] = n0;
    split3_bf16(n0, sNs[0][tid], sNs[1][tid], sNs[2][tid]);
    sNs[3][tid] = 0;
  }
  if (tid < 3 * L) sWs[tid / L][3][tid % L] = 0;
  // P tiles above the diagonal that P V reads (key tile 1 of query tile 0,
  // key tile 3 of query tile 2 in both buffers): zero once, never written
  for (int x = tid; x < 3 * 256; x += NTH) {
    const int t = x >> 8, r = (x >> 4) & 15, cc = x & 15;
    const int row = t == 0 ? r : 32 + 32 * (t - 1) + r;
    const int col = t == 0 ? 16 + cc : 48 + cc;
    sP[row * PROW + col] = 0;
  }
  float m_s = a.C0 ? a.m0[head] : 0.0f;

  // ---- loads (the loading role; lw = 0..3 is the loading wave's index)
  const int lw = cg;
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  int qk_off[NB_QK];
#pragma unroll
  for (int m = 0; m < NB_QK; ++m) {
    const int Gr = (lw * NB_QK + m) % (L / 8);
    const int row = 8 * Gr + ld_r;
    qk_off[m] = row * DQK + 8 * (ld_pc ^ ((row >> 1) & 7));
  }
  int v_off[NB_V];
#pragma unroll
  for (int m = 0; m < NB_V; ++m) {
    const int row = 8 * (lw * NB_V + m) + ld_r;
    v_off[m] = row * dv + 8 * (ld_pc ^ ((row >> 1) & 7));
  }
  auto issue_stage = [&](int x) {
    const int cx = x / NS, sx = x % NS;
    const int cc = cx < nchunks ? cx : nchunks - 1;    // past the end: harmless re-read
    char* slot = sRing[x % NSLOT][0];
    const int64_t base = static_cast<int64_t>(cc) * L * DQK + sx * AS;
#pragma unroll
    for (int m = 0; m < NB_QK; ++m) {
      const int G = lw * NB_QK + m;
      const int mat = G / (L / 8);
      dma16((mat ? gk : gq) + base + qk_off[m], lds_addr(slot + mat * TILE + (G % (L / 8)) * 1024));
    }
    if (sx == 0) {
#pragma unroll
      for (int m = 0; m < NB_V; ++m)
        dma16_nt(gv + static_cast<int64_t>(cc) * L * dv + v_off[m], lds_addr(sV + (lw * NB_V + m) * 1024));
    }
  };
  auto issue_chunk_extras = [&](int c) {
    if (OM != O_NONE) {
      constexpr int RPI = 1024 / C::OROW;
      constexpr int NCH = C::OROW / 16;
#pragma unroll
      for (int m = 0; m < C::NB_O; ++m) {
        const int G = lw * C::NB_O + m;
        const int row = RPI * G + lane / NCH;
        const int pc = lane % NCH;
        const int lc = (OM == O_F32) ? (pc ^ (row & 15)) : (pc ^ ((row >> 1) & 7));
        const int64_t r = head * Ts + static_cast<int64_t>(c) * L + row;
        const char* src = (OM == O_F32)
            ? reinterpret_cast<const char*>(static_cast<const float*>(a.o_pre) + r * dv + vt * TV + 4 * lc)
            : reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.o_pre) + r * dv + vt * TV + 8 * lc);
        dma16_nt(src, lds_addr(sO[c & 1] + G * 1024));
      }
    }
    const int cn = (c + 2 < nchunks) ? c + 2 : nchunks - 1;
    dma4(gi + static_cast<int64_t>(cn) * L + lane, lds_addr(&sGin[c & 1][0][0]));
    dma4(gf + static_cast<int64_t>(cn) * L + lane, lds_addr(&sGin[c & 1][1][0]));
  };

  // Gate scan of one chunk from raw gates gin into sGate[gb], in four parts
  // (spread over the stages of the previous chunk, so that no stage carries
  // the whole dependency chain).  ms is m before the chunk, sg the state
  // scale before it; the last part returns m after it.
  struct GScan {
    float xi, lf, bcum, u, Mx, ML, bL;
  };
  auto scan_part = [&](int part, int gin, int gb, float ms, float sg, GScan& x) {
    float m_after = 0.0f;
    if (part == 0) {
      x.xi = sGin[gin][0][lane];
      x.lf = log_forget_fast(sGin[gin][1][lane], a.fgate_exp);
    } else if (part == 1) {
      x.bcum = scan_add(x.lf);
      x.u = x.xi - x.bcum;
    } else if (part == 2) {
      x.Mx = fmaxf(ms, scan_max(x.u));
      x.ML = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x.Mx), L - 1));
      x.bL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x.bcum), L - 1));
    } else {
      const float gv_ = __expf(ms - x.Mx);
      const float wv = __expf(x.u - x.ML);
      const float gLn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv_), L - 1));
      const float sg_new = gLn * sg < 0x1p-64f ? 1.0f : gLn * sg;
      sGate[gb][0][lane] = x.u;
      sGate[gb][1][lane] = x.Mx;
      sGate[gb][2][lane] = gv_;
      split3_bf16(wv, sWs[gb][0][lane], sWs[gb][1][lane], sWs[gb][2][lane]);
      sGate[gb][3][lane] = __expf(-(x.bcum + x.Mx));
      sGate[gb][4][lane] = wv * __builtin_amdgcn_rcpf(sg_new);
      m_after = x.bL + x.ML;
    }
    return m_after;
  };
  auto scan_gates = [&](int gin, int gb, float ms, float sg) {
    GScan x;
    float m_after = 0.0f;
#pragma unroll
    for (int part = 0; part < 4; ++part) m_after = scan_part(part, gin, gb, ms, sg, x);
    return m_after;
  };

  // ---- prologue
  const bool load_wave = state_wave == STATE_LOADS;
  if (load_wave) {
#pragma unroll
    for (int x = 0; x < D; ++x) issue_stage(x);
    dma4(gi + lane, lds_addr(&sGin[0][0][0]));
    dma4(gf + lane, lds_addr(&sGin[0][1][0]));
    dma4(gi + (nchunks > 1 ? L : 0) + lane, lds_addr(&sGin[1][0][0]));
    dma4(gf + (nchunks > 1 ? L : 0) + lane, lds_addr(&sGin[1][1][0]));
    wait_vm<0>();
  }
  __syncthreads();
  // the gate scans run on state wave 3 (SCAN_WAVE), which has the fewest
  // score tiles
  constexpr int SCAN_WAVE = 3;
  float m_n1 = 0.0f;   // m after the current chunk (scan wave)
  if (wave == SCAN_WAVE) m_n1 = scan_gates(0, 0, m_s, 1.0f);
  __syncthreads();

  const int vr = l16 >> 2, vq = l16 & 3;
  const int kr = l16 >> 2, kq = l16 & 3;

  // Everything below is written without branches on the wave index: the
  // per-wave choices are uniform offsets, so that each stage is one basic
  // block in which the compiler can overlap LDS latency with MFMA work.

  // row sums of P by (chunk parity, key tile, query tile)
  __shared__ float sRs[2][NT][NT][16];
  auto row_sum = [&](int par, int it, int i16) {
    float r = sRs[par][0][it][i16];
#pragma unroll
    for (int jt = 1; jt < NT; ++jt)
      if (jt <= it) r += sRs[par][jt][it][i16];
    return r;
  };

  // P = S (.) D of one tile (key tile jt, query tile it) of the chunk whose
  // transposed scores are in sp, and its row sums (gates from buffer gbx);
  // the part above the diagonal comes out as zeros
  auto finish_one = [&](const f32x4& sp, int it, int jt, int par, int gbx) {
    const float4 uj = *reinterpret_cast<const float4*>(&sGate[gbx][0][jt * 16 + 4 * g]);
    const float uj4[4] = {uj.x, uj.y, uj.z, uj.w};
    const int i = it * 16 + l16;
    const float Mi = sGate[gbx][1][i];
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = jt * 16 + 4 * g + e;
      const float pv = sp[e] * __expf(uj4[e] - Mi);
      pe[e] = (j <= i) ? pv : 0.0f;
    }
    *reinterpret_cast<uint2*>(sP + (i < 32 ? i : i + 32 * par) * PROW + jt * 16 + 4 * g) =
        make_uint2(cvt2(pe[0], pe[1]), cvt2(pe[2], pe[3]));
    sRs[par][jt][it][l16] = sum_groups((pe[0] + pe[1]) + (pe[2] + pe[3]));
  };
  // P V of query tiles it0, it0 + 1 onto their scaled readout, in two steps
  // (the readout can be read a stage before the products)
  auto pv_init = [&](int it0, f32x4* o) {
#pragma unroll
    for (int r = 0; r < 2; ++r) o[r] = *reinterpret_cast<const f32x4*>(&sR[cg][it0 + r][lane][0]);
  };
  auto pv_mma = [&](const bf16x8* vfr, int it0, int par, f32x4* o) {
    uint4 Pf[2][NKS];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = (it0 + r) * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Pf[r][ks] = *reinterpret_cast<const uint4*>(sP + (i < 32 ? i : i + 32 * par) * PROW + 32 * ks + 8 * g);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (32 * ks <= (it0 + r) * 16 + 15) o[r] = mfma16x16x32(vfr[ks], as_bf16x8(Pf[r][ks]), o[r]);
      }
    }
  };
  auto pv_tiles = [&](const bf16x8* vfr, int it0, int par, f32x4* o) {
    pv_init(it0, o);
    pv_mma(vfr, it0, par, o);
  };
  // h of query tiles it0, it0 + 1 of chunk cp in two steps: the reciprocal
  // denominators and the o~ values (gates gb, o~ slot ob), then h from the
  // numerators o
  struct HOp {
    float inv[2];
    float ov[2][4];
  };
  auto h_prep = [&](int it0, int cp, int gb, int ob, HOp& x) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int it = it0 + r;
      const int i = it * 16 + l16;
      const float rs = row_sum(cp & 1, it, l16);
      const float den = fmaxf(fabsf(sGate[gb][2][i] * sQn[i] + rs), sGate[gb][3][i]);
      x.inv[r] = __builtin_amdgcn_rcpf(den);
      if (OM == O_F32) {
        const float4 o4 = *reinterpret_cast<const float4*>(sO[ob] + i * 256 + 16 * ((cg * 4 + g) ^ (i & 15)));
        x.ov[r][0] = o4.x; x.ov[r][1] = o4.y; x.ov[r][2] = o4.z; x.ov[r][3] = o4.w;
      } else if (OM == O_BF16) {
        const uint2 o2 = *reinterpret_cast<const uint2*>(sO[ob] + swz(i, cg * 16 + 4 * g));
        x.ov[r][0] = bf_lo(o2.x); x.ov[r][1] = bf_hi(o2.x); x.ov[r][2] = bf_lo(o2.y); x.ov[r][3] = bf_hi(o2.y);
      }
    }
  };
  auto h_store = [&](const f32x4* o, const HOp& x, int it0, int cp) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = (it0 + r) * 16 + l16;
      float hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = o[r][e] * x.inv[r];
      if (OM != O_NONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] *= sigmoid_fast(x.ov[r][e]);
      }
      st8_nt(gh + (static_cast<int64_t>(cp) * L + i) * dv, cvt2(hv[0], hv[1]), cvt2(hv[2], hv[3]));
    }
  };
  auto h_tiles = [&](const f32x4* o, int it0, int cp, int gb, int ob) {
    HOp x;
    h_prep(it0, cp, gb, ob, x);
    h_store(o, x, it0, cp);
  };
  // in the loop: h of query tiles it0, it0 + 1 into sH (16-byte chunks
  // swizzled by row), written out after the next barrier as whole rows
  auto h_stage = [&](const f32x4* o, const HOp& x) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = o[r][e] * x.inv[r];
      if (OM != O_NONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] *= sigmoid_fast(x.ov[r][e]);
      }
      const int srow = 16 * r + l16, col = cg * 16 + 4 * g;
      *reinterpret_cast<uint2*>(sH + srow * 128 + (((col >> 3) ^ (srow & 7)) << 4) + (col & 7) * 2) =
          make_uint2(cvt2(hv[0], hv[1]), cvt2(hv[2], hv[3]));
    }
  };
  bf16_t* const hrow = static_cast<bf16_t*>(a.h) + head * Ts * dv + vt * TV;
  auto h_flush = [&](int it0, int cp) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int srow = 8 * cg + (lane >> 3), ch = lane & 7;
    const u32x4v v = *reinterpret_cast<const u32x4v*>(sH + srow * 128 + ((ch ^ (srow & 7)) << 4));
    bf16_t* dst = hrow + (static_cast<int64_t>(cp) * L + it0 * 16 + srow) * dv + 8 * ch;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4v*>(dst));
  };
  // value fragments (V^T, this wave's 16 columns) of the chunk in sV
  auto load_vf = [&](bf16x8* dst, uint2* raw) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int col = cg * 16 + 4 * vq;
      raw[2 * ks] = lds_tr(sV, swz(32 * ks + 8 * g + vr, col));
      raw[2 * ks + 1] = lds_tr(sV, swz(32 * ks + 8 * g + 4 + vr, col));
      dst[ks] = join(raw[2 * ks], raw[2 * ks + 1]);
    }
  };

  // Both roles run the same stage sequence (same barriers); each role has
  // its own loop so that its registers are its own.  The loading role waits
  // for the stage's loads before the barrier and issues the loads D stages
  // ahead after it.
  auto wait_next_stage = [&](int s) {
    switch (s) {
      case 0: wait_vm<loads_after_next<C::NB_X>(0)>(); break;
      case 1: wait_vm<loads_after_next<C::NB_X>(1)>(); break;
      case 2: wait_vm<loads_after_next<C::NB_X>(2)>(); break;
      default: wait_vm<loads_after_next<C::NB_X>(3)>(); break;
    }
  };
  auto stage_top_load = [&](int c, int s) {
    const int x = c * NS + s;
    if (x < D) wait_vm<0>();
    else wait_next_stage(s);
    __syncthreads();
    issue_stage(x + D);
    if (s == 0) issue_chunk_extras(c);
    return x % NSLOT;
  };
  auto stage_top_wait = [&](int c, int s) {
    __syncthreads();
    return (c * NS + s) % NSLOT;
  };
  auto stage_top_state = [&](int c, int s) {
    return STATE_LOADS ? stage_top_load(c, s) : stage_top_wait(c, s);
  };
  auto stage_top_intra = [&](int c, int s) {
    return STATE_LOADS ? stage_top_wait(c, s) : stage_top_load(c, s);
  };

  if (state_wave) {
    // compiled once per state wave: its score tiles are fixed at compile time
    for_wave<4>(cg, [&](auto Wc) {
    constexpr int W = decltype(Wc)::value;
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
    float sig = 1.0f;    // C~ = sig * cacc
    f32x4 outT[NT];
    bf16x8 wVf[NKS];
    // score tiles of this wave: key tile W against query tiles W..3, except
    // that wave 3 takes (key 0, query 3) from wave 0 (in sacc_x): 3, 3, 2, 2
    // tiles for waves 0..3
    f32x4 sacc[NT], sacc_x;
    auto own_tile = [&](int it) { return it >= W && !(W == 0 && it == NT - 1); };
    // fragments of one half slice (32 d_qk rows): Q of every query tile and
    // K of key tile W (and of key tile 0 on wave 3) for the scores and the
    // readout; K^T of the half's two C~ row tiles for the update (Kt)
    struct Frag {
      uint4 Qf[NT], Kf, Kf0;
    };
    auto load_half = [&](Frag& f, const char* Qb, const char* Kb, int p) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < NT; ++it) f.Qf[it] = lds_ld16(Qb, swz(it * 16 + l16, 32 * p + 8 * g));
      f.Kf = lds_ld16(Kb, W * 2048 + swz(l16, 32 * p + 8 * g));
      if (W == 3) f.Kf0 = lds_ld16(Kb, swz(l16, 32 * p + 8 * g));
    };
    bf16x8 Kt[NKS][2];
    auto load_kt = [&](const char* Kb, int p) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 32 * p + 8 * kq + 4 * j;
          Kt[ks][j] = join(lds_tr(Kb, swz(32 * ks + 8 * g + kr, col)),
                           lds_tr(Kb, swz(32 * ks + 8 * g + 4 + kr, col)));
        }
      }
    };
    // C~ enters the readout as a (high, remainder) pair of bf16 operands:
    // rounding it to bf16 alone costs up to ~2% of h where the carried and
    // the in-chunk terms cancel.  The pair of the next half's rows is formed
    // during this half's products (those rows are final for the chunk).
    bf16x8 Ahi[2], Alo[2];
    auto split_rows = [&](int t0, bf16x8& hi, bf16x8& lo) __attribute__((always_inline)) {
      float ca[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ca[e] = cacc[t0][e];
        ca[4 + e] = cacc[t0 + 1][e];
      }
      cvt8_split(ca, hi, lo);
    };
    // scores, readout and update of half p of slice s (C~ row tiles
    // 4 s + 2 p + j): the readout of the rows comes before their update
    auto compute_half = [&](const Frag& f, int s, int p, bool renorm, float rf) __attribute__((always_inline)) {
      const int t0 = 4 * s + 2 * p;
#pragma unroll
      for (int it = 0; it < NT; ++it)
        if (own_tile(it)) sacc[it] = mfma16x16x32(as_bf16x8(f.Kf), as_bf16x8(f.Qf[it]), sacc[it]);
      if (W == 3) sacc_x = mfma16x16x32(as_bf16x8(f.Kf0), as_bf16x8(f.Qf[NT - 1]), sacc_x);
#pragma unroll
      for (int it = 0; it < NT; ++it) outT[it] = mfma16x16x32(Ahi[p], as_bf16x8(f.Qf[it]), outT[it]);
#pragma unroll
      for (int it = 0; it < NT; ++it) outT[it] = mfma16x16x32(Alo[p], as_bf16x8(f.Qf[it]), outT[it]);
      split_rows((t0 + 2) & (NCT - 1), Ahi[p ^ 1], Alo[p ^ 1]);
      // scheduling hint: one MFMA, then two VALU, twelve times
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      {
        // the pair is formed here, beside the products, not sunk past the
        // renormalisation branch to its first use
        const uint4 h_ = __builtin_bit_cast(uint4, Ahi[p ^ 1]), l_ = __builtin_bit_cast(uint4, Alo[p ^ 1]);
        asm volatile("" :: "v"(h_.x), "v"(h_.y), "v"(h_.z), "v"(h_.w), "v"(l_.x), "v"(l_.y), "v"(l_.z), "v"(l_.w));
      }
      // the renormalisation (rare) scales the rows before their update
      if (renorm) {
        cacc[t0] *= rf;
        cacc[t0 + 1] *= rf;
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          cacc[t0 + j] = mfma16x16x32(Kt[ks][j], wVf[ks], cacc[t0 + j]);
      }
    };
    Frag F0, F1;
    load_half(F0, sRing[0][0], sRing[0][1], 0);
    split_rows(0, Ahi[0], Alo[0]);
    int gb = 0, gbn = 1, gbp = 2;   // gate buffers of chunks c, c + 1, c - 1
    for (int c = 0; c < nchunks; ++c) {
      // the chunk's gates are read after the first stage's barrier (the
      // scan that writes them ends one stage earlier)
      float gL = 0.0f, sig_new = 0.0f;
      bool renorm = false;
      float m_n2 = 0.0f;
      GScan gsc;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int slot = stage_top_state(c, s);
        if (s == 0) {
          gL = sGate[gb][2][L - 1];
          renorm = gL * sig < 0x1p-64f;
          sig_new = renorm ? 1.0f : gL * sig;
        }
        const char* Qb = sRing[slot][0];
        const char* Kb = sRing[slot][1];
        if (s == 0) {
          uint2 raw[2 * NKS];
          bf16x8 vtmp[NKS];
          load_vf(vtmp, raw);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const float4 w0 = *reinterpret_cast<const float4*>(&sGate[gb][4][32 * ks + 8 * g]);
            const float4 w1 = *reinterpret_cast<const float4*>(&sGate[gb][4][32 * ks + 8 * g + 4]);
            const uint2 lo = raw[2 * ks], hi = raw[2 * ks + 1];
            float xw[8];
            xw[0] = bf_lo(lo.x) * w0.x; xw[1] = bf_hi(lo.x) * w0.y;
            xw[2] = bf_lo(lo.y) * w0.z; xw[3] = bf_hi(lo.y) * w0.w;
            xw[4] = bf_lo(hi.x) * w1.x; xw[5] = bf_hi(hi.x) * w1.y;
            xw[6] = bf_lo(hi.y) * w1.z; xw[7] = bf_hi(hi.y) * w1.w;
            wVf[ks] = cvt8(xw);
          }
#pragma unroll
          for (int it = 0; it < NT; ++it) {
            outT[it] = f32x4{0.f, 0.f, 0.f, 0.f};
            sacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          sacc_x = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // gate operands of this stage's P pass and scaled readout
        float gi4[NT];
        if (s == NS - 1) {
#pragma unroll
          for (int it = 0; it < NT; ++it) gi4[it] = sGate[gb][2][it * 16 + l16];
        }
        // the slice in two halves of 32 d_qk rows; the fragments of each half
        // are read one half ahead (those of half 0 during the previous
        // stage, from the slot its barrier published)
        load_kt(Kb, 0);
        load_half(F1, Qb, Kb, 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(F0, s, 0, renorm, gL * sig);
        __builtin_amdgcn_sched_barrier(0);
        load_kt(Kb, 1);
        {
          const int nslot = (c * NS + s + 1) % NSLOT;
          load_half(F0, sRing[nslot][0], sRing[nslot][1], 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute_half(F1, s, 1, renorm, gL * sig);
        __builtin_amdgcn_sched_barrier(0);
        if (s == NS - 1) {
          // scaled readout for the intra waves
#pragma unroll
          for (int it = 0; it < NT; ++it)
            *reinterpret_cast<f32x4*>(&sR[W][it][lane][0]) = outT[it] * (gi4[it] * sig);
        }
        // P of the chunk at the last stage (tiles 0, 1 are read from stage 1
        // of the next chunk on, tiles 2, 3 from its stage 3)
        if (s == NS - 1) {
#pragma unroll
          for (int it = 0; it < NT; ++it)
            if (own_tile(it)) finish_one(sacc[it], it, W, c & 1, gb);
          if (W == 3) finish_one(sacc_x, NT - 1, 0, c & 1, gb);
        }
        // gate scan of the next chunk: part 0 at stage 0, parts 1 and 2 at
        // stage 1, part 3 at stage 2 (the last stage carries the P pass)
        if (wave == SCAN_WAVE) {
          if (s == 0) scan_part(0, (c + 1) & 1, gbn, m_n1, sig_new, gsc);
          if (s == 1) {
            scan_part(1, (c + 1) & 1, gbn, m_n1, sig_new, gsc);
            scan_part(2, (c + 1) & 1, gbn, m_n1, sig_new, gsc);
          }
          if (s == 2) m_n2 = scan_part(3, (c + 1) & 1, gbn, m_n1, sig_new, gsc);
        }
      }
      m_s = m_n1;
      m_n1 = m_n2;
      sig = sig_new;
      gbp = gb;
      gb = gbn;
      gbn = (gbn == 2) ? 0 : gbn + 1;
    }
    // ---- drain (the two barriers of the intra role's drain)
    if (STATE_LOADS) wait_vm<0>();
    __syncthreads();
    __syncthreads();
    if (a.C1) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
          a.C1[(head * DQK + arow) * dv + b0w + l16] = cacc[t][e] * sig;
        }
      }
      if (vt == 0) {
        if (tid < DQK) a.n1[head * DQK + tid] = sN[tid];
        if (wave == SCAN_WAVE && lane == 0) a.m1[head] = m_s;
      }
    }
    });
  } else {
    const int W = cg;
    // q.n~ of query tile qt = W
    const int qt = W;
    // n~ increments: this wave covers the rows of tile W of every slice
    // (every lane of a 16-lane column holds the same value)
    const int nrow = 32 * (W >> 1) + 8 * (l16 >> 2) + 4 * (W & 1) + (l16 & 3);
    const int ncol = 32 * (W >> 1) + 8 * kq + 4 * (W & 1);   // its K^T fragment column
    // MFMA results are consumed one stage after their issue: the n~
    // increment of the previous slice, q.n~ of the previous chunk, the
    // numerators of two query tiles of chunk c - 1
    f32x4 niP = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 qn = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oacc[2];
    HOp hx;
    uint4 Wx[NKS];   // w terms of the current chunk (A operand, see below)
    float gL_prev = 1.0f;   // with niP = 0: the update before chunk 0 keeps n~
    // value fragments of the current and the previous chunk
    bf16x8 Vf[NKS], Vp[NKS];
    int gb = 0, gbp = 2;   // gate buffers of chunks c, c - 1
    for (int c = 0; c < nchunks; ++c) {
      // (wave-uniform: kept in a scalar register)
      // (read after the first stage's barrier, as in the state role)
      float gL = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int slot = stage_top_intra(c, s);
        if (s == 0) {
          // (wave-uniform: kept in a scalar register)
          gL = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sGate[gb][2][L - 1])));
        }
        const char* Qb = sRing[slot][0];
        const char* Kb = sRing[slot][1];
        if (s == 0) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) Vp[ks] = Vf[ks];
          uint2 raw[2 * NKS];
          load_vf(Vf, raw);
          // q.n~ of chunk c - 1 (its outputs are finished from stage 2 on)
          if (c > 0) sQn[qt * 16 + l16] = (qn[0] + qn[1]) + qn[2];
          qn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            Wx[ks] = *reinterpret_cast<const uint4*>(&sWs[gb][l16 & 3][32 * ks + 8 * g]);
        }
        // Q fragments of query tile qt over the slice
        uint4 Qf[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) Qf[p] = lds_ld16(Qb, qt * 2048 + swz(l16, 32 * p + 8 * g));
        // q.n~ and the n~ increment as MFMAs whose A operand holds the
        // vector (n~, w) split into three bf16 terms, in rows 4r, 4r+1,
        // 4r+2 (row 4r+3 is zero): with B = the Q fragment, D[4r+e][c] is
        // term e of q_c . n~; with B = the K^T fragment of the update, term e
        // of sum_j w_j K[j][row c].  Summing the terms gives the float32
        // product to about 24 significant bits of the vector.
        uint4 Nx[2];
        uint2 Klo[NKS], Khi[NKS];
#pragma unroll
        for (int p = 0; p < 2; ++p)
          Nx[p] = *reinterpret_cast<const uint4*>(&sNs[l16 & 3][32 * (2 * s + p) + 8 * g]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          Klo[ks] = lds_tr(Kb, swz(32 * ks + 8 * g + kr, ncol));
          Khi[ks] = lds_tr(Kb, swz(32 * ks + 8 * g + 4 + kr, ncol));
        }
        // n~ rows of the previous slice: every intra wave has finished
        // reading them (q.n~) before this stage's barrier
        const int sp_ = (s + NS - 1) % NS;
        const int nprow = sp_ * AS + nrow;
        const float nprev = sN[nprow];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < 2; ++p) qn = mfma16x16x32(as_bf16x8(Nx[p]), as_bf16x8(Qf[p]), qn);
        f32x4 ni = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ni = mfma16x16x32(as_bf16x8(Wx[ks]), join(Klo[ks], Khi[ks]), ni);
        {
          const float nv = (s > 0 ? gL : gL_prev) * nprev + ((niP[0] + niP[1]) + niP[2]);
          sN[nprow] = nv;
          split3_bf16(nv, sNs[0][nprow], sNs[1][nprow], sNs[2][nprow]);
        }
        niP = ni;
        __builtin_amdgcn_sched_barrier(0);
        // finishing of chunk c - 1: P V of query tiles 0, 1 at stage 1, their
        // h at stage 2, P V of tiles 2, 3 and the operands of their h at
        // stage 3, and that h at stage 0 of the next chunk
        if (s == 0 && c > 1) h_stage(oacc, hx);
        if (s == 1 && c > 1) h_flush(2, c - 2);
        if (s == 3 && c > 0) h_flush(0, c - 1);
        if (c > 0) {
          if (s == 1) pv_tiles(Vp, 0, (c - 1) & 1, oacc);
          if (s == 2) {
            HOp hy;
            h_prep(0, c - 1, gbp, (c - 1) & 1, hy);
            h_stage(oacc, hy);
            pv_init(2, oacc);   // (the state waves rewrite the readout at stage 3)
          }
          if (s == 3) {
            pv_mma(Vp, 2, (c - 1) & 1, oacc);
            h_prep(2, c - 1, gbp, (c - 1) & 1, hx);
          }
        }
      }
      gL_prev = gL;
      gbp = gb;
      gb = (gb == 2) ? 0 : gb + 1;
    }
    // ---- drain: finish the last two chunks (and the n~ rows of the last
    // slice)
    if (!STATE_LOADS) wait_vm<0>();
    if (nchunks > 1) h_store(oacc, hx, 2, nchunks - 2);
    {
      const int arow = (NS - 1) * AS + nrow;
      sN[arow] = gL_prev * sN[arow] + ((niP[0] + niP[1]) + niP[2]);   // (its bf16 terms are not read again)
    }
    __syncthreads();
    sQn[qt * 16 + l16] = (qn[0] + qn[1]) + qn[2];
    __syncthreads();
#pragma unroll
    for (int it0 = 0; it0 < NT; it0 += 2) {
      pv_tiles(Vf, it0, (nchunks - 1) & 1, oacc);
      h_tiles(oacc, it0, nchunks - 1, gbp, (nchunks - 1) & 1);
    }
  }
}

}  // namespace

bool chunk_ws_supported(const SeqArgs& a, int64_t chunk) {
  return a.qkv_bf16 && a.dqk == DQK && a.dv % TV == 0 && chunk == L && a.T % L == 0;
}

hipError_t launch_chunk_ws(const SeqArgs& a, hipStream_t stream) {
  const unsigned nwg = static_cast<unsigned>(a.B * a.H * (a.dv / TV));
  switch (a.o_mode) {
    case O_F32: chunk_ws_kernel<O_F32><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    case O_BF16: chunk_ws_kernel<O_BF16><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    default: chunk_ws_kernel<O_NONE><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace mlstm
