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
// Because m is known from the gates alone, every weight is <= 1 and no online
// rescaling is needed (unlike softmax attention).
//
// Design (MI355X):
// * One workgroup (4 waves) per (head, 64 value columns).  It walks the chunks
//   in order and keeps its [d_qk x 64] slice of C~ in float32 registers (each
//   wave owns 16 columns, all d_qk rows) for the whole sequence, so the state
//   never round-trips through HBM between chunks.  Workgroups of one head are
//   placed on one XCD so q/k re-reads hit that XCD's L2.
// * Five contractions per chunk, all bf16 MFMA 16x16x32 with fp32 accumulate:
//     S^T = K Q^T (causal tiles only), readout (C~^T Q^T) with C~ taken
//     straight from its accumulator registers, P V, and the state update
//     K^T (w V).  The accumulator layout of the state update is arranged
//     (rows permuted) so that each lane holds 8 consecutive d_qk rows: the
//     readout then feeds C~ to the MFMA without any data movement.
// * q/k are staged through LDS in 64-wide d_qk slices, double buffered, with
//   the next slice's global loads in flight during the current slice's math.
//   k is written twice: row-major (for Q K^T) and transposed (for K^T V, whose
//   contraction runs over tokens).  The transposes are 8x8 register transposes
//   done while staging.
// * The denominator uses the float32 decay-weighted row sums (before P is
//   rounded to bf16) and the float32 n~.
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

constexpr int NW = 4;       // waves per workgroup
constexpr int NTH = 256;    // threads per workgroup
constexpr int TV = 64;      // value columns per workgroup (16 per wave)
constexpr int AS = 64;      // d_qk slice width
constexpr int PAD = 8;      // bf16 row padding in LDS (bank spread)

template <int DQK, int L>
struct CK {
  static constexpr int NT = L / 16;                // 16-token tiles per chunk
  static constexpr int NKS = L / 32;               // 32-token MFMA k-steps
  static constexpr int NS = DQK / AS;              // d_qk slices
  static constexpr int NCT = DQK / 16;             // 16-row C~ tiles
  static constexpr int QROW = AS + PAD;            // row stride of Q/K slices
  static constexpr int KTROW = L + PAD;            // row stride of K^T slice
  static constexpr int PROW = L + PAD;             // row stride of P and V^T
  static constexpr int NTILES = NT * (NT + 1) / 2; // causal 16x16 score tiles
  static constexpr int TPW = (NTILES + NW - 1) / NW;
  static constexpr int NBLK = L * AS / 64;         // 8x8 blocks per staged slice
  static constexpr int PBUF = (L > TV ? L : TV) * PROW;
  static constexpr int NQN = (NT + NW - 1) / NW;
  static_assert(DQK % AS == 0 && NS <= NW, "d_qk must be 64, 128, 192 or 256");
  static_assert(L % 32 == 0 && L <= 128, "chunk must be 32, 64 or 128");
  static_assert(2 * NBLK <= NTH && L <= NTH, "staging roles");
};

// Physical row of d_qk row `a` (within a 64-wide slice) in the staged K^T
// buffer.  The state-update MFMA for C~ tile t reads rows 16t..16t+15 and its
// output row r then holds d_qk row 32(t/2) + 8(r/4) + 4(t%2) + r%4, so a lane
// (group g) ends up with rows 32p + 8g + 0..7 of tile pair p.
__device__ __forceinline__ int kt_row(int a) {
  const int p = a >> 5, rem = a & 31;
  return 32 * p + 16 * ((rem & 7) >> 2) + 4 * (rem >> 3) + (rem & 3);
}

__device__ __forceinline__ uint4 ld16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(bf16_t* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 8x8 transpose of bf16: in[r] holds row r (8 elements); out[e] = column e.
__device__ __forceinline__ void transpose8x8(const uint4* in, uint4* out) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[4r + d] = elems 2d, 2d+1 of row r
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t A = w[4 * (2 * p) + d], Bw = w[4 * (2 * p + 1) + d];
      lo[p] = (A & 0xffffu) | (Bw << 16);
      hi[p] = (A >> 16) | (Bw & 0xffff0000u);
    }
    out[2 * d] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    out[2 * d + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

template <int DQK, int L, int OM, int MINW>
__global__ __launch_bounds__(NTH, MINW) void chunk_mfma_kernel(SeqArgs a) {
  using C = CK<DQK, L>;
  __shared__ __align__(16) bf16_t sQ[2][L * C::QROW];
  __shared__ __align__(16) bf16_t sK[2][L * C::QROW];
  __shared__ __align__(16) bf16_t sKt[2][AS * C::KTROW];
  __shared__ __align__(16) bf16_t sPV[C::PBUF];   // V^T (chunk prologue) / P (epilogue)
  __shared__ __align__(16) float sGate[2][5][L];  // u, M, g, w, exp(-m)  by chunk parity
  __shared__ float sRs[NW][L];
  __shared__ float sQn[L];
  __shared__ __align__(16) float sN[DQK];
  __shared__ float sMs[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // ---- workgroup -> (head, value tile); the tiles of a head share an XCD
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
  const int64_t T = a.T;
  const int nchunks = static_cast<int>(T / L);
  const int b0w = vt * TV + wave * 16;   // first value column of this wave

  const bf16_t* gq = static_cast<const bf16_t*>(a.q) + head * T * DQK;
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * T * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * T * dv + vt * TV;
  const float* gi = a.i_pre + head * T;
  const float* gf = a.f_pre + head * T;
  bf16_t* gh = static_cast<bf16_t*>(a.h) + head * T * dv;

  // ---- state: C~ columns of this wave in registers, n~ in LDS, m in a register
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

  // ---- staging roles
  const bool k_role = tid < C::NBLK;
  const bool q_role = !k_role && tid < 2 * C::NBLK;
  const int sblk = k_role ? tid : tid - C::NBLK;
  const int s_jb = sblk / (AS / 8), s_ab = sblk % (AS / 8);
  const bf16_t* s_src = k_role ? gk : gq;
  uint4 pre[8];  // next slice (8 rows x 8 d_qk columns)
  auto load_slice = [&](int c, int s) {
    if (k_role || q_role) {
      const bf16_t* src = s_src + (static_cast<int64_t>(c) * L + 8 * s_jb) * DQK + s * AS + 8 * s_ab;
#pragma unroll
      for (int r = 0; r < 8; ++r) pre[r] = ld16(src + r * DQK);
    }
  };
  auto store_slice = [&](int buf) {
    if (k_role || q_role) {
      bf16_t* dst = (k_role ? sK[buf] : sQ[buf]) + 8 * s_jb * C::QROW + 8 * s_ab;
#pragma unroll
      for (int r = 0; r < 8; ++r) st16(dst + r * C::QROW, pre[r]);
    }
    if (k_role) {
      uint4 col[8];
      transpose8x8(pre, col);
#pragma unroll
      for (int e = 0; e < 8; ++e) st16(sKt[buf] + kt_row(8 * s_ab + e) * C::KTROW + 8 * s_jb, col[e]);
    }
  };
  // V tile: thread t < L owns an 8x8 block (8 tokens x 8 columns)
  const bool v_role = tid < L;
  const int v_jb = tid >> 3, v_cb = tid & 7;
  uint4 pv[8];
  auto load_v = [&](int c) {
    if (v_role) {
      const bf16_t* src = gv + (static_cast<int64_t>(c) * L + 8 * v_jb) * dv + 8 * v_cb;
#pragma unroll
      for (int r = 0; r < 8; ++r) pv[r] = ld16(src + static_cast<int64_t>(r) * dv);
    }
  };
  float pgi[2], pgf[2];  // wave 0: gate preactivations of tokens lane, lane + 64
  auto load_gates = [&](int c) {
    if (wave == 0) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = lane + 64 * h2;
        pgi[h2] = (j < L) ? gi[static_cast<int64_t>(c) * L + j] : 0.0f;
        pgf[h2] = (j < L) ? gf[static_cast<int64_t>(c) * L + j] : 0.0f;
      }
    }
  };

  load_gates(0);
  load_v(0);
  load_slice(0, 0);

  f32x4 outT[C::NT];
  f32x4 sacc[C::TPW];
  uint4 Vf[C::NKS];
  bf16x8 wVf[C::NKS];
  float nnew = 0.0f;

  for (int c = 0; c < nchunks; ++c) {
    const int par = c & 1;
    // ================= prologue: gates, V^T fragments
    if (wave == 0) {
      float lf[2], bcum[2], u[2], Mx[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = lane + 64 * h2;
        lf[h2] = (j < L) ? log_forget(pgf[h2], a.fgate_exp) : 0.0f;
      }
      bcum[0] = wave_incl_sum(lf[0], lane);
      u[0] = (lane < L) ? pgi[0] - bcum[0] : -INFINITY;
      Mx[0] = fmaxf(m_s, wave_incl_max(u[0], lane));
      if (L > 64) {
        bcum[1] = wave_incl_sum(lf[1], lane) + __shfl(bcum[0], 63, 64);
        u[1] = pgi[1] - bcum[1];
        Mx[1] = fmaxf(__shfl(Mx[0], 63, 64), wave_incl_max(u[1], lane));
      }
      const float Mlast = (L > 64) ? __shfl(Mx[1], (L - 1) & 63, 64) : __shfl(Mx[0], (L - 1) & 63, 64);
      const float blast = (L > 64) ? __shfl(bcum[1], (L - 1) & 63, 64) : __shfl(bcum[0], (L - 1) & 63, 64);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = lane + 64 * h2;
        if (j < L) {
          sGate[par][0][j] = u[h2];
          sGate[par][1][j] = Mx[h2];
          sGate[par][2][j] = __expf(m_s - Mx[h2]);
          sGate[par][3][j] = __expf(u[h2] - Mlast);
          sGate[par][4][j] = __expf(-(bcum[h2] + Mx[h2]));
        }
      }
      if (lane == 0) sMs[par] = blast + Mlast;
    }
    if (v_role) {
      uint4 col[8];
      transpose8x8(pv, col);
#pragma unroll
      for (int e = 0; e < 8; ++e) st16(sPV + (8 * v_cb + e) * C::PROW + 8 * v_jb, col[e]);
    }
    if (c + 1 < nchunks) {
      load_gates(c + 1);
      load_v(c + 1);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      Vf[ks] = ld16(sPV + (wave * 16 + l16) * C::PROW + 32 * ks + 8 * g);
      const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g + 4]);
      float x[8];
      x[0] = bf_lo(Vf[ks].x) * w0.x; x[1] = bf_hi(Vf[ks].x) * w0.y;
      x[2] = bf_lo(Vf[ks].y) * w0.z; x[3] = bf_hi(Vf[ks].y) * w0.w;
      x[4] = bf_lo(Vf[ks].z) * w1.x; x[5] = bf_hi(Vf[ks].z) * w1.y;
      x[6] = bf_lo(Vf[ks].w) * w1.z; x[7] = bf_hi(Vf[ks].w) * w1.w;
      wVf[ks] = to_bf16x8(x);
    }
    const float gL = sGate[par][2][L - 1];

#pragma unroll
    for (int it = 0; it < C::NT; ++it) outT[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C::TPW; ++k) sacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    float qnp[C::NQN];
#pragma unroll
    for (int k = 0; k < C::NQN; ++k) qnp[k] = 0.0f;
    float4 oreg[C::NT];

    // ================= d_qk slices
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const int buf = (c * C::NS + s) & 1;
      store_slice(buf);
      if (s + 1 < C::NS) load_slice(c, s + 1);
      else if (c + 1 < nchunks) load_slice(c + 1, 0);
      if (s == C::NS - 1 && OM != O_NONE) {
#pragma unroll
        for (int it = 0; it < C::NT; ++it) {
          const int64_t row = head * T + static_cast<int64_t>(c) * L + it * 16 + l16;
          if (OM == O_F32) {
            oreg[it] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.o_pre) + row * dv + b0w + 4 * g);
          } else {
            const uint2 u2 = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(a.o_pre) + row * dv + b0w + 4 * g);
            oreg[it] = make_float4(bf_lo(u2.x), bf_hi(u2.x), bf_lo(u2.y), bf_hi(u2.y));
          }
        }
      }
      __syncthreads();

      const bf16_t* Qb = sQ[buf];
      const bf16_t* Kb = sK[buf];
      const bf16_t* Ktb = sKt[buf];
#pragma unroll
      for (int p = 0; p < AS / 32; ++p) {
        const int P = s * (AS / 32) + p;   // C~ tile pair index
        float ca[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ca[e] = cacc[2 * P][e];
          ca[4 + e] = cacc[2 * P + 1][e];
        }
        const bf16x8 A_C = to_bf16x8(ca);
        const float4 n0v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g]);
        const float4 n1v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g + 4]);
        uint4 Qf[C::NT];
#pragma unroll
        for (int it = 0; it < C::NT; ++it) {
          Qf[it] = ld16(Qb + (it * 16 + l16) * C::QROW + 32 * p + 8 * g);
          outT[it] = mfma16x16x32(A_C, as_bf16x8(Qf[it]), outT[it]);
          if (it % NW == wave) {
            qnp[it / NW] += bf_lo(Qf[it].x) * n0v.x + bf_hi(Qf[it].x) * n0v.y +
                            bf_lo(Qf[it].y) * n0v.z + bf_hi(Qf[it].y) * n0v.w +
                            bf_lo(Qf[it].z) * n1v.x + bf_hi(Qf[it].z) * n1v.y +
                            bf_lo(Qf[it].w) * n1v.z + bf_hi(Qf[it].w) * n1v.w;
          }
        }
#pragma unroll
        for (int it = 0; it < C::NT; ++it) {
#pragma unroll
          for (int jt = 0; jt <= it; ++jt) {
            const int n = it * (it + 1) / 2 + jt;
            if (n % NW == wave) {
              const uint4 Kf = ld16(Kb + (jt * 16 + l16) * C::QROW + 32 * p + 8 * g);
              sacc[n / NW] = mfma16x16x32(as_bf16x8(Kf), as_bf16x8(Qf[it]), sacc[n / NW]);
            }
          }
        }
      }
      // state update of this slice's rows (after their readout above)
#pragma unroll
      for (int tl = 0; tl < AS / 16; ++tl) {
        const int t = s * (AS / 16) + tl;
        cacc[t] *= gL;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          const uint4 Af = ld16(Ktb + (16 * tl + l16) * C::KTROW + 32 * ks + 8 * g);
          cacc[t] = mfma16x16x32(as_bf16x8(Af), wVf[ks], cacc[t]);
        }
      }
      // n~ update for this slice's rows: wave (s % NW), lane = row in slice
      if (wave == s % NW) {
        float acc = gL * sN[s * AS + lane];
        const bf16_t* kr = Ktb + kt_row(lane) * C::KTROW;
#pragma unroll
        for (int j = 0; j < L; j += 8) {
          const uint4 k8 = ld16(kr + j);
          const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][3][j]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][3][j + 4]);
          acc += bf_lo(k8.x) * w0.x + bf_hi(k8.x) * w0.y + bf_lo(k8.y) * w0.z + bf_hi(k8.y) * w0.w +
                 bf_lo(k8.z) * w1.x + bf_hi(k8.z) * w1.y + bf_lo(k8.w) * w1.z + bf_hi(k8.w) * w1.w;
        }
        nnew = acc;
      }
    }

    // ================= epilogue: P = S (.) D, row sums, P V, output
    float rsp[C::NT];
#pragma unroll
    for (int it = 0; it < C::NT; ++it) rsp[it] = 0.0f;
#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
#pragma unroll
     for (int jt = 0; jt <= it; ++jt) {
      const int n = it * (it + 1) / 2 + jt;
      if (n % NW == wave) {
        const int i = it * 16 + l16;
        const float Mi = sGate[par][1][i];
        const float4 uj = *reinterpret_cast<const float4*>(&sGate[par][0][jt * 16 + 4 * g]);
        float pe[4];
        const float ujv[4] = {uj.x, uj.y, uj.z, uj.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jt * 16 + 4 * g + e;
          pe[e] = (j <= i) ? sacc[n / NW][e] * __expf(ujv[e] - Mi) : 0.0f;
        }
        rsp[it] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
        uint2 pk;
        pk.x = pack_bf2(pe[0], pe[1]);
        pk.y = pack_bf2(pe[2], pe[3]);
        *reinterpret_cast<uint2*>(sPV + i * C::PROW + jt * 16 + 4 * g) = pk;
        // P V runs in 32-token k-steps: the tile right of an even diagonal
        // tile lies in the same step and must read as zero (j > i)
        if (jt == it && (it & 1) == 0)
          *reinterpret_cast<uint2*>(sPV + i * C::PROW + (jt + 1) * 16 + 4 * g) = make_uint2(0u, 0u);
      }
     }
    }
#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
      float r = rsp[it];
      r += __shfl_xor(r, 16, 64);
      r += __shfl_xor(r, 32, 64);
      if (g == 0) sRs[wave][it * 16 + l16] = r;
      if (it % NW == wave) {
        float qv = qnp[it / NW];
        qv += __shfl_xor(qv, 16, 64);
        qv += __shfl_xor(qv, 32, 64);
        if (g == 0) sQn[it * 16 + l16] = qv;
      }
    }
    __syncthreads();
    if (wave < C::NS) sN[wave * AS + lane] = nnew;

#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
      const int i = it * 16 + l16;
      const float gi_ = sGate[par][2][i];
      f32x4 o = outT[it] * gi_;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        if (32 * ks <= it * 16 + 15) {
          const uint4 Pf = ld16(sPV + i * C::PROW + 32 * ks + 8 * g);
          o = mfma16x16x32(as_bf16x8(Vf[ks]), as_bf16x8(Pf), o);
        }
      }
      const float rs = (sRs[0][i] + sRs[1][i]) + (sRs[2][i] + sRs[3][i]);
      const float den = fmaxf(fabsf(gi_ * sQn[i] + rs), sGate[par][4][i]);
      const float inv = 1.0f / den;
      float hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = o[e] * inv;
      if (OM != O_NONE) {
        hv[0] *= sigmoidf_(oreg[it].x);
        hv[1] *= sigmoidf_(oreg[it].y);
        hv[2] *= sigmoidf_(oreg[it].z);
        hv[3] *= sigmoidf_(oreg[it].w);
      }
      uint2 pk;
      pk.x = pack_bf2(hv[0], hv[1]);
      pk.y = pack_bf2(hv[2], hv[3]);
      *reinterpret_cast<uint2*>(gh + (static_cast<int64_t>(c) * L + i) * dv + b0w + 4 * g) = pk;
    }
    m_s = sMs[par];
    __syncthreads();
  }

  // ---- final state
  if (a.C1) {
#pragma unroll
    for (int t = 0; t < C::NCT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int arow = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
        a.C1[(head * DQK + arow) * dv + b0w + l16] = cacc[t][e];
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
  constexpr int MINW = 1;  // one 4-wave workgroup per CU: up to 512 registers per lane
  chunk_mfma_kernel<DQK, L, OM, MINW><<<dim3(nwg), dim3(NTH), 0, stream>>>(a);
  return hipGetLastError();
}

template <int DQK, int OM>
hipError_t launch_L(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  switch (chunk) {
    case 32: return launch_shape<DQK, 32, OM>(a, stream);
    case 64: return launch_shape<DQK, 64, OM>(a, stream);
    default: return launch_shape<DQK, 128, OM>(a, stream);
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
  return a.qkv_bf16 && (a.dqk == 64 || a.dqk == 128 || a.dqk == 256) && a.dv % TV == 0 &&
         (chunk == 32 || chunk == 64 || chunk == 128) && a.T % chunk == 0;
}

size_t chunk_mfma_workspace(const SeqArgs&, int64_t) { return 0; }

hipError_t launch_chunk_mfma(const SeqArgs& a, int64_t chunk, void*, hipStream_t stream) {
  switch (a.o_mode) {
    case O_F32: return launch_D<O_F32>(a, chunk, stream);
    case O_BF16: return launch_D<O_BF16>(a, chunk, stream);
    default: return launch_D<O_NONE>(a, chunk, stream);
  }
}

}  // namespace mlstm
