// Chunkwise backward pass of the mLSTM cell (gfx950): gradients of h (and of
// the final memory) with respect to q, k, v, i~, f~, o~ and the initial state.
//
// Method: the forward pass of the xLSTM post (llms.blog), section 3
// "Associative Matrix Cell State" and "The Parallel Dual Form", with the
// running maximum of section 2 "The Normalizer State and Numerical
// Stabilization".  The pages print no gradient; the one evaluated here is
// the derivative of that forward pass, written in the chunk variables of the
// forward kernels.  Within a chunk of L tokens starting from the stored state
// (C~_s, n~_s, m_s), with u_j, M_i, m_i, D_ij, g_i, w_j as in the forward:
//
//   den_i  = max(|g_i q_i.n~_s + sum_j D_ij (q_i.k_j)|, exp(-m_i))
//   r_i    = sigmoid(o~_i) (.) dh_i / den_i
//   dnq_i  = -(dh_i . h_i) / den_i * sign(.)   where |.| >= exp(-m_i), else 0
//   W_ij   = D_ij (r_i . v_j + dnq_i)                     (j <= i)
//   dq_i   = sum_j W_ij k_j + g_i (C~_s r_i + dnq_i n~_s)
//   dk_j   = sum_i W_ij q_i + w_j (dC_e v_j + dn_e)
//   dv_j   = sum_i D_ij (q_i.k_j) r_i + w_j dC_e^T k_j
//   do~_i  = dh_i (.) h_i (.) (1 - sigmoid(o~_i))
//   dC_s   = g_L dC_e + sum_i g_i q_i r_i^T,   dn_s = g_L dn_e + sum_i g_i dnq_i q_i
//
// where dC, dn are the gradients of the memory in the scale of the stored
// state at the chunk boundary (dC = e^{m} dL/dC_true).  Every factor is the
// forward's own stabilized one, so nothing overflows.  Summing the token
// contributions gives two identities used for the gates:
//   di~_t = k_t . dk_t,
//   d(log f_t) = sum_{t'>=t} (q_t'.dq_t' - k_t'.dk_t') + <dC1, C~_T> + <dn1, n~_T>.
//
// Passes (all on the launch stream, sharing one workspace):
//   1. beta_t = dh_t . h_t per token;
//   2. a forward state pass that stores (C~, n~, m) at every chunk boundary;
//   3. a reverse pass over the chunks per (head, 32 or 16 value columns): it
//      carries dC in registers and writes dv, do~ and per-column-block
//      partial sums of dq and dk;
//   4. per token: the sums of the partials, di~ and q.dq - k.dk;
//   5. per head: the reverse prefix sum that gives df~, and dm0.
// All arithmetic is float32 on the vector ALUs; this is the first, simple
// form of the backward pass.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

constexpr int NTB = 256;   // threads per workgroup

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return to_f32<T>(static_cast<const T*>(p)[i]);
}

// Copy of an R x NC tile (row-major source of element type S, leading
// dimension ld elements, first element at src[base]) into LDS as float32 with
// row stride dst_ld, by 16-byte vector loads: all of a thread's loads are
// issued before any is converted, so their latencies overlap.  NC must be a
// multiple of 8 (bf16) / 4 (float32) and every row 16-byte aligned.
template <typename S, int MAXE>
__device__ __forceinline__ void load_tile(float* dst, int dst_ld, const void* src, int64_t base,
                                          int64_t ld, int R, int NC) {
  constexpr int VE = 16 / static_cast<int>(sizeof(S));
  constexpr int MAXV = (MAXE / VE + NTB - 1) / NTB;
  const int per_row = NC / VE;
  const int nv = R * per_row;
  uint4 buf[MAXV];
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int e = static_cast<int>(threadIdx.x) + k * NTB;
    if (e < nv) {
      const int r = e / per_row, c = (e % per_row) * VE;
      buf[k] = *reinterpret_cast<const uint4*>(static_cast<const S*>(src) + base + r * ld + c);
    }
  }
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int e = static_cast<int>(threadIdx.x) + k * NTB;
    if (e < nv) {
      const int r = e / per_row, c = (e % per_row) * VE;
      float* d = dst + r * dst_ld + c;
      if (sizeof(S) == 2) {
        d[0] = bf_lo(buf[k].x); d[1] = bf_hi(buf[k].x); d[2] = bf_lo(buf[k].y); d[3] = bf_hi(buf[k].y);
        d[4] = bf_lo(buf[k].z); d[5] = bf_hi(buf[k].z); d[6] = bf_lo(buf[k].w); d[7] = bf_hi(buf[k].w);
      } else {
        d[0] = __uint_as_float(buf[k].x); d[1] = __uint_as_float(buf[k].y);
        d[2] = __uint_as_float(buf[k].z); d[3] = __uint_as_float(buf[k].w);
      }
    }
  }
}

// sum_{x < n} a[x sa] b[x sb] with four partial sums, so that the LDS reads
// of several terms are in flight at once.
__device__ __forceinline__ float dot4(const float* a, int sa, const float* b, int sb, int n) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int x = 0;
#pragma unroll 2
  for (; x + 4 <= n; x += 4) {
    s0 += a[x * sa] * b[x * sb];
    s1 += a[(x + 1) * sa] * b[(x + 1) * sb];
    s2 += a[(x + 2) * sa] * b[(x + 2) * sb];
    s3 += a[(x + 3) * sa] * b[(x + 3) * sb];
  }
  for (; x < n; ++x) s0 += a[x * sa] * b[x * sb];
  return (s0 + s1) + (s2 + s3);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < NTB / 64; ++w) s += red[w];
  return s;
}

// ---- pass 1: beta_t = dh_t . h_t: half a wave per token, 8 elements (16 or
// 32 bytes) per lane per step; d_v is a multiple of 16
template <typename T>
__device__ __forceinline__ void load8f(const void* p, int64_t i, float* x) {
  if (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(p) + i);
    x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
    x[4] = bf_lo(u.z); x[5] = bf_hi(u.z); x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
  } else {
    const float4 f0 = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 f1 = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    x[0] = f0.x; x[1] = f0.y; x[2] = f0.z; x[3] = f0.w;
    x[4] = f1.x; x[5] = f1.y; x[6] = f1.z; x[7] = f1.w;
  }
}

template <typename T>
__global__ __launch_bounds__(NTB) void bwd_beta_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63, hl = lane & 31;
  const int64_t tok = (static_cast<int64_t>(blockIdx.x) * (NTB / 64) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool live = tok < a.B * a.H * a.T;
  float s = 0.0f;
  if (live) {
    for (int64_t b = 8 * hl; b < a.dv; b += 256) {
      float x[8], y[8];
      load8f<T>(a.dh, tok * a.dv + b, x);
      load8f<T>(a.h, tok * a.dv + b, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += x[e] * y[e];
    }
  }
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);   // within the half-wave
  if (live && hl == 0) a.ws_beta[tok] = s;
}

// Gate scan of one chunk of L <= 64 tokens by wave 0 into LDS: per token j,
// u_j = i~_j - b_j (b: in-chunk prefix sum of log f), M_j = max(ms, max u),
// m_j = b_j + M_j, g_j = exp(ms - M_j), w_j = exp(u_j - M_L).  Returns nothing;
// every wave reads the arrays after the next barrier.
struct GateLds {
  float u[64], M[64], m[64], g[64], w[64], lfv[64];
};

template <int L>
__device__ __forceinline__ void gate_scan(const BwdArgs& a, int64_t tok0, float ms, GateLds& G) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < L;
  const float fpre = in ? a.f_pre[tok0 + lane] : 0.0f;
  const float lf = in ? (a.fgate_exp ? fpre : log_sigmoid(fpre)) : 0.0f;
  const float bc = mk::scan_add(lf);
  const float u = in ? a.i_pre[tok0 + lane] - bc : -INFINITY;
  const float Mx = fmaxf(ms, mk::scan_max(u));
  const float ML = __shfl(Mx, L - 1, 64);
  if (in) {
    G.u[lane] = u;
    G.M[lane] = Mx;
    G.m[lane] = bc + Mx;
    G.g[lane] = __expf(ms - Mx);
    G.w[lane] = __expf(u - ML);
    G.lfv[lane] = lf;
  }
}

// ---- pass 2: chunk-boundary states.  Workgroup = (head, TV value columns);
// thread t owns column t % TV of rows t / TV + (NTB / TV) r of C~.
template <typename T, int TV, int L>
__global__ __launch_bounds__(NTB) void bwd_states_kernel(BwdArgs a) {
  constexpr int RSTEP = NTB / TV;
  __shared__ float sK[L * 256];
  __shared__ float sWV[L * TV];
  __shared__ GateLds G;
  __shared__ float sMs;
  const int tid = threadIdx.x;
  const int ncb = static_cast<int>(a.dv / TV);
  const int64_t bh = blockIdx.x / ncb;
  const int cb = blockIdx.x % ncb;
  const int dqk = static_cast<int>(a.dqk), dv = static_cast<int>(a.dv);
  const int ne = dqk / RSTEP;                    // owned rows (<= 256 / RSTEP)
  const int b = tid % TV, r0 = tid / TV;
  const int64_t nT = a.T;
  const int nc = static_cast<int>(nT / L);
  float C[256 / RSTEP];
  float n[256 / RSTEP];
  float m = a.C0 ? a.m0[bh] : 0.0f;
  for (int r = 0; r < ne; ++r) {
    const int row = r0 + RSTEP * r;
    C[r] = a.C0 ? a.C0[(bh * dqk + row) * dv + cb * TV + b] : 0.0f;
    n[r] = a.C0 ? a.n0[bh * dqk + row] : 0.0f;
  }
  const int64_t nb = static_cast<int64_t>(nc + 1);
  for (int c = 0; c <= nc; ++c) {
    // stored state at boundary c (before chunk c; c = nc: the final state)
    float* wsC = a.ws_C + ((bh * nb + c) * dqk) * dv + cb * TV + b;
    for (int r = 0; r < ne; ++r) {
      const int row = r0 + RSTEP * r;
      wsC[static_cast<int64_t>(row) * dv] = C[r];
      if (cb == 0 && b == 0) a.ws_n[(bh * nb + c) * dqk + row] = n[r];
    }
    if (cb == 0 && tid == 0) a.ws_m[bh * nb + c] = m;
    if (c == nc) break;
    const int64_t tok0 = bh * nT + static_cast<int64_t>(c) * L;
    __syncthreads();
    if (tid < 64) gate_scan<L>(a, tok0, m, G);
    load_tile<T, L * 256>(sK, dqk, a.k, tok0 * dqk, dqk, L, dqk);
    load_tile<T, L * TV>(sWV, TV, a.v, tok0 * dv + cb * TV, dv, L, TV);
    __syncthreads();
    for (int e = tid; e < L * TV; e += NTB) sWV[e] *= G.w[e / TV];
    if (tid == 0) sMs = G.m[L - 1];
    __syncthreads();
    const float gL = G.g[L - 1];
    for (int r = 0; r < ne; ++r) {
      const int row = r0 + RSTEP * r;
      float acc = gL * C[r], accn = gL * n[r];
#pragma unroll 8
      for (int j = 0; j < L; ++j) {
        const float kv = sK[j * dqk + row];
        acc += kv * sWV[j * TV + b];
        accn += kv * G.w[j];
      }
      C[r] = acc;
      n[r] = accn;
    }
    m = sMs;
  }
}

// ---- pass 3: reverse over the chunks.
template <typename T, typename TO, int TV, int L>
__global__ __launch_bounds__(NTB) void bwd_rev_kernel(BwdArgs a) {
  constexpr int RSTEP = NTB / TV;
  // LDS rows are padded by one float so that lanes walking a column (token
  // index across lanes) hit distinct banks
  constexpr int TP = TV + 1;   // [d_qk][TV] tiles
  constexpr int LP = L + 1;    // [L][L] tiles
  __shared__ float sQ[L * 257];
  __shared__ float sKt[L * 257];
  __shared__ float sX[256 * TP];       // C~_s, then dC_e (own columns)
  __shared__ float sV[L * TP];
  __shared__ float sR[L * TP];
  __shared__ float sS[L * LP];         // q_i . k_j
  __shared__ float sDm[L * LP];        // D_ij, zero above the diagonal
  __shared__ float sW[L * LP];
  __shared__ float sRg[L * TP];        // g_i r_i
  __shared__ float sN[256];            // n~_s
  __shared__ float sDn[256];           // dn_e, then dn_s
  __shared__ float sQn[L], sDen[L], sDnq[L], sBeta[L];
  __shared__ GateLds G;
  __shared__ float sRed[NTB / 64];
  const int tid = threadIdx.x;
  const int ncb = static_cast<int>(a.dv / TV);
  const int64_t bh = blockIdx.x / ncb;
  const int cb = blockIdx.x % ncb;
  const bool lead = cb == 0;           // adds the terms shared by all column blocks
  const int dqk = static_cast<int>(a.dqk), dv = static_cast<int>(a.dv);
  const int QP = dqk + 1;              // padded row of the [L][d_qk] tiles
  const int ne = dqk / RSTEP;
  const int b = tid % TV, r0 = tid / TV;
  const int64_t nT = a.T;
  const int nc = static_cast<int>(nT / L);
  const int64_t nb = static_cast<int64_t>(nc + 1);
  // carried dC (own columns, this thread's rows) and dn (all rows, in LDS)
  float dC[256 / RSTEP];
  {
    const float* src = a.dC1 ? a.dC1 + (bh * dqk) * dv + cb * TV + b : nullptr;
    for (int r = 0; r < ne; ++r) dC[r] = src ? src[static_cast<int64_t>(r0 + RSTEP * r) * dv] : 0.0f;
    for (int e = tid; e < dqk; e += NTB) sDn[e] = a.dn1 ? a.dn1[bh * dqk + e] : 0.0f;
  }
  for (int c = nc - 1; c >= 0; --c) {
    const int64_t tok0 = bh * nT + static_cast<int64_t>(c) * L;
    const float ms = a.ws_m[bh * nb + c];
    __syncthreads();
    // ---- loads
    if (tid < 64) gate_scan<L>(a, tok0, ms, G);
    load_tile<T, L * 256>(sQ, QP, a.q, tok0 * dqk, dqk, L, dqk);
    load_tile<T, L * 256>(sKt, QP, a.k, tok0 * dqk, dqk, L, dqk);
    load_tile<T, L * TV>(sV, TP, a.v, tok0 * dv + cb * TV, dv, L, TV);
    load_tile<float, 256 * TV>(sX, TP, a.ws_C, ((bh * nb + c) * dqk) * dv + cb * TV, dv, dqk, TV);
    for (int e = tid; e < dqk; e += NTB) sN[e] = a.ws_n[(bh * nb + c) * dqk + e];
    for (int e = tid; e < L; e += NTB) sBeta[e] = a.ws_beta[tok0 + e];
    __syncthreads();
    // ---- scores, q.n~_s and the decay matrix
    for (int e = tid; e < L * L; e += NTB) {
      const int i = e / L, j = e % L;
      sS[i * LP + j] = dot4(sQ + i * QP, 1, sKt + j * QP, 1, dqk);
      sDm[i * LP + j] = j <= i ? __expf(G.u[j] - G.M[i]) : 0.0f;
    }
    for (int i = tid; i < L; i += NTB) {
      sQn[i] = dot4(sQ + i * QP, 1, sN, 1, dqk);
    }
    __syncthreads();
    // ---- denominators and the normalizer gradient per token
    for (int i = tid; i < L; i += NTB) {
      float nq = G.g[i] * sQn[i];
#pragma unroll 8
      for (int j = 0; j <= i; ++j) nq += sDm[i * LP + j] * sS[i * LP + j];
      const float floor_ = __expf(-G.m[i]);
      const float den = fmaxf(fabsf(nq), floor_);
      sDen[i] = den;
      sDnq[i] = fabsf(nq) >= floor_ ? (nq >= 0.0f ? -sBeta[i] / den : sBeta[i] / den) : 0.0f;
    }
    __syncthreads();
    // ---- r = sigmoid(o~) dh / den, and do~ (own columns)
    for (int e = tid; e < L * TV; e += NTB) {
      const int i = e / TV, bb = e % TV;
      const int64_t gi = (tok0 + i) * dv + cb * TV + bb;
      const float dh = ld<T>(a.dh, gi);
      float gate = 1.0f;
      if (a.o_pre) {
        gate = mk::sigmoid_fast(ld<TO>(a.o_pre, gi));
        a.d_o[gi] = dh * ld<T>(a.h, gi) * (1.0f - gate);
      }
      sR[i * TP + bb] = gate * dh / sDen[i];
    }
    __syncthreads();
    // ---- W = D (.) (r.v + dnq)
    for (int e = tid; e < L * L; e += NTB) {
      const int i = e / L, j = e % L;
      const float rv = (lead ? sDnq[i] : 0.0f) + dot4(sR + i * TP, 1, sV + j * TP, 1, TV);
      sW[i * LP + j] = sDm[i * LP + j] * rv;
    }
    __syncthreads();
    // (D (.) S replaces S: only dv reads it from here on)
    for (int e = tid; e < L * L; e += NTB) sS[(e / L) * LP + e % L] *= sDm[(e / L) * LP + e % L];
    // r scaled by g, for the state gradient
    for (int e = tid; e < L * TV; e += NTB) sRg[(e / TV) * TP + e % TV] = G.g[e / TV] * sR[(e / TV) * TP + e % TV];
    __syncthreads();
    // ---- dq partial: sum_j W_ij k_j + g_i (C~_s r_i + dnq_i n~_s)
    {
      float* out = a.ws_dq + ((static_cast<int64_t>(cb) * a.B * a.H + bh) * nT + static_cast<int64_t>(c) * L) * dqk;
      for (int e = tid; e < L * dqk; e += NTB) {
        const int i = e / dqk, x = e % dqk;
        const float s = dot4(sW + i * LP, 1, sKt + x, QP, i + 1);
        const float cr = (lead ? sDnq[i] * sN[x] : 0.0f) + dot4(sX + x * TP, 1, sR + i * TP, 1, TV);
        out[e] = s + G.g[i] * cr;
      }
    }
    __syncthreads();
    // ---- the carried gradient dC_e into LDS (replaces C~_s)
    for (int r = 0; r < ne; ++r) sX[(r0 + RSTEP * r) * TP + b] = dC[r];
    __syncthreads();
    // ---- dk partial: sum_i W_ij q_i + w_j (dC_e v_j + dn_e)
    {
      float* out = a.ws_dk + ((static_cast<int64_t>(cb) * a.B * a.H + bh) * nT + static_cast<int64_t>(c) * L) * dqk;
      for (int e = tid; e < L * dqk; e += NTB) {
        const int j = e / dqk, x = e % dqk;
        const float s = dot4(sW + j * LP + j, LP, sQ + j * QP + x, QP, L - j);
        const float cv = (lead ? sDn[x] : 0.0f) + dot4(sX + x * TP, 1, sV + j * TP, 1, TV);
        out[e] = s + G.w[j] * cv;
      }
    }
    // ---- dv: sum_i D_ij (q_i.k_j) r_i + w_j dC_e^T k_j (own columns)
    for (int e = tid; e < L * TV; e += NTB) {
      const int j = e / TV, bb = e % TV;
      const float s = dot4(sS + j * LP + j, LP, sR + j * TP + bb, TP, L - j);   // sS holds D (.) S
      const float ck = dot4(sX + bb, TP, sKt + j * QP, 1, dqk);
      a.d_v[(tok0 + j) * dv + cb * TV + bb] = s + G.w[j] * ck;
    }
    // ---- dC_s = g_L dC_e + sum_i g_i q_i r_i^T (this thread's entries)
    const float gL = G.g[L - 1];
    for (int r = 0; r < ne; ++r) {
      const int row = r0 + RSTEP * r;
      dC[r] = gL * dC[r] + dot4(sQ + row, QP, sRg + b, TP, L);
    }
    __syncthreads();   // every read of sDn (dk) is done
    // ---- dn_s = g_L dn_e + sum_i g_i dnq_i q_i
    for (int x = tid; x < dqk; x += NTB) {
      float s = gL * sDn[x];
#pragma unroll 8
      for (int i = 0; i < L; ++i) s += G.g[i] * sDnq[i] * sQ[i * QP + x];
      sDn[x] = s;
    }
  }
  // ---- initial state: gradients in its stored scale, and dm0's share
  __syncthreads();
  float part = 0.0f;
  for (int r = 0; r < ne; ++r) {
    const int row = r0 + RSTEP * r;
    const int64_t gi = (bh * dqk + row) * dv + cb * TV + b;
    if (a.dC0) a.dC0[gi] = dC[r];
    if (a.C0) part += dC[r] * a.C0[gi];
  }
  if (lead) {
    for (int x = tid; x < dqk; x += NTB) {
      if (a.dn0) a.dn0[bh * dqk + x] = sDn[x];
      if (a.C0) part += sDn[x] * a.n0[bh * dqk + x];
    }
  }
  part = block_sum(part, sRed);
  if (tid == 0) a.ws_dm0[static_cast<int64_t>(cb) * a.B * a.H + bh] = part;
}

// ---- pass 4: per token, the partial sums of dq and dk, di~ and q.dq - k.dk
// (one wave per token, 4 consecutive d_qk entries per lane per step: 16-byte
// partial loads; d_qk is a multiple of 16)
template <typename T>
__device__ __forceinline__ void load4f(const void* p, int64_t i, float* x) {
  if (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p) + i);
    x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
}

template <typename T>
__global__ __launch_bounds__(NTB) void bwd_tok_kernel(BwdArgs a, int ncb) {
  const int64_t ntok = a.B * a.H * a.T;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * (NTB / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= ntok) return;
  const int64_t dqk = a.dqk;
  float kdk = 0.0f, qdq = 0.0f;
  for (int64_t x = 4 * lane; x < dqk; x += 256) {
    float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
    for (int p = 0; p < ncb; ++p) {
      const int64_t o = (static_cast<int64_t>(p) * ntok + tok) * dqk + x;
      const float4 vq = *reinterpret_cast<const float4*>(a.ws_dq + o);
      const float4 vk = *reinterpret_cast<const float4*>(a.ws_dk + o);
      sq.x += vq.x; sq.y += vq.y; sq.z += vq.z; sq.w += vq.w;
      sk.x += vk.x; sk.y += vk.y; sk.z += vk.z; sk.w += vk.w;
    }
    *reinterpret_cast<float4*>(a.d_q + tok * dqk + x) = sq;
    *reinterpret_cast<float4*>(a.d_k + tok * dqk + x) = sk;
    float qv[4], kv[4];
    load4f<T>(a.q, tok * dqk + x, qv);
    load4f<T>(a.k, tok * dqk + x, kv);
    qdq += (qv[0] * sq.x + qv[1] * sq.y) + (qv[2] * sq.z + qv[3] * sq.w);
    kdk += (kv[0] * sk.x + kv[1] * sk.y) + (kv[2] * sk.z + kv[3] * sk.w);
  }
  qdq = wave_sum(qdq);
  kdk = wave_sum(kdk);
  if (lane == 0) {
    a.d_i[tok] = kdk;
    a.ws_s[tok] = qdq - kdk;
  }
}

// ---- pass 5: per head, d(log f_t) = sum_{t'>=t} s_t' + <dC1, C~_T> + <dn1, n~_T>
// (a reverse prefix sum, one block scan per tile of NTB tokens), df~ and dm0
// (chunk 16/32; chunk 64 has its own pass in bwd_mfma.hip).
__global__ __launch_bounds__(NTB) void bwd_head_kernel(BwdArgs a, int ncb, int nc) {
  __shared__ float sRed[NTB / 64];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t T = a.T, dqk = a.dqk, dv = a.dv;
  const int64_t nb = nc + 1;
  // constant term from the final-state gradient
  float kend = 0.0f;
  if (a.dC1) {
    const float* CT = a.ws_CT ? a.ws_CT + bh * dqk * dv : a.ws_C + (bh * nb + nc) * dqk * dv;
    const float* G1 = a.dC1 + bh * dqk * dv;
    float k4[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // independent sums: loads overlap
    int64_t e = tid;
    for (; e + 3 * NTB < dqk * dv; e += 4 * NTB) {
#pragma unroll
      for (int u = 0; u < 4; ++u) k4[u] += G1[e + u * NTB] * CT[e + u * NTB];
    }
    for (; e < dqk * dv; e += NTB) k4[0] += G1[e] * CT[e];
    kend += (k4[0] + k4[1]) + (k4[2] + k4[3]);
    for (int64_t e = tid; e < dqk; e += NTB) kend += a.dn1[bh * dqk + e] * a.ws_n[(bh * nb + nc) * dqk + e];
  }
  kend = block_sum(kend, sRed);
  // reverse prefix sum over tiles of NTB tokens, last tile first: thread
  // tid takes token tile * NTB + NTB - 1 - tid, so an inclusive prefix sum
  // over the threads is the sum over the tokens after it in the tile
  // (coalesced loads, one block scan per tile)
  const int lane = tid & 63, wave = tid >> 6;
  float carry = kend;   // sum over the tiles after this one, plus the constant term
  __syncthreads();      // every read of sRed by block_sum is done
  const int64_t ntile = (T + NTB - 1) / NTB;
  auto s_at = [&](int64_t t) { return a.ws_s[bh * T + t]; };
  float sv_n, fp_n;   // the next tile's inputs, loaded one tile ahead
  {
    const int64_t t = (ntile - 1) * NTB + (NTB - 1 - tid);
    sv_n = t < T ? s_at(t) : 0.0f;
    fp_n = t < T ? a.f_pre[bh * T + t] : 0.0f;
  }
  for (int64_t tile = ntile - 1; tile >= 0; --tile) {
    const int64_t t = tile * NTB + (NTB - 1 - tid);
    const float sv = sv_n, fpre = fp_n;
    if (tile > 0) {
      sv_n = s_at(t - NTB);
      fp_n = a.f_pre[bh * T + t - NTB];
    }
    const float incl = mk::scan_add(sv);
    if (lane == 63) sRed[wave] = incl;
    __syncthreads();
    float before = 0.0f, total = 0.0f;
#pragma unroll
    for (int w = 0; w < NTB / 64; ++w) {
      before += w < wave ? sRed[w] : 0.0f;
      total += sRed[w];
    }
    __syncthreads();   // sRed is rewritten by the next tile
    if (t < T) {
      const float after = carry + before + incl;
      a.d_f[bh * T + t] = a.fgate_exp ? after : after * (1.0f - mk::sigmoid_fast(fpre));
    }
    carry += total;
  }
  if (a.dm0 && tid == 0) {
    float s = 0.0f;
    for (int p = 0; p < ncb; ++p) s += a.ws_dm0[static_cast<int64_t>(p) * a.B * a.H + bh];
    a.dm0[bh] = s;
  }
}

template <typename T, typename TO, int TV, int L>
hipError_t launch_typed(const BwdArgs& a, hipStream_t st) {
  const int64_t ntok = a.B * a.H * a.T;
  const int ncb = static_cast<int>(a.dv / TV);
  const int nc = static_cast<int>(a.T / L);
  const unsigned tok_blocks = static_cast<unsigned>((ntok + NTB / 64 - 1) / (NTB / 64));
  const unsigned wgs = static_cast<unsigned>(a.B * a.H * ncb);
  bwd_beta_kernel<T><<<(tok_blocks + 1) / 2, NTB, 0, st>>>(a);
  bwd_states_kernel<T, TV, L><<<wgs, NTB, 0, st>>>(a);
  bwd_rev_kernel<T, TO, TV, L><<<wgs, NTB, 0, st>>>(a);
  bwd_tok_kernel<T><<<tok_blocks, NTB, 0, st>>>(a, ncb);
  bwd_head_kernel<<<static_cast<unsigned>(a.B * a.H), NTB, 0, st>>>(a, ncb, nc);
  return hipGetLastError();
}

// Chunk 64 (bf16 q, k, v): the state, reverse and dq/dk passes on MFMA and
// the per-chunk gate pass (bwd_mfma.hip).  beta (a bandwidth-bound pass over
// dh and h) is needed first by the reverse pass, not by the state pass, which
// is latency-bound and leaves room on every CU: beta runs on a side stream of
// the library's own, forked from the caller's stream after everything already
// queued there and joined back before the reverse pass (two events; the same
// fork and join when the caller's stream is being captured into a graph).
constexpr int kSideDevices = 64;
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;   // one fork / join sequence at a time per process
SideStream g_side[kSideDevices];

hipError_t side_stream(hipStream_t st, SideStream** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (st) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return e;
    dev = sdev;
  }
  if (dev < 0 || dev >= kSideDevices) return hipErrorInvalidDevice;
  SideStream& s = g_side[dev];
  if (!s.st) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    hipStream_t ns = nullptr;
    hipEvent_t ef = nullptr, ej = nullptr;
    e = hipStreamCreateWithFlags(&ns, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ef, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ej, hipEventDisableTiming);
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    s.st = ns;
    s.fork = ef;
    s.join = ej;
  }
  *out = &s;
  return hipSuccess;
}

template <typename T>
hipError_t launch_mfma(const BwdArgs& a, hipStream_t st) {
  const int64_t ntok = a.B * a.H * a.T;
  const unsigned tok_blocks = static_cast<unsigned>((ntok + NTB / 64 - 1) / (NTB / 64));
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  hipError_t e = side_stream(st, &side);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(side->fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(side->st, side->fork, 0)) != hipSuccess) return e;
  bwd_beta_kernel<T><<<(tok_blocks + 1) / 2, NTB, 0, side->st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipEventRecord(side->join, side->st)) != hipSuccess) return e;
  e = launch_bwd_states_mfma(a, st);
  if (e != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(st, side->join, 0)) != hipSuccess) return e;
  e = launch_bwd_rev_mfma(a, st);
  if (e != hipSuccess) return e;
  e = launch_bwd_qk_mfma(a, st);
  if (e != hipSuccess) return e;
  return launch_bwd_gates_mfma(a, st);
}

template <typename T, typename TO>
hipError_t launch_dt(const BwdArgs& a, hipStream_t st) {
  if (a.L == 64) return launch_mfma<T>(a, st);
  const int TV = bwd_tile_columns(a);
  if (a.L == 16) return TV == 32 ? launch_typed<T, TO, 32, 16>(a, st) : launch_typed<T, TO, 16, 16>(a, st);
  return TV == 32 ? launch_typed<T, TO, 32, 32>(a, st) : launch_typed<T, TO, 16, 32>(a, st);
}

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int bwd_tile_columns(const BwdArgs& a) {
  if (a.L == 64) return 64;
  return a.dv % 32 == 0 ? 32 : 16;
}

bool bwd_supported(const BwdArgs& a) {
  if (a.L == 64) return bwd_mfma_supported(a);
  const int TV = a.dv % 32 == 0 ? 32 : 16;
  return (a.L == 16 || a.L == 32) && a.T % a.L == 0 && a.dqk <= 256 && a.dqk % (NTB / TV) == 0 &&
         a.dv % 16 == 0;
}

// Workspace layout, in order: the boundary states, ws_n, ws_m, ws_beta, then
// chunk 16/32: ws_dq, ws_dk (per-column-block partials), ws_s, ws_dm0;
// chunk 64: ws_dCb, ws_R, ws_qd, ws_kd, ws_dm0, ws_dnq, ws_dn, ws_csum, ws_kend.
size_t bwd_workspace(const BwdArgs& a, size_t offsets[16]) {
  const size_t BH = static_cast<size_t>(a.B * a.H), T = static_cast<size_t>(a.T);
  const size_t nb = static_cast<size_t>(a.T / a.L) + 1, dqk = static_cast<size_t>(a.dqk);
  const size_t dv = static_cast<size_t>(a.dv);
  const size_t ncb = dv / static_cast<size_t>(bwd_tile_columns(a));
  const size_t nc = nb - 1;
  size_t sizes[16] = {0};
  size_t n = 0;
  if (a.L == 64) {
    // the boundary states the reverse pass reads as bf16 tiles, and the
    // final state (for the forget-gate term) in float32 after them
    const size_t nspl = static_cast<size_t>(bwd_qk_slices(a));
    const size_t tiles = BH * nc * dqk * dv * 2;
    const size_t s64[13] = {round_up(tiles) + BH * dqk * dv * 4, BH * nb * dqk * 4, BH * nb * 4, BH * T * 4,
                            tiles, BH * T * dv * 2, nspl * BH * T * 4, nspl * BH * T * 4, ncb * BH * 4,
                            BH * T * 4, BH * nc * dqk * 4, nspl * BH * nc * 2 * 4, ncb * BH * 4};
    n = 13;
    for (size_t i = 0; i < n; ++i) sizes[i] = s64[i];
  } else {
    const size_t s16[8] = {BH * nb * dqk * dv * 4, BH * nb * dqk * 4, BH * nb * 4, BH * T * 4,
                           ncb * BH * T * dqk * 4, ncb * BH * T * dqk * 4, BH * T * 4, ncb * BH * 4};
    n = 8;
    for (size_t i = 0; i < n; ++i) sizes[i] = s16[i];
  }
  size_t off = 0;
  for (size_t i = 0; i < 16; ++i) {
    if (offsets) offsets[i] = off;
    off += round_up(sizes[i]);
  }
  return off;
}

hipError_t launch_bwd(BwdArgs a, void* ws, hipStream_t st) {
  size_t off[16];
  bwd_workspace(a, off);
  char* base = static_cast<char*>(ws);
  a.ws_n = reinterpret_cast<float*>(base + off[1]);
  a.ws_m = reinterpret_cast<float*>(base + off[2]);
  a.ws_beta = reinterpret_cast<float*>(base + off[3]);
  a.ws_dCb = a.ws_R = nullptr;
  a.ws_dnq = a.ws_dn = a.ws_qd = a.ws_kd = a.ws_csum = a.ws_kend = nullptr;
  if (a.L == 64) {
    const size_t tiles = static_cast<size_t>(a.B * a.H) * static_cast<size_t>(a.T / 64) *
                         static_cast<size_t>(a.dqk * a.dv) * 2;
    a.ws_C = nullptr;
    a.ws_Cb = reinterpret_cast<uint16_t*>(base + off[0]);
    a.ws_CT = reinterpret_cast<float*>(base + off[0] + round_up(tiles));
    a.ws_dCb = reinterpret_cast<uint16_t*>(base + off[4]);
    a.ws_R = reinterpret_cast<uint16_t*>(base + off[5]);
    a.ws_qd = reinterpret_cast<float*>(base + off[6]);
    a.ws_kd = reinterpret_cast<float*>(base + off[7]);
    a.ws_dm0 = reinterpret_cast<float*>(base + off[8]);
    a.ws_dnq = reinterpret_cast<float*>(base + off[9]);
    a.ws_dn = reinterpret_cast<float*>(base + off[10]);
    a.ws_csum = reinterpret_cast<float*>(base + off[11]);
    a.ws_kend = reinterpret_cast<float*>(base + off[12]);
    a.ws_dq = a.ws_dk = a.ws_s = nullptr;
  } else {
    a.ws_C = reinterpret_cast<float*>(base + off[0]);
    a.ws_Cb = nullptr;
    a.ws_CT = nullptr;
    a.ws_dq = reinterpret_cast<float*>(base + off[4]);
    a.ws_dk = reinterpret_cast<float*>(base + off[5]);
    a.ws_s = reinterpret_cast<float*>(base + off[6]);
    a.ws_dm0 = reinterpret_cast<float*>(base + off[7]);
  }
  if (a.qkv_bf16) {
    if (a.o_mode == O_BF16) return launch_dt<bf16_t, bf16_t>(a, st);
    return launch_dt<bf16_t, float>(a, st);
  }
  if (a.o_mode == O_BF16) return launch_dt<float, bf16_t>(a, st);
  return launch_dt<float, float>(a, st);
}

namespace {
__global__ __launch_bounds__(NTB) void fill_words_kernel(uint32_t* base, int64_t rows, int64_t pitch,
                                                         int64_t off, int64_t count, uint32_t value) {
  const int64_t n = rows * count;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(NTB) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * NTB) {
    const int64_t r = e / count, c = e % count;
    base[r * pitch + off + c] = value;
  }
}
}  // namespace

namespace {
// Backward of an empty sequence (T = 0), one workgroup per head: the memory
// gradients pass through (dC0 = dC1, dn0 = dn1; zeros without them) and
// dm0 = <dC1, C~0> + <dn1, n~0> (zero without an initial state).
__global__ __launch_bounds__(NTB) void bwd_empty_kernel(BwdArgs a) {
  __shared__ float sRed[NTB / 64];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x, S = a.dqk * a.dv;
  float acc = 0.0f;
  for (int64_t e = tid; e < S; e += NTB) {
    const float gC = a.dC1 ? a.dC1[bh * S + e] : 0.0f;
    if (a.dC0) a.dC0[bh * S + e] = gC;
    if (a.C0) acc += gC * a.C0[bh * S + e];
  }
  for (int64_t e = tid; e < a.dqk; e += NTB) {
    const float gn = a.dn1 ? a.dn1[bh * a.dqk + e] : 0.0f;
    if (a.dn0) a.dn0[bh * a.dqk + e] = gn;
    if (a.C0) acc += gn * a.n0[bh * a.dqk + e];
  }
  acc = block_sum(acc, sRed);
  if (tid == 0 && a.dm0) a.dm0[bh] = acc;
}
}  // namespace

hipError_t launch_bwd_empty(const BwdArgs& a, hipStream_t st) {
  const int64_t BH = a.B * a.H;
  if (BH <= 0) return hipSuccess;
  bwd_empty_kernel<<<static_cast<unsigned>(BH), NTB, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fill_words(uint32_t* base, int64_t rows, int64_t pitch, int64_t off, int64_t count,
                             uint32_t value, hipStream_t st) {
  const int64_t n = rows * count;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + NTB - 1) / NTB;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  fill_words_kernel<<<grid, NTB, 0, st>>>(base, rows, pitch, off, count, value);
  return hipGetLastError();
}

}  // namespace mlstm
