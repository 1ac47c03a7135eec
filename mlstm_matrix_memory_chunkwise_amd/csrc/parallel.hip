// Parallel (quadratic) form of the mLSTM forward pass.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form": with the
// causal decay matrix S_ij = (prod_{tau=j+1..i} f_tau) i_j (i >= j), the hidden
// states of the whole sequence are H = ((Q K^T) (.) S) V, normalized as in
// "Associative Matrix Cell State".  Stabilized with the closed form of the
// running maximum (section 2, "The Normalizer State and Numerical
// Stabilization", unrolled):
//   F_i = sum_{t<=i} log f_t,  u_j = i~_j - F_j,  M_i = max(m_0, max_{j<=i} u_j),
//   m_i = F_i + M_i,  D_ij = exp(u_j - M_i),  g_i = exp(m_0 - M_i),
//   num_i = g_i q_i^T C~_0 + sum_{j<=i} D_ij (q_i . k_j) v_j
//   den_i = max(|g_i q_i . n~_0 + sum_{j<=i} D_ij (q_i . k_j)|, exp(-m_i))
//   C~_T = g_T C~_0 + sum_j D_Tj k_j v_j^T,  n~_T = g_T n~_0 + sum_j D_Tj k_j.
// No chunking: one window of T tokens.  F, u, M, m are scanned in float64
// (T can be long and exponents are differences of large sums).
//
// Launches: (1) one wave per head scans the gates into the workspace;
// (2) outputs, one workgroup per (head, 64-query block, 16 value columns);
// (3) final state, one thread per state element.
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

constexpr int kThreads = 256;
constexpr int kQB = 64;   // queries per workgroup
constexpr int kJB = 64;   // keys per step
constexpr int kTV = 16;   // value columns per workgroup

// workspace per head: u[T], M[T], m[T] (float64)
__global__ __launch_bounds__(64) void par_scan_kernel(SeqArgs a, double* ws) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t T = a.T;
  const float* ip = a.i_pre + bh * T;
  const float* fp = a.f_pre + bh * T;
  double* U = ws + bh * 3 * T;
  double* Mx = U + T;
  double* Mm = Mx + T;
  const double m0 = a.C0 ? static_cast<double>(a.m0[bh]) : 0.0;
  const int64_t seg = (T + 63) / 64;
  const int64_t t0 = lane * seg;
  const int64_t t1 = t0 + seg < T ? t0 + seg : T;

  // pass 1: segment sum of log f and segment max of (i~ - local cumsum)
  double fsum = 0.0, umax = -INFINITY;
  for (int64_t t = t0; t < t1; ++t) {
    fsum += static_cast<double>(log_forget(fp[t], a.fgate_exp));
    umax = fmax(umax, static_cast<double>(ip[t]) - fsum);
  }
  // exclusive scan over lanes of (fsum) and of (umax - Fprefix)
  double incl = fsum;
  for (int o = 1; o < 64; o <<= 1) {
    double y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const double fpre = incl - fsum;
  double segmax = umax - fpre;
  double mincl = segmax;
  for (int o = 1; o < 64; o <<= 1) {
    double y = __shfl_up(mincl, o, 64);
    if (lane >= o) mincl = fmax(mincl, y);
  }
  double mprev = __shfl_up(mincl, 1, 64);
  if (lane == 0) mprev = -INFINITY;
  // pass 2
  double F = fpre, M = fmax(m0, mprev);
  for (int64_t t = t0; t < t1; ++t) {
    F += static_cast<double>(log_forget(fp[t], a.fgate_exp));
    const double u = static_cast<double>(ip[t]) - F;
    M = fmax(M, u);
    U[t] = u;
    Mx[t] = M;
    Mm[t] = F + M;
  }
  if (t0 < T && t1 == T && a.m1) a.m1[bh] = static_cast<float>(F + M);
}

template <typename TQ, int OM>
__global__ __launch_bounds__(kThreads) void par_out_kernel(SeqArgs a, const double* ws) {
  __shared__ float sP[kQB][kJB + 1];
  __shared__ float sRs[kQB];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t T = a.T;
  const int dqk = static_cast<int>(a.dqk);
  const int dv = static_cast<int>(a.dv);
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kQB;
  const int b0 = blockIdx.z * kTV;
  const TQ* q = static_cast<const TQ*>(a.q) + bh * T * dqk;
  const TQ* k = static_cast<const TQ*>(a.k) + bh * T * dqk;
  const TQ* v = static_cast<const TQ*>(a.v) + bh * T * dv;
  const double* U = ws + bh * 3 * T;
  const double* Mx = U + T;
  const double* Mm = Mx + T;
  const double m0 = a.C0 ? static_cast<double>(a.m0[bh]) : 0.0;

  // each thread owns 4 (query, column) outputs: query ii = tid / 4 ... spread
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float rs_acc = 0.0f;
  if (tid < kQB) sRs[tid] = 0.0f;

  for (int64_t j0 = 0; j0 <= i0 && j0 < T; j0 += kJB) {
    __syncthreads();
    for (int idx = tid; idx < kQB * kJB; idx += kThreads) {
      const int ii = idx / kJB, jj = idx % kJB;
      const int64_t i = i0 + ii, j = j0 + jj;
      float p = 0.0f;
      if (i < T && j <= i) {
        const TQ* qi = q + i * dqk;
        const TQ* kj = k + j * dqk;
        float s = 0.0f;
        for (int r = 0; r < dqk; ++r) s += to_f32(qi[r]) * to_f32(kj[r]);
        p = s * static_cast<float>(exp(U[j] - Mx[i]));
      }
      sP[ii][jj] = p;
    }
    __syncthreads();
    if (tid < kQB) {
      float r = 0.0f;
      for (int jj = 0; jj < kJB; ++jj) r += sP[tid][jj];
      rs_acc += r;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * kThreads;      // 0 .. kQB*kTV-1
      const int ii = idx / kTV, cc = idx % kTV, c = b0 + cc;
      if (c < dv) {
        float s = 0.0f;
        for (int jj = 0; jj < kJB; ++jj) {
          const int64_t j = j0 + jj;
          if (j < T) s += sP[ii][jj] * to_f32(v[j * dv + c]);
        }
        acc[e] += s;
      }
    }
  }
  if (tid < kQB) sRs[tid] = rs_acc;
  __syncthreads();

#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + e * kThreads;
    const int ii = idx / kTV, cc = idx % kTV, c = b0 + cc;
    const int64_t i = i0 + ii;
    if (c >= dv || i >= T) continue;
    const TQ* qi = q + i * dqk;
    const float g = static_cast<float>(exp(m0 - Mx[i]));
    float inter = 0.0f, qn = 0.0f;
    if (a.C0) {
      const float* C0 = a.C0 + bh * static_cast<int64_t>(dqk) * dv;
      const float* n0 = a.n0 + bh * dqk;
      for (int r = 0; r < dqk; ++r) {
        const float qr = to_f32(qi[r]);
        inter += qr * C0[static_cast<int64_t>(r) * dv + c];
        qn += qr * n0[r];
      }
    }
    const float num = g * inter + acc[e];
    const float den = fmaxf(fabsf(g * qn + sRs[ii]), static_cast<float>(exp(-Mm[i])));
    float gate = 1.0f;
    const int64_t oi = (bh * T + i) * dv + c;
    if (OM == O_F32) gate = sigmoidf_(static_cast<const float*>(a.o_pre)[oi]);
    if (OM == O_BF16) gate = sigmoidf_(bf2f(static_cast<const bf16_t*>(a.o_pre)[oi]));
    static_cast<TQ*>(a.h)[(bh * T + i) * dv + c] = from_f32<TQ>(gate * num / den);
  }
}

template <typename TQ>
__global__ __launch_bounds__(kThreads) void par_state_kernel(SeqArgs a, const double* ws) {
  const int64_t bh = blockIdx.x;
  const int64_t T = a.T;
  const int dqk = static_cast<int>(a.dqk);
  const int dv = static_cast<int>(a.dv);
  const TQ* k = static_cast<const TQ*>(a.k) + bh * T * dqk;
  const TQ* v = static_cast<const TQ*>(a.v) + bh * T * dv;
  const double* U = ws + bh * 3 * T;
  const double* Mx = U + T;
  const double Ml = Mx[T - 1];
  const double m0 = a.C0 ? static_cast<double>(a.m0[bh]) : 0.0;
  const float gT = static_cast<float>(exp(m0 - Ml));
  const int64_t e = static_cast<int64_t>(blockIdx.y) * kThreads + threadIdx.x;
  if (e < static_cast<int64_t>(dqk) * dv) {
    const int r = static_cast<int>(e / dv), c = static_cast<int>(e % dv);
    float acc = a.C0 ? gT * a.C0[bh * static_cast<int64_t>(dqk) * dv + e] : 0.0f;
    for (int64_t j = 0; j < T; ++j)
      acc += static_cast<float>(exp(U[j] - Ml)) * to_f32(k[j * dqk + r]) * to_f32(v[j * dv + c]);
    a.C1[bh * static_cast<int64_t>(dqk) * dv + e] = acc;
  }
  if (blockIdx.y == 0) {
    for (int r = threadIdx.x; r < dqk; r += kThreads) {
      float acc = a.C0 ? gT * a.n0[bh * dqk + r] : 0.0f;
      for (int64_t j = 0; j < T; ++j) acc += static_cast<float>(exp(U[j] - Ml)) * to_f32(k[j * dqk + r]);
      a.n1[bh * dqk + r] = acc;
    }
  }
}

template <typename TQ, int OM>
hipError_t launch_typed(const SeqArgs& a, double* ws, hipStream_t stream) {
  const unsigned BH = static_cast<unsigned>(a.B * a.H);
  par_scan_kernel<<<BH, 64, 0, stream>>>(a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(BH, static_cast<unsigned>((a.T + kQB - 1) / kQB), static_cast<unsigned>((a.dv + kTV - 1) / kTV));
  par_out_kernel<TQ, OM><<<g2, kThreads, 0, stream>>>(a, ws);
  e = hipGetLastError();
  if (e != hipSuccess || !a.C1) return e;
  dim3 g3(BH, static_cast<unsigned>((a.dqk * a.dv + kThreads - 1) / kThreads));
  par_state_kernel<TQ><<<g3, kThreads, 0, stream>>>(a, ws);
  return hipGetLastError();
}

template <typename TQ>
hipError_t launch_o(const SeqArgs& a, double* ws, hipStream_t stream) {
  switch (a.o_mode) {
    case O_F32: return launch_typed<TQ, O_F32>(a, ws, stream);
    case O_BF16: return launch_typed<TQ, O_BF16>(a, ws, stream);
    default: return launch_typed<TQ, O_NONE>(a, ws, stream);
  }
}

}  // namespace

size_t parallel_workspace(const SeqArgs& a) {
  return sizeof(double) * 3 * static_cast<size_t>(a.B * a.H * a.T);
}

hipError_t launch_parallel(const SeqArgs& a, void* ws, hipStream_t stream) {
  double* w = static_cast<double*>(ws);
  return a.qkv_bf16 ? launch_o<bf16_t>(a, w, stream) : launch_o<float>(a, w, stream);
}

}  // namespace mlstm
