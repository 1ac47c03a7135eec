// Decode step of the mLSTM cell: one token for every (batch, head).
//
// Method: xLSTM post (llms.blog), section 3 "Associative Matrix Cell State"
// (C_t = f_t C_{t-1} + i_t v_t k_t^T, n_t = f_t n_{t-1} + i_t k_t, retrieval
// C_t q_t / max(|n_t . q_t|, 1), h = o (.) h~) with the running maximum of
// section 2 "The Normalizer State and Numerical Stabilization".  Section 5
// ("Inference Memory and Throughput Trade-Offs") is why this is its own
// kernel: the state has a fixed size, so one step streams C~ from HBM once
// and writes it back once.  Arithmetic intensity is ~0.6 flop/byte: the
// kernel is bound by HBM bandwidth, and it is written for that (16-byte
// vector accesses, every byte of C~ touched exactly once, many independent
// loads in flight per thread, no MFMA).
//
// Per head, with L = 1 the stabilized update is
//   M   = max(m_in, i~ - log f)      m_out = log f + M  (= max(log f + m_in, i~))
//   g   = exp(m_in - M)              (the stabilized forget factor)
//   w   = exp(i~ - log f - M)        (the stabilized input factor)
//   C~' = g C~ + w k v^T,  n~' = g n~ + w k,  h = sigmoid(o~) (.) q^T C~' / max(|n~'.q|, e^{-m_out})
//
// Launch 1 (step_stream_kernel): grid (B*H, column blocks).  A workgroup owns a
// block of d_v columns of one head's C~ for all d_qk rows, so the readout
// q^T C~' over rows finishes inside the workgroup (no cross-workgroup sum),
// and it writes exactly the C~ columns it read (safe in place).  It reads n~
// and m but does not write them: other workgroups of the head still read them.
// Launch 2 (step_state_kernel): writes n~' and m_out after launch 1 is done,
// each element by the thread that read it (safe in place).
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

struct StepScalars {
  float g, w, m_new;
};

__device__ __forceinline__ StepScalars step_scalars(float i_pre, float f_pre, float m_in,
                                                    int fgate_exp) {
  float lf = log_forget(f_pre, fgate_exp);
  float u = i_pre - lf;
  float M = fmaxf(m_in, u);
  StepScalars s;
  s.g = __expf(m_in - M);
  s.w = __expf(u - M);
  s.m_new = lf + M;
  return s;
}

template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  uint2 u;
  u.x = pack_bf2(v.x, v.y);
  u.y = pack_bf2(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = u;
}

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// C~ is touched exactly once per step: stream it past the caches.
__device__ __forceinline__ float4 ld_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream(float* p, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

// CT column threads (4 floats each) x (256 / CT) row groups.  Dynamic LDS:
// w k and q as float32 for all d_qk rows (2 d_qk floats).
template <typename TQ, int OM, int CT>
__global__ __launch_bounds__(kThreads) void step_stream_kernel(StepArgs a) {
  constexpr int R = kThreads / CT;   // row groups
  constexpr int CB = 4 * CT;         // columns per workgroup
  __shared__ float s_red[R][CB];
  __shared__ float s_qn[kThreads / 64];
  extern __shared__ float s_dyn[];   // [0, dqk): w k_r, [dqk, 2 dqk): q_r

  const int tid = threadIdx.x;
  const int ct = tid % CT;
  const int rg = tid / CT;
  const int64_t bh = blockIdx.x;
  const int dqk = static_cast<int>(a.dqk);
  const int dv = static_cast<int>(a.dv);
  const int col = blockIdx.y * CB + 4 * ct;
  const bool col_ok = col < dv;
  float* s_kw = s_dyn;
  float* s_q = s_dyn + dqk;

  const TQ* q = static_cast<const TQ*>(a.q) + bh * dqk;
  const TQ* k = static_cast<const TQ*>(a.k) + bh * dqk;
  const TQ* v = static_cast<const TQ*>(a.v) + bh * dv;
  const float* n_in = a.n_in + bh * dqk;
  const float* Cin = a.C_in + bh * static_cast<int64_t>(dqk) * dv + col;
  float* Cout = a.C_out + bh * static_cast<int64_t>(dqk) * dv + col;
  const StepScalars sc = step_scalars(a.i_pre[bh], a.f_pre[bh], a.m_in[bh], a.fgate_exp);

  // the first batch of C~ rows is in flight while the row vectors are staged
  float4 c[kUnroll];
  const bool full_first = col_ok && (kUnroll - 1) * R + rg < dqk;
  if (full_first) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) c[u] = ld_stream(Cin + static_cast<int64_t>(rg + u * R) * dv);
  }

  // w k and q into LDS; n~' . q over all rows (every workgroup of the head
  // needs it)
  float qn = 0.0f;
  for (int r = tid; r < dqk; r += kThreads) {
    const float kw = sc.w * to_f32(k[r]);
    const float qr = to_f32(q[r]);
    s_kw[r] = kw;
    s_q[r] = qr;
    qn += (sc.g * n_in[r] + kw) * qr;
  }
  qn = wave_sum(qn);
  if ((tid & 63) == 0) s_qn[tid >> 6] = qn;
  __syncthreads();

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col_ok) {
    const float4 v4 = load4<TQ>(v + col);
    auto update = [&](int r, float4 cv) {
      const float kw = s_kw[r];
      const float qr = s_q[r];
      float4 cn;
      cn.x = sc.g * cv.x + kw * v4.x;
      cn.y = sc.g * cv.y + kw * v4.y;
      cn.z = sc.g * cv.z + kw * v4.z;
      cn.w = sc.g * cv.w + kw * v4.w;
      st_stream(Cout + static_cast<int64_t>(r) * dv, cn);
      acc.x += qr * cn.x;
      acc.y += qr * cn.y;
      acc.z += qr * cn.z;
      acc.w += qr * cn.w;
    };
    int r0 = rg;
    if (full_first) {
      // steady state: kUnroll independent 16-byte loads in flight per thread
      for (;;) {
        const int rn = r0 + kUnroll * R;
        const bool more = rn + (kUnroll - 1) * R < dqk;
        float4 cnext[kUnroll];
        if (more) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) cnext[u] = ld_stream(Cin + static_cast<int64_t>(rn + u * R) * dv);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) update(r0 + u * R, c[u]);
        r0 = rn;
        if (!more) break;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) c[u] = cnext[u];
      }
    }
    for (; r0 < dqk; r0 += R) update(r0, ld_stream(Cin + static_cast<int64_t>(r0) * dv));
  }
  s_red[rg][4 * ct + 0] = acc.x;
  s_red[rg][4 * ct + 1] = acc.y;
  s_red[rg][4 * ct + 2] = acc.z;
  s_red[rg][4 * ct + 3] = acc.w;
  __syncthreads();

  // Column sums over the R row groups; thread t < CB finishes column t.
  if (tid < CB) {
    const int cc = blockIdx.y * CB + tid;
    if (cc < dv) {
      float num = 0.0f;
#pragma unroll 8
      for (int r = 0; r < R; ++r) num += s_red[r][tid];
      float qn_all = 0.0f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) qn_all += s_qn[w];
      const float den = fmaxf(fabsf(qn_all), __expf(-sc.m_new));
      float gate = 1.0f;
      if (OM == O_F32) gate = sigmoidf_(static_cast<const float*>(a.o_pre)[bh * dv + cc]);
      if (OM == O_BF16) gate = sigmoidf_(bf2f(static_cast<const bf16_t*>(a.o_pre)[bh * dv + cc]));
      static_cast<TQ*>(a.h)[bh * dv + cc] = from_f32<TQ>(gate * num / den);
    }
  }
}

// In place (m_out == m_in, n_out == n_in): every thread reads m_in at entry,
// and each n~ element is read and written by the same thread.  m_out is
// written only after the barrier, when every wave of the workgroup has read
// m_in; without it a late wave could read the new m and scale its n~ rows
// with the wrong factors.
template <typename TQ>
__global__ __launch_bounds__(kThreads) void step_state_kernel(StepArgs a) {
  const int64_t bh = blockIdx.x;
  const int dqk = static_cast<int>(a.dqk);
  const StepScalars sc = step_scalars(a.i_pre[bh], a.f_pre[bh], a.m_in[bh], a.fgate_exp);
  const TQ* k = static_cast<const TQ*>(a.k) + bh * dqk;
  for (int r = threadIdx.x; r < dqk; r += kThreads)
    a.n_out[bh * dqk + r] = sc.g * a.n_in[bh * dqk + r] + sc.w * to_f32(k[r]);
  __syncthreads();
  if (threadIdx.x == 0) a.m_out[bh] = sc.m_new;
}

template <typename TQ, int OM>
hipError_t launch_typed(const StepArgs& a, hipStream_t stream) {
  const int64_t BH = a.B * a.H;
  const int ctmax = static_cast<int>(a.dv / 4);
  int ct = 32;
  while (ct > ctmax) ct >>= 1;
  const int cb = 4 * ct;
  dim3 grid(static_cast<unsigned>(BH), static_cast<unsigned>((a.dv + cb - 1) / cb));
  const size_t lds = 2 * static_cast<size_t>(a.dqk) * sizeof(float);
  switch (ct) {
    case 32: step_stream_kernel<TQ, OM, 32><<<grid, kThreads, lds, stream>>>(a); break;
    case 16: step_stream_kernel<TQ, OM, 16><<<grid, kThreads, lds, stream>>>(a); break;
    case 8: step_stream_kernel<TQ, OM, 8><<<grid, kThreads, lds, stream>>>(a); break;
    default: step_stream_kernel<TQ, OM, 4><<<grid, kThreads, lds, stream>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  step_state_kernel<TQ><<<dim3(static_cast<unsigned>(BH)), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename TQ>
hipError_t launch_o(const StepArgs& a, hipStream_t stream) {
  switch (a.o_mode) {
    case O_F32: return launch_typed<TQ, O_F32>(a, stream);
    case O_BF16: return launch_typed<TQ, O_BF16>(a, stream);
    default: return launch_typed<TQ, O_NONE>(a, stream);
  }
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  return a.qkv_bf16 ? launch_o<bf16_t>(a, stream) : launch_o<float>(a, stream);
}

}  // namespace mlstm
