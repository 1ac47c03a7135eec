// Chunkwise mLSTM forward on the vector ALUs (float32 arithmetic throughout).
//
// Serves the float32 path (where bf16 matrix cores would not meet float32
// accuracy) and bf16 shapes the MFMA kernel does not cover.  It follows the
// same chunk algebra as the MFMA kernel, with no tiling tricks.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form" (the
// decay matrix S with S_ij = (prod of f after j up to i) i_j for i >= j and
// H = ((Q K^T) (.) S) V), applied to one chunk of L tokens at a time with the
// state carried between chunks ("Associative Matrix Cell State" updates), and
// the running maximum of section 2 "The Normalizer State and Numerical
// Stabilization".  For a chunk starting after token s with carried
// (C~_s, n~_s, m_s) and chunk-local cumulative log forget gates b_i:
//   u_j = i~_j - b_j,  M_i = max(m_s, max_{j<=i} u_j),  m_i = b_i + M_i
//   D_ij = exp(u_j - M_i) (j <= i),  g_i = exp(m_s - M_i),  w_j = exp(u_j - M_L)
//   num_i = g_i q_i^T C~_s + sum_j D_ij (q_i . k_j) v_j
//   den_i = max(|g_i q_i . n~_s + sum_j D_ij (q_i . k_j)|, exp(-m_i))
//   C~ <- g_L C~_s + sum_j w_j k_j v_j^T,  n~ <- g_L n~_s + sum_j w_j k_j
// m_i equals the sequential recurrence's running maximum exactly (in exact
// arithmetic), and every exponent is <= 0.
//
// Grid: (B*H, ceil(d_v / 16)); one workgroup walks all chunks of one head for
// 16 value columns; its C~ tile [d_qk][16] and n~ stay in LDS.  It processes
// tokens t0 .. T-1 of each head (heads Ts tokens apart); the last chunk may
// hold fewer than L tokens, which serves sequences whose length is not a
// multiple of the chunk.
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

constexpr int kThreads = 256;
constexpr int kTV = 16;

template <typename TQ, int OM>
__global__ __launch_bounds__(kThreads) void chunk_valu_kernel(SeqArgs a, int L) {
  extern __shared__ float smem[];
  const int dqk = static_cast<int>(a.dqk);
  const int dv = static_cast<int>(a.dv);
  const int T = static_cast<int>(a.T), t0 = static_cast<int>(a.t0);
  const int64_t Ts = a.Ts;
  float* sC = smem;                      // [dqk][kTV]
  float* sN = sC + dqk * kTV;            // [dqk]
  float* sP = sN + dqk;                  // [L][L]
  float* sLf = sP + L * L;               // [L] log f, then scratch
  float* sU = sLf + L;                   // [L]
  float* sM = sU + L;                    // [L]
  float* sG = sM + L;                    // [L]
  float* sW = sG + L;                    // [L]
  float* sEm = sW + L;                   // [L] exp(-m_i)
  float* sRs = sEm + L;                  // [L] row sums of D (.) QK^T
  float* sQn = sRs + L;                  // [L] q_i . n~_s
  float* sMs = sQn + L;                  // [1] carried m

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int b0 = blockIdx.y * kTV;
  const TQ* q = static_cast<const TQ*>(a.q) + bh * Ts * dqk;
  const TQ* k = static_cast<const TQ*>(a.k) + bh * Ts * dqk;
  const TQ* v = static_cast<const TQ*>(a.v) + bh * Ts * dv;
  const float* ip = a.i_pre + bh * Ts;
  const float* fp = a.f_pre + bh * Ts;
  TQ* h = static_cast<TQ*>(a.h) + bh * Ts * dv;

  for (int idx = tid; idx < dqk * kTV; idx += kThreads) {
    const int r = idx / kTV, c = b0 + idx % kTV;
    sC[idx] = (a.C0 && c < dv) ? a.C0[(bh * dqk + r) * dv + c] : 0.0f;
  }
  for (int r = tid; r < dqk; r += kThreads) sN[r] = a.C0 ? a.n0[bh * dqk + r] : 0.0f;
  if (tid == 0) sMs[0] = a.C0 ? a.m0[bh] : 0.0f;
  __syncthreads();

  for (int c0 = t0; c0 < T; c0 += L) {
    const int Lc = min(L, T - c0);   // tokens in this chunk
    const float ms = sMs[0];
    for (int j = tid; j < Lc; j += kThreads) sLf[j] = log_forget(fp[c0 + j], a.fgate_exp);
    __syncthreads();
    if (tid == 0) {
      float b = 0.0f, Mx = ms;
      for (int j = 0; j < Lc; ++j) {
        b += sLf[j];
        const float u = ip[c0 + j] - b;
        Mx = fmaxf(Mx, u);
        sU[j] = u;
        sM[j] = Mx;
        sLf[j] = b;  // now the cumulative sum b_j
      }
      sMs[0] = b + Mx;  // m at the chunk's last token
    }
    __syncthreads();
    for (int j = tid; j < Lc; j += kThreads) {
      sG[j] = expf(ms - sM[j]);
      sW[j] = expf(sU[j] - sM[Lc - 1]);
      sEm[j] = expf(-(sLf[j] + sM[j]));
    }
    // P_ij = (q_i . k_j) D_ij
    for (int idx = tid; idx < Lc * Lc; idx += kThreads) {
      const int i = idx / Lc, j = idx % Lc;
      float s = 0.0f;
      if (j <= i) {
        const TQ* qi = q + static_cast<int64_t>(c0 + i) * dqk;
        const TQ* kj = k + static_cast<int64_t>(c0 + j) * dqk;
        for (int r = 0; r < dqk; ++r) s += to_f32(qi[r]) * to_f32(kj[r]);
        s *= expf(sU[j] - sM[i]);
      }
      sP[i * L + j] = s;
    }
    __syncthreads();
    for (int i = tid; i < Lc; i += kThreads) {
      float rs = 0.0f;
      for (int j = 0; j <= i; ++j) rs += sP[i * L + j];
      sRs[i] = rs;
      const TQ* qi = q + static_cast<int64_t>(c0 + i) * dqk;
      float qn = 0.0f;
      for (int r = 0; r < dqk; ++r) qn += to_f32(qi[r]) * sN[r];
      sQn[i] = qn;
    }
    __syncthreads();
    for (int idx = tid; idx < Lc * kTV; idx += kThreads) {
      const int i = idx / kTV, cc = idx % kTV, c = b0 + cc;
      if (c >= dv) continue;
      const TQ* qi = q + static_cast<int64_t>(c0 + i) * dqk;
      float inter = 0.0f;
      for (int r = 0; r < dqk; ++r) inter += to_f32(qi[r]) * sC[r * kTV + cc];
      float intra = 0.0f;
      for (int j = 0; j <= i; ++j) intra += sP[i * L + j] * to_f32(v[static_cast<int64_t>(c0 + j) * dv + c]);
      const float num = sG[i] * inter + intra;
      const float den = fmaxf(fabsf(sG[i] * sQn[i] + sRs[i]), sEm[i]);
      float gate = 1.0f;
      const int64_t oi = (bh * Ts + c0 + i) * static_cast<int64_t>(dv) + c;
      if (OM == O_F32) gate = sigmoidf_(static_cast<const float*>(a.o_pre)[oi]);
      if (OM == O_BF16) gate = sigmoidf_(bf2f(static_cast<const bf16_t*>(a.o_pre)[oi]));
      h[static_cast<int64_t>(c0 + i) * dv + c] = from_f32<TQ>(gate * num / den);
    }
    __syncthreads();
    const float gL = sG[Lc - 1];
    for (int idx = tid; idx < dqk * kTV; idx += kThreads) {
      const int r = idx / kTV, cc = idx % kTV, c = b0 + cc;
      if (c >= dv) continue;
      float acc = gL * sC[idx];
      for (int j = 0; j < Lc; ++j)
        acc += sW[j] * to_f32(k[static_cast<int64_t>(c0 + j) * dqk + r]) *
               to_f32(v[static_cast<int64_t>(c0 + j) * dv + c]);
      sC[idx] = acc;
    }
    for (int r = tid; r < dqk; r += kThreads) {
      float acc = gL * sN[r];
      for (int j = 0; j < Lc; ++j) acc += sW[j] * to_f32(k[static_cast<int64_t>(c0 + j) * dqk + r]);
      sN[r] = acc;
    }
    __syncthreads();
  }

  if (a.C1) {
    for (int idx = tid; idx < dqk * kTV; idx += kThreads) {
      const int r = idx / kTV, c = b0 + idx % kTV;
      if (c < dv) a.C1[(bh * dqk + r) * dv + c] = sC[idx];
    }
    if (blockIdx.y == 0) {
      for (int r = tid; r < dqk; r += kThreads) a.n1[bh * dqk + r] = sN[r];
      if (tid == 0) a.m1[bh] = sMs[0];
    }
  }
}

template <typename TQ, int OM>
hipError_t launch_typed(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  const int L = static_cast<int>(chunk);
  const size_t lds = sizeof(float) * (static_cast<size_t>(a.dqk) * kTV + a.dqk +
                                      static_cast<size_t>(L) * L + 9 * L + 1);
  auto fn = chunk_valu_kernel<TQ, OM>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>((a.dv + kTV - 1) / kTV));
  fn<<<grid, kThreads, lds, stream>>>(a, L);
  return hipGetLastError();
}

template <typename TQ>
hipError_t launch_o(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  switch (a.o_mode) {
    case O_F32: return launch_typed<TQ, O_F32>(a, chunk, stream);
    case O_BF16: return launch_typed<TQ, O_BF16>(a, chunk, stream);
    default: return launch_typed<TQ, O_NONE>(a, chunk, stream);
  }
}

}  // namespace

hipError_t launch_chunk_valu(const SeqArgs& a, int64_t chunk, hipStream_t stream) {
  return a.qkv_bf16 ? launch_o<bf16_t>(a, chunk, stream) : launch_o<float>(a, chunk, stream);
}

}  // namespace mlstm
