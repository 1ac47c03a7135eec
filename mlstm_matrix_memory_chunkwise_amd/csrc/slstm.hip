// sLSTM forward cell (gfx950): scalar memory with exponential gating,
// normalizer and stabilizer, and head-wise recurrent mixing.
//
// Method: the xLSTM post (llms.blog), section 2 "sLSTM: Scalar Memory with
// Exponential Gating and Normalization".  Per step t, head hd, unit u:
//   pre_g = wx[t, g, u] + sum_v R[hd, g, u, v] h_{t-1}[v]     (g = i, f, z, o)
//   m_t = max(log f + m_{t-1}, i~),  f' = exp(log f + m_{t-1} - m_t),
//   i' = exp(i~ - m_t),  c_t = f' c + i' z,  n_t = f' n + i',
//   h_t = sigmoid(o~) c_t / n_t,
// with log f = f~ (exponential gate) or log sigmoid(f~).  The recurrence
// through h is strictly sequential, so one workgroup runs one (batch, head)
// sequence and the design minimizes the latency of a step:
//  * 4 DH threads: lane (u, q) holds, in registers, the quarter q of the four
//    recurrent rows of unit u (4 x DH/4 floats) and forms their partial dot
//    products with h_{t-1} read from LDS (broadcast float4 reads; the four
//    quarters are padded apart so that they sit in different banks);
//  * the four partials of a unit are summed within its lane quad with DPP
//    quad permutations (no LDS, no barrier); every lane of the quad then
//    holds the four full preactivations and updates c, n, m redundantly;
//  * h_t goes to a double-buffered LDS vector, so one barrier per step
//    separates the writes of step t from the reads of step t + 1;
//  * the input projections wx of the next 8 steps are loaded while the
//    current 8 run.
// Everything is float32; the recurrent h stays float32 (a bf16 output is a
// rounded copy).
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

constexpr int PF = 8;   // steps of wx loaded ahead

template <typename T>
__device__ __forceinline__ float ldx(const void* p, int64_t i) {
  return to_f32<T>(static_cast<const T*>(p)[i]);
}

// x + x of lane (l ^ 1) and of lane (l ^ 2) within each quad: the quad sum
__device__ __forceinline__ float quad_sum(float x) {
  x += mk::dppf<0xB1, 0xf>(0.0f, x);   // quad_perm (1, 0, 3, 2)
  x += mk::dppf<0x4E, 0xf>(0.0f, x);   // quad_perm (2, 3, 0, 1)
  return x;
}

template <int DH, typename TX>
__global__ __launch_bounds__(4 * DH) void slstm_kernel(SlstmArgs a) {
  constexpr int QV = DH / 4;          // h entries per quarter
  constexpr int QS = QV + 4;          // padded quarter stride (floats)
  __shared__ __align__(16) float sh[2][4 * QS];
  const int tid = threadIdx.x;
  const int u = tid >> 2, q = tid & 3;
  const int64_t bh = blockIdx.x;
  const int hd = static_cast<int>(bh % a.NH);
  const int64_t T = a.T;

  float r[4][QV];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float* Rrow = a.R + ((static_cast<int64_t>(hd) * 4 + g) * DH + u) * DH + q * QV;
#pragma unroll
    for (int j = 0; j < QV; j += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(Rrow + j);
      r[g][j] = v4.x; r[g][j + 1] = v4.y; r[g][j + 2] = v4.z; r[g][j + 3] = v4.w;
    }
  }
  const int64_t si = bh * DH + u;
  float c = a.c0 ? a.c0[si] : 0.0f;
  float n = a.c0 ? a.n0[si] : 0.0f;
  float m = a.c0 ? a.m0[si] : 0.0f;
  float hv = a.c0 ? a.h0[si] : 0.0f;
  const int hslot = (u / QV) * QS + (u % QV);   // where unit u's h lives
  if (q == 0) sh[0][hslot] = hv;
  __syncthreads();

  // lane (u, q) supplies the input projection of gate q of unit u
  const int64_t xbase = bh * T * 4 * DH + q * DH + u;
  float xb[PF], xn[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) xb[k] = k < T ? ldx<TX>(a.wx, xbase + static_cast<int64_t>(k) * 4 * DH) : 0.0f;

  for (int64_t t0 = 0; t0 < T; t0 += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int64_t t = t0 + PF + k;
      xn[k] = t < T ? ldx<TX>(a.wx, xbase + t * 4 * DH) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int64_t t = t0 + k;
      if (t >= T) break;   // uniform across the workgroup
      const float* hp = sh[t & 1] + q * QS;
      float hq[QV];   // all LDS reads first, so that their latencies overlap
#pragma unroll
      for (int j = 0; j < QV; j += 4) {
        const float4 h4 = *reinterpret_cast<const float4*>(hp + j);
        hq[j] = h4.x; hq[j + 1] = h4.y; hq[j + 2] = h4.z; hq[j + 3] = h4.w;
      }
      // two fused multiply-add chains per gate
      float acc[4], acc2[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[g] = q == g ? xb[k] : 0.0f;
        acc2[g] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < QV; j += 2)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          acc[g] = fmaf(r[g][j], hq[j], acc[g]);
          acc2[g] = fmaf(r[g][j + 1], hq[j + 1], acc2[g]);
        }
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] = quad_sum(acc[g] + acc2[g]);
      // hardware exp / log / reciprocal (relative error ~1e-7)
      const float lf = a.fgate_exp ? acc[1] : mk::log_sigmoid_fast(acc[1]);
      const float m_new = fmaxf(lf + m, acc[0]);
      const float fp = __expf(lf + m - m_new);
      const float ip = __expf(acc[0] - m_new);
      c = fp * c + ip * acc[2];
      n = fp * n + ip;
      m = m_new;
      hv = c * __builtin_amdgcn_rcpf(n * (1.0f + __expf(-acc[3])));
      if (q == 0) {
        sh[(t + 1) & 1][hslot] = hv;
        if (sizeof(TX) == 2) static_cast<bf16_t*>(a.h)[(bh * T + t) * DH + u] = f2bf(hv);
        else static_cast<float*>(a.h)[(bh * T + t) * DH + u] = hv;
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) xb[k] = xn[k];
  }
  if (q == 0 && a.c1) {
    a.c1[si] = c;
    a.n1[si] = n;
    a.m1[si] = m;
    a.h1[si] = hv;
  }
}

template <typename TX>
hipError_t launch_tx(const SlstmArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>(a.B * a.NH);
  switch (a.DH) {
    case 16: slstm_kernel<16, TX><<<grid, 64, 0, st>>>(a); break;
    case 32: slstm_kernel<32, TX><<<grid, 128, 0, st>>>(a); break;
    case 64: slstm_kernel<64, TX><<<grid, 256, 0, st>>>(a); break;
    default: slstm_kernel<128, TX><<<grid, 512, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_slstm(const SlstmArgs& a, hipStream_t st) {
  return a.x_bf16 ? launch_tx<bf16_t>(a, st) : launch_tx<float>(a, st);
}

}  // namespace mlstm
