// The two block operations around the mLSTM cell (gfx950), both bound by HBM
// bandwidth.  Method: the mLSTM block of the xLSTM post (llms.blog), section 4
// "xLSTM Block Architecture and Residual Stacking", "mLSTM Block Structure",
// items 3 and 5 and the block figure.
//
//  * Per-head group normalization with the output gate, on the cell output
//    h [B, H, T, d_v]: y = sigmoid(o~) (gamma (h - mean) / sqrt(var + eps) +
//    beta), mean and (biased) variance over the d_v features of one (b, head,
//    t).  One wave per (b, head, t) row: the row is loaded once into
//    registers, reduced twice across the wave (mean, then the centred second
//    moment, so no cancellation), and written once.
//  * Causal depthwise convolution over the token axis, x [B, T, C]:
//    y[t, c] = bias[c] + sum_{s<K} w[c, s] x[t - K + 1 + s, c], with an
//    optional carried window of the K - 1 inputs before t = 0.  One thread per
//    (b, 8 or 4 channels, run of tokens) slides the window along its run in
//    registers; a wave covers 64 neighbouring channel groups, so every token
//    row is read as contiguous 16-byte pieces.
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

// ---------------------------------------------------------------- GroupNorm

constexpr int GN_WAVES = 4;
constexpr int GN_MAXC = 4;   // 4-element pieces per lane: d_v <= 1024

__device__ __forceinline__ void load4(const void* p, int bf16, int64_t i, float* x) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p) + i);
    x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
}

__device__ __forceinline__ float wave_allsum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(GN_WAVES * 64) void groupnorm_ogate_kernel(GnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * GN_WAVES + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int dv = a.dv;
  const int64_t base = row * dv;
  const int head = static_cast<int>((row / a.T) % a.H);
  float x[GN_MAXC][4];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < GN_MAXC; ++c) {
    const int e = 4 * lane + 256 * c;
    if (e < dv) {
      load4(a.h, a.h_bf16, base + e, x[c]);
      s += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
    }
  }
  const float mean = wave_allsum(s) / static_cast<float>(dv);
  float s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < GN_MAXC; ++c) {
    const int e = 4 * lane + 256 * c;
    if (e < dv) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[c][j] -= mean;
        s2 += x[c][j] * x[c][j];
      }
    }
  }
  const float rstd = rsqrtf(wave_allsum(s2) / static_cast<float>(dv) + a.eps);
#pragma unroll
  for (int c = 0; c < GN_MAXC; ++c) {
    const int e = 4 * lane + 256 * c;
    if (e >= dv) continue;
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = x[c][j] * rstd;
    if (a.gamma) {
      const float4 g = *reinterpret_cast<const float4*>(a.gamma + static_cast<int64_t>(head) * dv + e);
      y[0] *= g.x; y[1] *= g.y; y[2] *= g.z; y[3] *= g.w;
    }
    if (a.beta) {
      const float4 b = *reinterpret_cast<const float4*>(a.beta + static_cast<int64_t>(head) * dv + e);
      y[0] += b.x; y[1] += b.y; y[2] += b.z; y[3] += b.w;
    }
    if (a.o_pre) {
      float o[4];
      load4(a.o_pre, a.o_bf16, base + e, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] *= 1.0f / (1.0f + __expf(-o[j]));
    }
    if (a.h_bf16) {
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.y) + base + e) =
          make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.y) + base + e) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

// ---------------------------------------------------------------- causal conv

constexpr int CONV_THREADS = 256;
constexpr int CONV_RUN = 64;      // tokens per thread

// VE channels per thread (8 for bf16, 4 for float32), kernel size K.
template <int VE, int K>
__global__ __launch_bounds__(CONV_THREADS) void causal_conv_kernel(ConvArgs a) {
  const int64_t ng = a.C / VE;                       // channel groups
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * CONV_THREADS + threadIdx.x;
  const int64_t nruns = (a.T + CONV_RUN - 1) / CONV_RUN;
  if (gid >= a.B * nruns * ng) return;
  const int64_t grp = gid % ng;
  const int64_t run = (gid / ng) % nruns;
  const int64_t b = gid / (ng * nruns);
  const int64_t c0 = grp * VE;
  const int64_t t0 = run * CONV_RUN;
  const int64_t t1 = t0 + CONV_RUN < a.T ? t0 + CONV_RUN : a.T;

  float w[VE][K], bias[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) {
#pragma unroll
    for (int s = 0; s < K; ++s) w[v][s] = a.w[(c0 + v) * K + s];
    bias[v] = a.bias ? a.bias[c0 + v] : 0.0f;
  }
  auto load = [&](int64_t t, float* dst) {
    if (a.x_bf16) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.x) + (b * a.T + t) * a.C + c0);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int v = 0; v < VE; ++v) dst[v] = (v & 1) ? bf_hi(wd[(v >> 1) & 3]) : bf_lo(wd[(v >> 1) & 3]);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (b * a.T + t) * a.C + c0);
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int v = 0; v < VE; ++v) dst[v] = fv[v & 3];
    }
  };
  // window: win[s] holds the input at t - (K - 1) + s for s < K - 1
  float win[K > 1 ? K - 1 : 1][VE];
#pragma unroll
  for (int s = 0; s < K - 1; ++s) {
    const int64_t t = t0 - (K - 1) + s;
    if (t >= 0) {
      load(t, win[s]);
    } else if (a.state_in) {
      const float* st = a.state_in + (b * (K - 1) + (K - 1 + t)) * a.C + c0;
#pragma unroll
      for (int v = 0; v < VE; ++v) win[s][v] = st[v];
    } else {
#pragma unroll
      for (int v = 0; v < VE; ++v) win[s][v] = 0.0f;
    }
  }
  constexpr int U = 4;   // tokens loaded ahead together
  for (int64_t t = t0; t < t1; t += U) {
    float cur[U][VE];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u < t1) load(t + u, cur[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u >= t1) break;
      float y[VE];
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        float acc = bias[v];
#pragma unroll
        for (int s = 0; s < K - 1; ++s) acc += w[v][s] * win[s][v];
        y[v] = acc + w[v][K - 1] * cur[u][v];
      }
#pragma unroll
      for (int s = 0; s + 1 < K - 1; ++s)
#pragma unroll
        for (int v = 0; v < VE; ++v) win[s][v] = win[s + 1][v];
      if (K > 1) {
#pragma unroll
        for (int v = 0; v < VE; ++v) win[K > 1 ? K - 2 : 0][v] = cur[u][v];
      }
      const int64_t o = (b * a.T + t + u) * a.C + c0;
      if (a.x_bf16) {
        uint32_t p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) p[v] = pack_bf2(y[(2 * v) % VE], y[(2 * v + 1) % VE]);
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.y) + o) = make_uint4(p[0], p[1], p[2], p[3]);
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.y) + o) =
            make_float4(y[0], y[1 % VE], y[2 % VE], y[3 % VE]);
      }
    }
  }
  // the run that ends the sequence leaves the last K - 1 inputs in its window
  if (a.state_out && t1 == a.T) {
#pragma unroll
    for (int s = 0; s < K - 1; ++s) {
      float* st = a.state_out + (b * (K - 1) + s) * a.C + c0;
#pragma unroll
      for (int v = 0; v < VE; ++v) st[v] = win[s][v];
    }
  }
}

template <int VE>
hipError_t launch_conv_ve(const ConvArgs& a, hipStream_t st) {
  const int64_t nruns = (a.T + CONV_RUN - 1) / CONV_RUN;
  const int64_t threads = a.B * nruns * (a.C / VE);
  const unsigned blocks = static_cast<unsigned>((threads + CONV_THREADS - 1) / CONV_THREADS);
  switch (a.K) {
    case 1: causal_conv_kernel<VE, 1><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 2: causal_conv_kernel<VE, 2><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 3: causal_conv_kernel<VE, 3><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 4: causal_conv_kernel<VE, 4><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 5: causal_conv_kernel<VE, 5><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 6: causal_conv_kernel<VE, 6><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    case 7: causal_conv_kernel<VE, 7><<<blocks, CONV_THREADS, 0, st>>>(a); break;
    default: causal_conv_kernel<VE, 8><<<blocks, CONV_THREADS, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_groupnorm_ogate(const GnArgs& a, hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((a.rows + GN_WAVES - 1) / GN_WAVES);
  groupnorm_ogate_kernel<<<blocks, GN_WAVES * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_causal_conv(const ConvArgs& a, hipStream_t st) {
  return a.x_bf16 ? launch_conv_ve<8>(a, st) : launch_conv_ve<4>(a, st);
}

}  // namespace mlstm
