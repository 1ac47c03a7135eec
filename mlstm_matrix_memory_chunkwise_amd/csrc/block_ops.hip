// The two block operations around the mLSTM cell (gfx950), both bound by HBM
// bandwidth.  Method: the mLSTM block of the xLSTM post (llms.blog), section 4
// "xLSTM Block Architecture and Residual Stacking", "mLSTM Block Structure",
// items 3 and 5 and the block figure.
//
//  * Per-head group normalization with the output gate, on the cell output
//    h [B, H, T, d_v]: y = sigmoid(o~) (gamma (h - mean) / sqrt(var + eps) +
//    beta), mean and (biased) variance over the d_v features of one (b, head,
//    t).  With d_v a multiple of 8, a row is held by half a wave in 16-byte
//    pieces (8 features per lane), so each load instruction covers two rows;
//    otherwise one wave per row, 4 features per lane.  The rows are loaded
//    once into registers with every load issued before the first reduction,
//    reduced twice (mean, then the centred second moment, so no
//    cancellation), and written once.
//  * Causal depthwise convolution over the token axis, x [B, T, C]:
//    y[t, c] = bias[c] + sum_{s<K} w[c, s] x[t - K + 1 + s, c], with an
//    optional carried window of the K - 1 inputs before t = 0.  One thread per
//    (b, 8 or 4 channels, run of 128 tokens) slides the window along its run
//    in registers, loading the next 4 tokens while it computes the current
//    4 (software pipeline); a wave covers 64
//    neighbouring channel groups, so every token row is read as contiguous
//    16-byte pieces.
#include "common.hpp"
#include "kernels.hpp"

namespace mlstm {
namespace {

// ---------------------------------------------------------------- GroupNorm

constexpr int GN_WAVES = 4;

// Data read or written exactly once go through non-temporal accesses, so
// that streaming them does not evict what the caches hold for others.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 ld8_nt(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st8_nt(void* p, uint2 x) {
  const u32x2 v = {x.x, x.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, uint4 x) {
  const u32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ void load4(const void* p, int bf16, int64_t i, float* x) {
  if (bf16) {
    const uint2 u = ld8_nt(static_cast<const bf16_t*>(p) + i);
    x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  } else {
    const uint4 f = ld16_nt(static_cast<const float*>(p) + i);
    x[0] = __uint_as_float(f.x); x[1] = __uint_as_float(f.y);
    x[2] = __uint_as_float(f.z); x[3] = __uint_as_float(f.w);
  }
}

__device__ __forceinline__ float wave_allsum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// NCH 4-feature pieces per lane (d_v <= 256 NCH), RW rows per wave: every
// load of the wave's RW rows (h and o~) is issued before the first
// reduction, so that RW * NCH * 64 * (h + o~ bytes) are in flight per wave.
template <int NCH, int RW>
__global__ __launch_bounds__(GN_WAVES * 64) void groupnorm_ogate_kernel(GnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * GN_WAVES + (threadIdx.x >> 6)) * RW;
  const int dv = a.dv;
  float x[RW][NCH][4], o[RW][NCH][4];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const int64_t row = row0 + w;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = 4 * lane + 256 * c;
      if (row < a.rows && e < dv) {
        load4(a.h, a.h_bf16, row * dv + e, x[w][c]);
        if (a.o_pre) load4(a.o_pre, a.o_bf16, row * dv + e, o[w][c]);
      }
    }
  }
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const int64_t row = row0 + w;
    if (row >= a.rows) break;   // uniform across the wave
    const int64_t base = row * dv;
    const int head = static_cast<int>((row / a.T) % a.H);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (4 * lane + 256 * c < dv) s += (x[w][c][0] + x[w][c][1]) + (x[w][c][2] + x[w][c][3]);
    const float mean = wave_allsum(s) / static_cast<float>(dv);
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (4 * lane + 256 * c < dv) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[w][c][j] -= mean;
          s2 += x[w][c][j] * x[w][c][j];
        }
      }
    }
    const float rstd = rsqrtf(wave_allsum(s2) / static_cast<float>(dv) + a.eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = 4 * lane + 256 * c;
      if (e >= dv) continue;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = x[w][c][j] * rstd;
      if (a.gamma) {
        const float4 g = *reinterpret_cast<const float4*>(a.gamma + static_cast<int64_t>(head) * dv + e);
        y[0] *= g.x; y[1] *= g.y; y[2] *= g.z; y[3] *= g.w;
      }
      if (a.beta) {
        const float4 b = *reinterpret_cast<const float4*>(a.beta + static_cast<int64_t>(head) * dv + e);
        y[0] += b.x; y[1] += b.y; y[2] += b.z; y[3] += b.w;
      }
      if (a.o_pre) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= 1.0f / (1.0f + __expf(-o[w][c][j]));
      }
      if (a.h_bf16) {
        st8_nt(static_cast<bf16_t*>(a.y) + base + e, make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])));
      } else {
        st16_nt(static_cast<float*>(a.y) + base + e,
                make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                           __float_as_uint(y[3])));
      }
    }
  }
}

// 8 features per lane (16-byte bf16 h loads): a row of d_v <= 256 NCH8
// features is held by one half-wave (32 lanes) in NCH8 pieces, so one load
// instruction covers two rows; RW row pairs per wave, every load issued
// before the first reduction.  d_v must be a multiple of 8.
__device__ __forceinline__ float half_allsum(float x) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ void load8(const void* p, int bf16, int64_t i, float* x) {
  if (bf16) {
    const uint4 u = ld16_nt(static_cast<const bf16_t*>(p) + i);
    x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
    x[4] = bf_lo(u.z); x[5] = bf_hi(u.z); x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
  } else {
    const uint4 f0 = ld16_nt(static_cast<const float*>(p) + i);
    const uint4 f1 = ld16_nt(static_cast<const float*>(p) + i + 4);
    x[0] = __uint_as_float(f0.x); x[1] = __uint_as_float(f0.y);
    x[2] = __uint_as_float(f0.z); x[3] = __uint_as_float(f0.w);
    x[4] = __uint_as_float(f1.x); x[5] = __uint_as_float(f1.y);
    x[6] = __uint_as_float(f1.z); x[7] = __uint_as_float(f1.w);
  }
}

template <int NCH8, int RW>
__global__ __launch_bounds__(GN_WAVES * 64) void groupnorm_ogate8_kernel(GnArgs a) {
  const int lane = threadIdx.x & 63, hl = lane & 31, half = lane >> 5;
  const int64_t pair0 = (static_cast<int64_t>(blockIdx.x) * GN_WAVES + (threadIdx.x >> 6)) * RW;
  const int dv = a.dv;
  float x[RW][NCH8][8], o[RW][NCH8][8];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const int64_t row = 2 * (pair0 + w) + half;
#pragma unroll
    for (int c = 0; c < NCH8; ++c) {
      const int e = 8 * hl + 256 * c;
      if (row < a.rows && e < dv) {
        load8(a.h, a.h_bf16, row * dv + e, x[w][c]);
        if (a.o_pre) load8(a.o_pre, a.o_bf16, row * dv + e, o[w][c]);
      }
    }
  }
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const int64_t row = 2 * (pair0 + w) + half;
    const bool live = row < a.rows;   // the two halves may differ only at the very end
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH8; ++c)
      if (live && 8 * hl + 256 * c < dv)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += x[w][c][j];
    const float mean = half_allsum(s) / static_cast<float>(dv);
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH8; ++c) {
      if (live && 8 * hl + 256 * c < dv) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[w][c][j] -= mean;
          s2 += x[w][c][j] * x[w][c][j];
        }
      }
    }
    const float rstd = rsqrtf(half_allsum(s2) / static_cast<float>(dv) + a.eps);
    if (!live) continue;
    const int64_t base = row * dv;
    const int head = static_cast<int>((row / a.T) % a.H);
#pragma unroll
    for (int c = 0; c < NCH8; ++c) {
      const int e = 8 * hl + 256 * c;
      if (e >= dv) continue;
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = x[w][c][j] * rstd;
      if (a.gamma) {
        const float4 g0 = *reinterpret_cast<const float4*>(a.gamma + static_cast<int64_t>(head) * dv + e);
        const float4 g1 = *reinterpret_cast<const float4*>(a.gamma + static_cast<int64_t>(head) * dv + e + 4);
        y[0] *= g0.x; y[1] *= g0.y; y[2] *= g0.z; y[3] *= g0.w;
        y[4] *= g1.x; y[5] *= g1.y; y[6] *= g1.z; y[7] *= g1.w;
      }
      if (a.beta) {
        const float4 b0 = *reinterpret_cast<const float4*>(a.beta + static_cast<int64_t>(head) * dv + e);
        const float4 b1 = *reinterpret_cast<const float4*>(a.beta + static_cast<int64_t>(head) * dv + e + 4);
        y[0] += b0.x; y[1] += b0.y; y[2] += b0.z; y[3] += b0.w;
        y[4] += b1.x; y[5] += b1.y; y[6] += b1.z; y[7] += b1.w;
      }
      if (a.o_pre) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] *= 1.0f / (1.0f + __expf(-o[w][c][j]));
      }
      if (a.h_bf16) {
        st16_nt(static_cast<bf16_t*>(a.y) + base + e,
                make_uint4(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]), pack_bf2(y[4], y[5]),
                           pack_bf2(y[6], y[7])));
      } else {
        float* yp = static_cast<float*>(a.y) + base + e;
        st16_nt(yp, make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                               __float_as_uint(y[3])));
        st16_nt(yp + 4, make_uint4(__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                                   __float_as_uint(y[7])));
      }
    }
  }
}

template <int NCH8, int RW>
hipError_t launch_gn8(const GnArgs& a, hipStream_t st) {
  const int64_t pairs = (a.rows + 1) / 2;
  const int64_t per_block = static_cast<int64_t>(GN_WAVES) * RW;
  const unsigned blocks = static_cast<unsigned>((pairs + per_block - 1) / per_block);
  groupnorm_ogate8_kernel<NCH8, RW><<<blocks, GN_WAVES * 64, 0, st>>>(a);
  return hipGetLastError();
}

template <int NCH, int RW>
hipError_t launch_gn(const GnArgs& a, hipStream_t st) {
  const int64_t per_block = static_cast<int64_t>(GN_WAVES) * RW;
  const unsigned blocks = static_cast<unsigned>((a.rows + per_block - 1) / per_block);
  groupnorm_ogate_kernel<NCH, RW><<<blocks, GN_WAVES * 64, 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- causal conv

constexpr int CONV_THREADS = 256;
constexpr int CONV_RUN = 128;     // tokens per thread (longer runs: fewer window and weight loads)

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
  // Software pipeline over batches of U tokens: the raw 16-byte rows of the
  // next batch are requested before the current batch is computed.  Loads
  // past the run's end re-read its last token (always in bounds, no branch).
  constexpr int U = 4;
  const char* xrow = static_cast<const char*>(a.x) + (b * a.T * a.C + c0) * (a.x_bf16 ? 2 : 4);
  const int64_t rstride = a.C * (a.x_bf16 ? 2 : 4);
  uint4 nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t tt = t0 + u < t1 ? t0 + u : t1 - 1;
    nxt[u] = *reinterpret_cast<const uint4*>(xrow + tt * rstride);
  }
  for (int64_t t = t0; t < t1; t += U) {
    uint4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t + U + u < t1 ? t + U + u : t1 - 1;
      nxt[u] = *reinterpret_cast<const uint4*>(xrow + tt * rstride);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u >= t1) break;
      float xv[VE];
      {
        const uint32_t wd[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
        for (int v = 0; v < VE; ++v)
          xv[v] = a.x_bf16 ? ((v & 1) ? bf_hi(wd[(v >> 1) & 3]) : bf_lo(wd[(v >> 1) & 3]))
                           : __uint_as_float(wd[v & 3]);
      }
      float y[VE];
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        float acc = bias[v];
#pragma unroll
        for (int s = 0; s < K - 1; ++s) acc += w[v][s] * win[s][v];
        y[v] = acc + w[v][K - 1] * xv[v];
      }
#pragma unroll
      for (int s = 0; s + 1 < K - 1; ++s)
#pragma unroll
        for (int v = 0; v < VE; ++v) win[s][v] = win[s + 1][v];
      if (K > 1) {
#pragma unroll
        for (int v = 0; v < VE; ++v) win[K > 1 ? K - 2 : 0][v] = xv[v];
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
  if (a.dv % 8 == 0) {
    if (a.dv <= 256) return launch_gn8<1, 2>(a, st);
    if (a.dv <= 512) return launch_gn8<2, 1>(a, st);
    return launch_gn8<4, 1>(a, st);
  }
  if (a.dv <= 256) return launch_gn<1, 4>(a, st);
  if (a.dv <= 512) return launch_gn<2, 2>(a, st);
  return launch_gn<4, 1>(a, st);
}

hipError_t launch_causal_conv(const ConvArgs& a, hipStream_t st) {
  return a.x_bf16 ? launch_conv_ve<8>(a, st) : launch_conv_ve<4>(a, st);
}

}  // namespace mlstm
