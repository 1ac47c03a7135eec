// Device helpers shared by the mLSTM kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

// ---------------------------------------------------------------- types
typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an IEEE float)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f2bf(x); }

// Low / high bfloat16 of a packed 32-bit word, as float.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// 8 floats -> MFMA bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  uint4 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  u.z = pack_bf2(x[4], x[5]);
  u.w = pack_bf2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ------------------------------------------------------- gate math
// log(sigmoid(x)) without overflow: min(x, 0) - log1p(exp(-|x|)).
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.0f) - log1pf(__expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// log f_t from the forget-gate preactivation: sigmoid gate or exponential gate.
__device__ __forceinline__ float log_forget(float f_pre, int fgate_exp) {
  return fgate_exp ? f_pre : log_sigmoid(f_pre);
}

// ------------------------------------------------------- wave64 scans
__device__ __forceinline__ float wave_incl_sum(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_incl_max(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(x, o, 64);
    if (lane >= o) x = fmaxf(x, y);
  }
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ------------------------------------------------------- MFMA
// D = A * B + C for a 16x16 tile with k = 32 (bf16 in, fp32 accumulate).
// Lane l holds A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16] (e = 0..7)
// and D[4 (l / 16) + e][l % 16] (e = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace mlstm
