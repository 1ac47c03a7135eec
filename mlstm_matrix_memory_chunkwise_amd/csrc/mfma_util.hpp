// LDS, DMA, conversion and cross-lane helpers of the MFMA chunkwise kernels
// (gfx950, wave64).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mlstm {
namespace mk {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Byte offset of element (row, col) in a [rows x 64] bf16 tile with 128-byte
// rows whose 16-byte chunks are XOR-swizzled by (row / 2) mod 8: the 16 rows
// read by one MFMA fragment land on 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int col) {
  return row * 128 + 16 * ((col >> 3) ^ ((row >> 1) & 7)) + 2 * (col & 7);
}

__device__ __forceinline__ uint4 lds_ld16(const char* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

// ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3 name 4
// consecutive bf16 of "row" r (r = 0..3); lane c of the group receives
// element c of the 16-wide concatenation of each row, for rows 0..3.
__device__ __forceinline__ uint2 lds_tr(const char* base, int off) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8 join(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 cvt8(const float* x) {
  return __builtin_bit_cast(
      bf16x8, make_uint4(cvt2(x[0], x[1]), cvt2(x[2], x[3]), cvt2(x[4], x[5]), cvt2(x[6], x[7])));
}

// 8 floats -> (hi, lo) bf16 operands with hi = bf16(x) and lo = bf16(x - hi):
// hi + lo carries about 16 significant bits, so two MFMAs with (hi, lo)
// contract a float32 operand nearly exactly.
__device__ __forceinline__ void cvt8_split(const float* x, bf16x8& hi, bf16x8& lo) {
  hi = cvt8(x);
  const uint4 h = __builtin_bit_cast(uint4, hi);
  float r[8];
  r[0] = x[0] - bf_lo(h.x); r[1] = x[1] - bf_hi(h.x);
  r[2] = x[2] - bf_lo(h.y); r[3] = x[3] - bf_hi(h.y);
  r[4] = x[4] - bf_lo(h.z); r[5] = x[5] - bf_hi(h.z);
  r[6] = x[6] - bf_lo(h.w); r[7] = x[7] - bf_hi(h.w);
  lo = cvt8(r);
}

// x -> three bf16 (storage bits) whose sum is x to about 24 significant
// bits: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid) (each
// difference is exact in float32)
__device__ __forceinline__ void split3_bf16(float x, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
  const uint32_t h = cvt2(x, 0.0f);
  const float r1 = x - bf_lo(h);
  const uint32_t m = cvt2(r1, 0.0f);
  hi = static_cast<bf16_t>(h);
  mid = static_cast<bf16_t>(m);
  lo = static_cast<bf16_t>(cvt2(r1 - bf_lo(m), 0.0f));
}

// global -> LDS loads.  Lane l's 16 (4) bytes land at lds + 16 l (4 l); the
// LDS base goes through M0.  Issued from asm so that the compiler neither
// tracks nor waits on them: every wait on them is an explicit vmcnt wait.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(gsrc) : "memory");
}
// the same, for data read once (streamed past the caches)
__device__ __forceinline__ void dma16_nt(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(lds), "v"(gsrc) : "memory");
}
__device__ __forceinline__ void dma4(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds), "v"(gsrc) : "memory");
}
// the same two loads from a wave-uniform base (SGPR pair) plus a 32-bit
// per-lane byte offset: no per-lane 64-bit address arithmetic
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma16_nt_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// 8-byte store of data written once
__device__ __forceinline__ void st8_nt(void* p, uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = {lo, hi};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- explicit wait counts for the stage ring.  Issue order of one wave: at
// the top of stage y (after its barrier) the loads of stage y + D (NBQK, plus
// NBV when y + D opens a chunk), then, when y opens chunk c, the per-chunk
// loads (NBX).  Loads of stage x were issued at the top of stage x - D; the
// loads issued after them when the wave waits for stage x (slice s) are
// counted here.  Vector-memory stores are not counted, which can only make a
// wait stricter.
template <int NS, int D, int NBQK, int NBV, int NBX>
__host__ __device__ constexpr int loads_after_stage(int s) {
  int n = 0;
  for (int k = 1; k < D; ++k) n += NBQK + (((s + k) % NS) == 0 ? NBV : 0);
  for (int k = 1; k <= D; ++k) n += (((s - k) % NS + NS) % NS == 0) ? NBX : 0;
  return n;
}
// ... and after the per-chunk loads of chunk c, at the end of chunk c.
template <int NS, int D, int NBQK, int NBV>
__host__ __device__ constexpr int loads_after_chunk_extras() {
  int n = 0;
  for (int k = 1; k < NS; ++k) n += NBQK + (((k + D) % NS) == 0 ? NBV : 0);
  return n;
}
// Wait for the stage with slice index s (folds to one s_waitcnt once the
// slice loop is unrolled).
template <int NS, int D, int NBQK, int NBV, int NBX>
__device__ __forceinline__ void wait_stage(int s) {
  switch (s) {
    case 0: wait_vm<loads_after_stage<NS, D, NBQK, NBV, NBX>(0)>(); break;
    case 1: wait_vm<loads_after_stage<NS, D, NBQK, NBV, NBX>(1 % NS)>(); break;
    case 2: wait_vm<loads_after_stage<NS, D, NBQK, NBV, NBX>(2 % NS)>(); break;
    default: wait_vm<loads_after_stage<NS, D, NBQK, NBV, NBX>(3 % NS)>(); break;
  }
}

template <int W>
using wave_c = std::integral_constant<int, W>;

// Runs f with the (wave-uniform) wave index as a compile-time constant, so that
// per-wave work splits fold into straight-line code instead of branches.
template <int NWAVES, typename F>
__device__ __forceinline__ void for_wave(int wave, F&& f) {
  static_assert(NWAVES == 4 || NWAVES == 8, "4 or 8 waves");
  switch (wave) {
    case 0: f(wave_c<0>{}); break;
    case 1: f(wave_c<1>{}); break;
    case 2: f(wave_c<2>{}); break;
    case 3: f(wave_c<3>{}); break;
    case 4: if constexpr (NWAVES == 8) f(wave_c<4>{}); break;
    case 5: if constexpr (NWAVES == 8) f(wave_c<5>{}); break;
    case 6: if constexpr (NWAVES == 8) f(wave_c<6>{}); break;
    default: if constexpr (NWAVES == 8) f(wave_c<7>{}); break;
  }
}

// ---- DPP wave64 scans (gfx9 row_shr / row_bcast): no LDS round trips.
template <int CTRL, int RMASK>
__device__ __forceinline__ float dppf(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, x),
                                                               CTRL, RMASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float scan_add(float x) {
  x += dppf<0x111, 0xf>(0.0f, x);   // row_shr:1
  x += dppf<0x112, 0xf>(0.0f, x);   // row_shr:2
  x += dppf<0x114, 0xf>(0.0f, x);   // row_shr:4
  x += dppf<0x118, 0xf>(0.0f, x);   // row_shr:8
  x += dppf<0x142, 0xa>(0.0f, x);   // row_bcast:15 into rows 1, 3
  x += dppf<0x143, 0xc>(0.0f, x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive prefix maximum over the 64 lanes.
__device__ __forceinline__ float scan_max(float x) {
  const float ninf = -INFINITY;
  x = fmaxf(x, dppf<0x111, 0xf>(ninf, x));
  x = fmaxf(x, dppf<0x112, 0xf>(ninf, x));
  x = fmaxf(x, dppf<0x114, 0xf>(ninf, x));
  x = fmaxf(x, dppf<0x118, 0xf>(ninf, x));
  x = fmaxf(x, dppf<0x142, 0xa>(ninf, x));
  x = fmaxf(x, dppf<0x143, 0xc>(ninf, x));
  return x;
}

// Sum of a value over the four 16-lane groups (lanes l, l^16, l^32, l^48),
// with the gfx950 lane-swap instructions: after v_permlane16_swap of (x, x)
// the two outputs hold x of row pairs (0, 1) and (2, 3) in swapped order, so
// their sum is the sum over lanes l and l^16; v_permlane32_swap does the same
// for the two halves.  The outputs are read as plain values: hipcc reads the
// wrong element when __builtin_bit_cast is applied to an element of the
// returned vector.
__device__ __forceinline__ float sum_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = r16[0], a1 = r16[1];
  const float s16 = __uint_as_float(a0) + __uint_as_float(a1);
  const uint32_t v = __float_as_uint(s16);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t b0 = r32[0], b1 = r32[1];
  return __uint_as_float(b0) + __uint_as_float(b1);
}

// log(sigmoid(x)) = min(x, 0) - log(1 + exp(-|x|)), with the hardware exp/log
// (absolute error ~1e-7, enough for a log-space gate).
__device__ __forceinline__ float log_sigmoid_fast(float x) {
  return fminf(x, 0.0f) - __logf(1.0f + __expf(-fabsf(x)));
}

__device__ __forceinline__ float log_forget_fast(float f_pre, int fgate_exp) {
  return fgate_exp ? f_pre : log_sigmoid_fast(f_pre);
}

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace mk
}  // namespace mlstm
