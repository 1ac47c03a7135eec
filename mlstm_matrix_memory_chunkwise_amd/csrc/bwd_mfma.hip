// State and reverse passes of the chunkwise backward on bf16 MFMA (gfx950):
// chunk 64, 64 value columns per workgroup, d_qk in {64, 128, 256}, bf16
// q/k/v/h/dh.
//
// The same gradient as the float32 passes in bwd.hip (the derivative of the
// forward pass of the xLSTM post, llms.blog, section 3 "Associative Matrix
// Cell State" and "The Parallel Dual Form", with the running maximum of
// section 2 "The Normalizer State and Numerical Stabilization"), with every
// matrix product on 16x16x32 MFMAs.  Per chunk of 64 tokens, with the stored
// state (C~_s, n~_s, m_s) and the carried memory gradient dC, the reverse
// pass forms
//
//   S = Q K^T,  DS = D (.) S              (masked; stored transposed, bf16;
//                                          row sums in float32)
//   r = sigmoid(o~) dh / den,  g r,  w V (bf16 in LDS)
//   W = D (.) (R V^T + dnq)               (bf16 in LDS)
//   dq^T = K^T W^T + C~_s (g R)^T  (+ g dnq n~_s)
//   dk^T = Q^T W + dC (w V)^T      (+ w dn)
//   dv^T = R^T DS + w (dC^T K^T)          (dC as a bf16 hi / lo pair)
//   dC^T <- g_L dC^T + (g R)^T Q,  dn <- g_L dn + sum_i g_i dnq_i q_i
//
// Operands are read from swizzled [rows][64] bf16 LDS tiles either as row
// fragments (8 consecutive columns, ds_read_b128) or as transposed column
// fragments (8 consecutive rows, two ds_read_b64_tr_b16), both in natural
// index order.  The memory gradient is carried transposed in float32
// registers (dC^T tiles, one 16-column block per wave), which makes its bf16
// copy for the products a run of 4 consecutive columns per lane.  The
// products round their other operands to bf16 (accumulation stays float32);
// q, k, v are exact.  Vectors that meet a matrix in float32 precision (dn's
// g dnq, the state pass's w (.) V and w) enter as bf16 hi / lo pairs.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT4 = 256;           // 4 waves
constexpr int LC = 64;             // chunk
constexpr int TVC = 64;            // value columns per workgroup
constexpr int TB = 64 * 128;       // bytes of a [64][64] bf16 tile

__device__ __forceinline__ bf16x8 rowfrag(const char* t, int r, int c) {
  return as_bf16x8(lds_ld16(t, swz(r, c)));
}
// X[l16][8g + e] = M[k0 + 8g + e][m0 + l16] of the tile M at t
__device__ __forceinline__ bf16x8 colfrag(const char* t, int k0, int m0, int g, int kr, int kq) {
  return join(lds_tr(t, swz(k0 + 8 * g + kr, m0 + 4 * kq)), lds_tr(t, swz(k0 + 8 * g + 4 + kr, m0 + 4 * kq)));
}
// the 64-column tile of a wide [64][DK] matrix holding column c
__device__ __forceinline__ const char* wide(const char* base, int c) { return base + (c >> 6) * TB; }

// Workgroup -> (head, column block).  Workgroups are dealt to the 8 XCDs in
// turn (block id mod 8); with B*H a multiple of 8 the column blocks of one
// head get ids equal mod 8, so their shared q/k reads meet in one L2.
__device__ __forceinline__ void head_block(int64_t nhead, int ncb, int64_t& bh, int& cb) {
  const int64_t w = blockIdx.x;
  if (nhead % 8 == 0) {
    const int64_t grp = w / (8 * ncb), r = w % (8 * ncb);
    cb = static_cast<int>(r / 8);
    bh = grp * 8 + r % 8;
  } else {
    bh = w / ncb;
    cb = static_cast<int>(w % ncb);
  }
}

struct Gate64 {
  float u[LC], M[LC], m[LC], g[LC], w[LC];
};

__device__ __forceinline__ void gate_scan64(const BwdArgs& a, int64_t tok0, float ms, Gate64& G) {
  const int lane = threadIdx.x & 63;
  const float fpre = a.f_pre[tok0 + lane];
  const float lf = a.fgate_exp ? fpre : log_sigmoid(fpre);
  const float bc = scan_add(lf);
  const float u = a.i_pre[tok0 + lane] - bc;
  const float Mx = fmaxf(ms, scan_max(u));
  const float ML = __shfl(Mx, LC - 1, 64);
  G.u[lane] = u;
  G.M[lane] = Mx;
  G.m[lane] = bc + Mx;
  G.g[lane] = __expf(ms - Mx);
  G.w[lane] = __expf(u - ML);
}

__device__ __forceinline__ uint32_t pk2(float a, float b) { return cvt2(a, b); }

template <int DK, typename TO>
__global__ __launch_bounds__(NT4, 1) void bwd_rev_mfma_kernel(BwdArgs a) {
  constexpr int NXT = DK / 16;      // 16-row tiles of x (d_qk)
  constexpr int XPW = NXT / 4;      // x tiles per wave in the dq / dk products
  constexpr int NQT = DK / 64;
  __shared__ __align__(1024) char sQ[NQT * TB];
  __shared__ __align__(1024) char sK[NQT * TB];
  __shared__ __align__(1024) char sV[TB];
  __shared__ __align__(1024) char sWV[TB];
  __shared__ __align__(1024) char sR[TB];
  __shared__ __align__(1024) char sGR[TB];
  __shared__ __align__(1024) char sW[TB];
  __shared__ __align__(1024) char sDST[TB];   // (D (.) S)^T: [j][i]
  __shared__ __align__(1024) char sCX[DK * 128];   // [DK][64]: C~_s, then dC
  __shared__ __align__(1024) char sGD[16 * 128];   // rows 0, 1: g (.) dnq as bf16 hi / lo; rest 0
  __shared__ __align__(16) char sTW[4 * 2048];     // per wave: [32 x][16 b] bf16 hi, then lo
  __shared__ float sN[DK], sDn[DK];
  __shared__ float sRs[LC];
  __shared__ float sDnq[LC], sBeta[LC];
  __shared__ Gate64 G;
  __shared__ float sRed[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int ncb = static_cast<int>(a.dv / TVC);
  int64_t bh;
  int cb;
  head_block(a.B * a.H, ncb, bh, cb);
  const bool lead = cb == 0;
  const int dv = static_cast<int>(a.dv);
  const int64_t T = a.T;
  const int nc = static_cast<int>(T / LC);
  const int64_t nb = nc + 1;
  const int64_t BH = a.B * a.H;
  const int c0 = cb * TVC;

  // carried dC^T: tile xt holds dC^T[b = 16 wave + 4 g + e][x = 16 xt + l16]
  f32x4 dCt[NXT];
#pragma unroll
  for (int xt = 0; xt < NXT; ++xt) {
    dCt[xt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.dC1) {
      const float4 v4 = *reinterpret_cast<const float4*>(
          a.dC1 + (bh * DK + xt * 16 + l16) * dv + c0 + wave * 16 + 4 * g);
      dCt[xt] = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
  }
  for (int x = tid; x < DK; x += NT4) sDn[x] = a.dn1 ? a.dn1[bh * DK + x] : 0.0f;
  reinterpret_cast<uint2*>(sGD)[tid] = make_uint2(0u, 0u);

  // The chunk's q, k, v (own columns) and C~_s (the state pass's bf16 tile)
  // are loaded into registers one chunk ahead: the loads of chunk c - 1 are
  // in flight while chunk c is computed, and land in LDS at the next top.
  constexpr int NQK = LC * DK / 8 / NT4;    // 16-byte pieces of q (and of k) per thread
  constexpr int NVV = LC * TVC / 8 / NT4;
  constexpr int NCC = DK * TVC / 8 / NT4;
  // native vectors: HIP's uint4 struct would be copied through private memory
  u32x4 pq[NQK], pk[NQK], pv[NVV], pc[NCC];
  {
    const int64_t t0 = bh * T + static_cast<int64_t>(nc - 1) * LC;
    const bf16_t* q = static_cast<const bf16_t*>(a.q) + t0 * DK;
    const bf16_t* k = static_cast<const bf16_t*>(a.k) + t0 * DK;
#pragma unroll
    for (int p = 0; p < NQK; ++p) {
      const int e = tid + p * NT4;
      const int r = e / (DK / 8), col = (e % (DK / 8)) * 8;
      pq[p] = *reinterpret_cast<const u32x4*>(q + r * DK + col);
      pk[p] = *reinterpret_cast<const u32x4*>(k + r * DK + col);
    }
    const bf16_t* v = static_cast<const bf16_t*>(a.v) + t0 * dv + c0;
#pragma unroll
    for (int p = 0; p < NVV; ++p) {
      const int e = tid + p * NT4;
      pv[p] = *reinterpret_cast<const u32x4*>(v + static_cast<int64_t>(e >> 3) * dv + (e & 7) * 8);
    }
    const u32x4* Cs = reinterpret_cast<const u32x4*>(a.ws_Cb + ((bh * ncb + cb) * nc + (nc - 1)) * (DK * TVC));
#pragma unroll
    for (int p = 0; p < NCC; ++p) pc[p] = Cs[tid + p * NT4];
  }

  for (int c = nc - 1; c >= 0; --c) {
    const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
    const float ms = a.ws_m[bh * nb + c];
    __syncthreads();
    // ---- this chunk's operands into LDS; the next chunk's loads go out
    if (wave == 0) gate_scan64(a, tok0, ms, G);
#pragma unroll
    for (int p = 0; p < NQK; ++p) {
      const int e = tid + p * NT4;
      const int r = e / (DK / 8), col = (e % (DK / 8)) * 8;
      *reinterpret_cast<u32x4*>(sQ + (col >> 6) * TB + swz(r, col & 63)) = pq[p];
      *reinterpret_cast<u32x4*>(sK + (col >> 6) * TB + swz(r, col & 63)) = pk[p];
    }
#pragma unroll
    for (int p = 0; p < NVV; ++p) {
      const int e = tid + p * NT4;
      *reinterpret_cast<u32x4*>(sV + swz(e >> 3, (e & 7) * 8)) = pv[p];
    }
#pragma unroll
    for (int p = 0; p < NCC; ++p) *reinterpret_cast<u32x4*>(sCX + 16 * (tid + p * NT4)) = pc[p];
    // the next chunk's loads (chunk 0 fetches itself again: in bounds, unused)
    {
      const int64_t t0 = bh * T + static_cast<int64_t>(c > 0 ? c - 1 : 0) * LC;
      const bf16_t* q = static_cast<const bf16_t*>(a.q) + t0 * DK;
      const bf16_t* k = static_cast<const bf16_t*>(a.k) + t0 * DK;
#pragma unroll
      for (int p = 0; p < NQK; ++p) {
        const int e = tid + p * NT4;
        const int r = e / (DK / 8), col = (e % (DK / 8)) * 8;
        pq[p] = *reinterpret_cast<const u32x4*>(q + r * DK + col);
        pk[p] = *reinterpret_cast<const u32x4*>(k + r * DK + col);
      }
      const bf16_t* v = static_cast<const bf16_t*>(a.v) + t0 * dv + c0;
#pragma unroll
      for (int p = 0; p < NVV; ++p) {
        const int e = tid + p * NT4;
        pv[p] = *reinterpret_cast<const u32x4*>(v + static_cast<int64_t>(e >> 3) * dv + (e & 7) * 8);
      }
      const u32x4* Cs = reinterpret_cast<const u32x4*>(a.ws_Cb + ((bh * ncb + cb) * nc + (c > 0 ? c - 1 : 0)) * (DK * TVC));
#pragma unroll
      for (int p = 0; p < NCC; ++p) pc[p] = Cs[tid + p * NT4];
    }
    for (int x = tid; x < DK; x += NT4) sN[x] = a.ws_n[(bh * nb + c) * DK + x];
    if (tid < LC) sBeta[tid] = a.ws_beta[tok0 + tid];
    // this thread's dh, h and o~ (row tid / 4, 16 columns) for the r step,
    // loaded now so that their latency overlaps the score products
    uint4 pdh[2], ph[2], po[4];
    {
      const int64_t gi = (tok0 + (tid >> 2)) * dv + c0 + (tid & 3) * 16;
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        pdh[h8] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.dh) + gi + 8 * h8);
        if (a.o_pre) {
          ph[h8] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.h) + gi + 8 * h8);
          if (sizeof(TO) == 4) {
            po[2 * h8] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.o_pre) + gi + 8 * h8);
            po[2 * h8 + 1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.o_pre) + gi + 8 * h8 + 4);
          } else {
            po[h8] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.o_pre) + gi + 8 * h8);
          }
        }
      }
    }
    __syncthreads();

    // ---- S = Q K^T for query tile it = wave (all key tiles): D (.) S goes to
    // LDS transposed ([j][i]); its row sums stay inside the wave, so the
    // denominators and the r step below need no workgroup barrier
    {
      f32x4 acc[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const int x0 = 32 * ks;
        const bf16x8 A = rowfrag(wide(sQ, x0), wave * 16 + l16, (x0 & 63) + 8 * g);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          acc[jt] = mfma16x16x32(A, rowfrag(wide(sK, x0), jt * 16 + l16, (x0 & 63) + 8 * g), acc[jt]);
      }
      // lane: S[i = 16 wave + 4 g + e][j = 16 jt + l16]
      float Mi[4], rs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Mi[e] = G.M[wave * 16 + 4 * g + e];
        rs[e] = 0.0f;
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = jt * 16 + l16;
        const float uj = G.u[j];
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ds[e] = j <= wave * 16 + 4 * g + e ? __expf(uj - Mi[e]) * acc[jt][e] : 0.0f;
          rs[e] += ds[e];
        }
        *reinterpret_cast<uint2*>(sDST + swz(j, wave * 16 + 4 * g)) = make_uint2(pk2(ds[0], ds[1]), pk2(ds[2], ds[3]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) rs[e] += __shfl_xor(rs[e], o, 64);   // over the 16 j lanes
      }
      if (l16 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sRs[wave * 16 + 4 * g + e] = rs[e];
      }
    }
    // q . n~_s, the denominator and the normalizer gradient: the four threads
    // of token i = tid / 4 (the query rows of this wave) each hold them
    float den;
    {
      const int i = tid >> 2, qq = tid & 3;
      float s = 0.0f;
#pragma unroll
      for (int x8 = qq * (DK / 4); x8 < (qq + 1) * (DK / 4); x8 += 8) {
        const uint4 v8 = lds_ld16(wide(sQ, x8), swz(i, x8 & 63));
        s += bf_lo(v8.x) * sN[x8] + bf_hi(v8.x) * sN[x8 + 1] + bf_lo(v8.y) * sN[x8 + 2] +
             bf_hi(v8.y) * sN[x8 + 3] + bf_lo(v8.z) * sN[x8 + 4] + bf_hi(v8.z) * sN[x8 + 5] +
             bf_lo(v8.w) * sN[x8 + 6] + bf_hi(v8.w) * sN[x8 + 7];
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      // the row sums of this wave's rows were written by lanes of this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float nq = G.g[i] * s + sRs[i];
      const float floor_ = __expf(-G.m[i]);
      den = fmaxf(fabsf(nq), floor_);
      const float dnq = fabsf(nq) >= floor_ ? (nq >= 0.0f ? -sBeta[i] / den : sBeta[i] / den) : 0.0f;
      if (qq == 0) {
        sDnq[i] = dnq;
        if (lead) {   // the A operand of dn += sum_i g_i dnq_i q_i (hi and lo rows)
          const float gd = G.g[i] * dnq;
          const bf16_t hi = f2bf(gd);
          *reinterpret_cast<bf16_t*>(sGD + swz(0, i)) = hi;
          *reinterpret_cast<bf16_t*>(sGD + swz(1, i)) = f2bf(gd - bf2f(hi));
        }
      }
    }
    // ---- r, g r, w V (bf16 to LDS) and do~ (16 columns per thread)
    {
      const int i = tid >> 2, b0 = (tid & 3) * 16;
      const int64_t gi = (tok0 + i) * dv + c0 + b0;
      const float inv = 1.0f / den;
      const float gi_ = G.g[i], wi = G.w[i];
      uint32_t rp[8], gp[8], wp[8];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const uint4 d8 = pdh[h8];
        const uint4 v8 = lds_ld16(sV, swz(i, b0 + 8 * h8));
        float dhv[8] = {bf_lo(d8.x), bf_hi(d8.x), bf_lo(d8.y), bf_hi(d8.y),
                        bf_lo(d8.z), bf_hi(d8.z), bf_lo(d8.w), bf_hi(d8.w)};
        float vv[8] = {bf_lo(v8.x), bf_hi(v8.x), bf_lo(v8.y), bf_hi(v8.y),
                       bf_lo(v8.z), bf_hi(v8.z), bf_lo(v8.w), bf_hi(v8.w)};
        float gate[8];
        if (a.o_pre) {
          const uint4 h8v = ph[h8];
          const float hv[8] = {bf_lo(h8v.x), bf_hi(h8v.x), bf_lo(h8v.y), bf_hi(h8v.y),
                               bf_lo(h8v.z), bf_hi(h8v.z), bf_lo(h8v.w), bf_hi(h8v.w)};
          float ov[8];
          if (sizeof(TO) == 4) {
            const uint4 o0 = po[2 * h8], o1 = po[2 * h8 + 1];
            ov[0] = __uint_as_float(o0.x); ov[1] = __uint_as_float(o0.y);
            ov[2] = __uint_as_float(o0.z); ov[3] = __uint_as_float(o0.w);
            ov[4] = __uint_as_float(o1.x); ov[5] = __uint_as_float(o1.y);
            ov[6] = __uint_as_float(o1.z); ov[7] = __uint_as_float(o1.w);
          } else {
            const uint4 o8 = po[h8];
            ov[0] = bf_lo(o8.x); ov[1] = bf_hi(o8.x); ov[2] = bf_lo(o8.y); ov[3] = bf_hi(o8.y);
            ov[4] = bf_lo(o8.z); ov[5] = bf_hi(o8.z); ov[6] = bf_lo(o8.w); ov[7] = bf_hi(o8.w);
          }
          float dov[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            gate[e] = sigmoid_fast(ov[e]);
            dov[e] = dhv[e] * hv[e] * (1.0f - gate[e]);
          }
          float* dO = a.d_o + gi + 8 * h8;
          *reinterpret_cast<float4*>(dO) = make_float4(dov[0], dov[1], dov[2], dov[3]);
          *reinterpret_cast<float4*>(dO + 4) = make_float4(dov[4], dov[5], dov[6], dov[7]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gate[e] = 1.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float r0 = gate[e] * dhv[e] * inv, r1 = gate[e + 1] * dhv[e + 1] * inv;
          rp[4 * h8 + e / 2] = pk2(r0, r1);
          gp[4 * h8 + e / 2] = pk2(gi_ * r0, gi_ * r1);
          wp[4 * h8 + e / 2] = pk2(wi * vv[e], wi * vv[e + 1]);
        }
      }
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        *reinterpret_cast<uint4*>(sR + swz(i, b0 + 8 * h8)) = make_uint4(rp[4 * h8], rp[4 * h8 + 1], rp[4 * h8 + 2], rp[4 * h8 + 3]);
        *reinterpret_cast<uint4*>(sGR + swz(i, b0 + 8 * h8)) = make_uint4(gp[4 * h8], gp[4 * h8 + 1], gp[4 * h8 + 2], gp[4 * h8 + 3]);
        *reinterpret_cast<uint4*>(sWV + swz(i, b0 + 8 * h8)) = make_uint4(wp[4 * h8], wp[4 * h8 + 1], wp[4 * h8 + 2], wp[4 * h8 + 3]);
      }
    }
    __syncthreads();
    // ---- W = D (.) (R V^T + dnq): (R V^T)^T = V R^T for key tile jt = wave
    {
      f32x4 acc[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < TVC / 32; ++ks) {
        const bf16x8 A = rowfrag(sV, wave * 16 + l16, 32 * ks + 8 * g);
#pragma unroll
        for (int it = 0; it < 4; ++it)
          acc[it] = mfma16x16x32(A, rowfrag(sR, it * 16 + l16, 32 * ks + 8 * g), acc[it]);
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int i = it * 16 + l16;
        const float Mi = G.M[i], dq_ = lead ? sDnq[i] : 0.0f;
        float wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = wave * 16 + 4 * g + e;
          wv[e] = j <= i ? __expf(G.u[j] - Mi) * (acc[it][e] + dq_) : 0.0f;
        }
        *reinterpret_cast<uint2*>(sW + swz(i, wave * 16 + 4 * g)) = make_uint2(pk2(wv[0], wv[1]), pk2(wv[2], wv[3]));
      }
    }
    __syncthreads();
    // ---- dq^T = K^T W^T + C~_s (g R)^T (+ g dnq n~_s): x tiles of this wave x query tiles
    {
      f32x4 acc[XPW][4];
#pragma unroll
      for (int p = 0; p < XPW; ++p)
#pragma unroll
        for (int it = 0; it < 4; ++it) acc[p][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 Bw[4], Bg[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          Bw[it] = rowfrag(sW, it * 16 + l16, 32 * ks + 8 * g);
          Bg[it] = rowfrag(sGR, it * 16 + l16, 32 * ks + 8 * g);
        }
#pragma unroll
        for (int p = 0; p < XPW; ++p) {
          const int xt = wave * XPW + p;
          const bf16x8 Ak = colfrag(wide(sK, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq);
          const bf16x8 Ac = rowfrag(sCX, xt * 16 + l16, 32 * ks + 8 * g);
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            acc[p][it] = mfma16x16x32(Ak, Bw[it], acc[p][it]);
            acc[p][it] = mfma16x16x32(Ac, Bg[it], acc[p][it]);
          }
        }
      }
      float* out = a.ws_dq + ((static_cast<int64_t>(cb) * BH + bh) * T + static_cast<int64_t>(c) * LC) * DK;
#pragma unroll
      for (int p = 0; p < XPW; ++p) {
        const int x0 = (wave * XPW + p) * 16 + 4 * g;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int i = it * 16 + l16;
          const float f = lead ? G.g[i] * sDnq[i] : 0.0f;
          *reinterpret_cast<float4*>(out + i * DK + x0) =
              make_float4(acc[p][it][0] + f * sN[x0], acc[p][it][1] + f * sN[x0 + 1],
                          acc[p][it][2] + f * sN[x0 + 2], acc[p][it][3] + f * sN[x0 + 3]);
        }
      }
    }
    __syncthreads();   // C~_s is no longer read
    // ---- dC (carried, float32) to LDS as bf16 [x][b]
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt)
      *reinterpret_cast<uint2*>(sCX + swz(xt * 16 + l16, wave * 16 + 4 * g)) =
          make_uint2(pk2(dCt[xt][0], dCt[xt][1]), pk2(dCt[xt][2], dCt[xt][3]));
    __syncthreads();
    // ---- dk^T = Q^T W + dC (w V)^T (+ w dn), in two halves of the key tiles
    // (half the accumulators live at a time: the register budget is full)
    {
      float* out = a.ws_dk + ((static_cast<int64_t>(cb) * BH + bh) * T + static_cast<int64_t>(c) * LC) * DK;
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        f32x4 acc[XPW][2];
#pragma unroll
        for (int p = 0; p < XPW; ++p) {
          acc[p][0] = f32x4{0.f, 0.f, 0.f, 0.f};
          acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 Bw[2], Bv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int jt = 2 * jh + u;
            Bw[u] = colfrag(sW, 32 * ks, jt * 16, g, kr, kq);
            Bv[u] = rowfrag(sWV, jt * 16 + l16, 32 * ks + 8 * g);
          }
#pragma unroll
          for (int p = 0; p < XPW; ++p) {
            const int xt = wave * XPW + p;
            const bf16x8 Aq = colfrag(wide(sQ, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq);
            const bf16x8 Ac = rowfrag(sCX, xt * 16 + l16, 32 * ks + 8 * g);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              acc[p][u] = mfma16x16x32(Aq, Bw[u], acc[p][u]);
              acc[p][u] = mfma16x16x32(Ac, Bv[u], acc[p][u]);
            }
          }
        }
#pragma unroll
        for (int p = 0; p < XPW; ++p) {
          const int x0 = (wave * XPW + p) * 16 + 4 * g;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int j = (2 * jh + u) * 16 + l16;
            const float f = lead ? G.w[j] : 0.0f;
            *reinterpret_cast<float4*>(out + j * DK + x0) =
                make_float4(acc[p][u][0] + f * sDn[x0], acc[p][u][1] + f * sDn[x0 + 1],
                            acc[p][u][2] + f * sDn[x0 + 2], acc[p][u][3] + f * sDn[x0 + 3]);
          }
        }
      }
    }
    // ---- dv^T = R^T DS + w (dC^T K^T) for value tile bt = wave
    {
      f32x4 accA[4], accB[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        accA[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accB[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Ar = colfrag(sR, 32 * ks, wave * 16, g, kr, kq);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          accA[jt] = mfma16x16x32(Ar, rowfrag(sDST, jt * 16 + l16, 32 * ks + 8 * g), accA[jt]);
      }
      // dC^T K^T: this wave's 16 value columns of the carried dC (float32, in
      // its own registers) enter as a bf16 (hi, lo) pair, transposed 32 rows
      // at a time through a wave-private LDS tile.  A single bf16 copy of dC
      // costs up to ~2% of dv where the two terms of dv cancel.
      char* tw = sTW + wave * 2048;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const int x0 = 32 * ks;
#pragma unroll
        for (int t = 0; t < 2; ++t) {   // lane: dC^T[b = 4 g + e][x = x0 + 16 t + l16]
          const f32x4 v = dCt[2 * ks + t];
          const uint32_t h0 = pk2(v[0], v[1]), h1 = pk2(v[2], v[3]);
          const int off = (16 * t + l16) * 32 + g * 8;   // row x (32 bytes), columns b = 4 g ..
          *reinterpret_cast<uint2*>(tw + off) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(tw + 1024 + off) =
              make_uint2(pk2(v[0] - bf_lo(h0), v[1] - bf_hi(h0)), pk2(v[2] - bf_lo(h1), v[3] - bf_hi(h1)));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A[b = l16][x = 8 g + e]: transposed reads of rows 8 g + kr (+4), columns 4 kq
        const int ro = (8 * g + kr) * 32 + 8 * kq;
        const bf16x8 Ah = join(lds_tr(tw, ro), lds_tr(tw, ro + 4 * 32));
        const bf16x8 Al = join(lds_tr(tw + 1024, ro), lds_tr(tw + 1024, ro + 4 * 32));
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const bf16x8 Bk = rowfrag(wide(sK, x0), jt * 16 + l16, (x0 & 63) + 8 * g);
          accB[jt] = mfma16x16x32(Ah, Bk, accB[jt]);
          accB[jt] = mfma16x16x32(Al, Bk, accB[jt]);
        }
        // the next rows overwrite the tile only after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = jt * 16 + l16;
        const float wj = G.w[j];
        *reinterpret_cast<float4*>(a.d_v + (tok0 + j) * dv + c0 + wave * 16 + 4 * g) =
            make_float4(accA[jt][0] + wj * accB[jt][0], accA[jt][1] + wj * accB[jt][1],
                        accA[jt][2] + wj * accB[jt][2], accA[jt][3] + wj * accB[jt][3]);
      }
    }
    // ---- dC^T <- g_L dC^T + (g R)^T Q; in column block 0 also the
    // normalizer's sum_i g_i dnq_i q_i for this wave's x tiles (rows 0 + 1)
    f32x4 dnacc[XPW];
    {
      const float gL = G.g[LC - 1];
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt) dCt[xt] *= gL;
#pragma unroll
      for (int p = 0; p < XPW; ++p) dnacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Ag = colfrag(sGR, 32 * ks, wave * 16, g, kr, kq);
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt)
          dCt[xt] = mfma16x16x32(Ag, colfrag(wide(sQ, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), dCt[xt]);
        if (lead) {
          const bf16x8 Ad = rowfrag(sGD, l16, 32 * ks + 8 * g);
#pragma unroll
          for (int p = 0; p < XPW; ++p) {
            const int xt = wave * XPW + p;
            dnacc[p] = mfma16x16x32(Ad, colfrag(wide(sQ, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), dnacc[p]);
          }
        }
      }
    }
    __syncthreads();   // every read of sDn (dk) is done
    // ---- dn <- g_L dn + sum_i g_i dnq_i q_i (column block 0 only uses dn)
    if (lead && g == 0) {
      const float gL = G.g[LC - 1];
#pragma unroll
      for (int p = 0; p < XPW; ++p) {
        const int x = (wave * XPW + p) * 16 + l16;
        sDn[x] = gL * sDn[x] + (dnacc[p][0] + dnacc[p][1]);
      }
    }
  }
  // ---- the initial state's gradients and dm0's share
  __syncthreads();
  float part = 0.0f;
#pragma unroll
  for (int xt = 0; xt < NXT; ++xt) {
    const int64_t gi = (bh * DK + xt * 16 + l16) * dv + c0 + wave * 16 + 4 * g;
    if (a.dC0) *reinterpret_cast<float4*>(a.dC0 + gi) = make_float4(dCt[xt][0], dCt[xt][1], dCt[xt][2], dCt[xt][3]);
    if (a.C0) {
      const float4 c4 = *reinterpret_cast<const float4*>(a.C0 + gi);
      part += (dCt[xt][0] * c4.x + dCt[xt][1] * c4.y) + (dCt[xt][2] * c4.z + dCt[xt][3] * c4.w);
    }
  }
  if (lead) {
    for (int x = tid; x < DK; x += NT4) {
      if (a.dn0) a.dn0[bh * DK + x] = sDn[x];
      if (a.C0) part += sDn[x] * a.n0[bh * DK + x];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) sRed[wave] = part;
  __syncthreads();
  if (tid == 0) a.ws_dm0[static_cast<int64_t>(cb) * BH + bh] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
}

// Direct global -> LDS load of one chunk's k ([64][DK] bf16) into swizzled
// [64 x 64] tiles: each wave instruction fills 8 rows of one tile (lane l:
// row 8 rg + l / 8, 16-byte slot l % 8, which holds the global column piece
// slot ^ ((row / 2) % 8)).  Waves 0..3 issue DK / 32 instructions each.
template <int DK>
__device__ __forceinline__ void dma_k_chunk(const BwdArgs& a, int64_t tok0, int wave, int lane, char* dst) {
  constexpr int PER_WAVE = DK / 32;   // (DK / 64 tiles) x (8 row groups) / 4 waves
  const bf16_t* k = static_cast<const bf16_t*>(a.k) + tok0 * DK;
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q) {
    const int R = wave * PER_WAVE + q;
    const int qt = R >> 3, rg = R & 7;
    const int row = rg * 8 + (lane >> 3), slot = lane & 7;
    const bf16_t* src = k + static_cast<int64_t>(row) * DK + qt * 64 + 8 * (slot ^ ((row >> 1) & 7));
    dma16(src, static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                   static_cast<int>(lds_addr(dst + qt * TB + rg * 1024)))));
  }
}

// Chunk-boundary states for the reverse pass: (C~, n~, m) before every chunk
// and after the last, C~_{c+1} = g_L C~_c + K^T (w (.) V) and
// n~_{c+1} = g_L n~_c + K^T w.  Workgroup = (head, 64 value columns); the
// state is carried transposed in float32 registers (wave w: value columns
// 16 w..16 w + 15, all d_qk rows), w (.) V enters the MFMAs as a bf16 hi/lo
// pair (about 16 significant bits; k is exact), n~ is a float32 sum on the
// vector ALUs (column block 0 only, which also writes n~ and m).  k of the
// next chunk streams into the other half of a double-buffered LDS tile while
// the current one is used; v of the next chunk is held in registers.
template <int DK>
__global__ __launch_bounds__(NT4, 1) void bwd_states_mfma_kernel(BwdArgs a) {
  constexpr int NXT = DK / 16;
  constexpr int NQT = DK / 64;
  __shared__ __align__(1024) char sK[2][NQT * TB];
  __shared__ __align__(1024) char sWH[TB];
  __shared__ __align__(1024) char sWL[TB];
  __shared__ __align__(1024) char sWD[16 * 128];   // rows 0, 1: w as bf16 hi / lo; rest 0
  __shared__ Gate64 G;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int ncb = static_cast<int>(a.dv / TVC);
  int64_t bh;
  int cb;
  head_block(a.B * a.H, ncb, bh, cb);
  const int dv = static_cast<int>(a.dv);
  const int64_t T = a.T;
  const int nc = static_cast<int>(T / LC);   // >= 1
  const int64_t nb = nc + 1;
  const int c0 = cb * TVC;
  const bool lead = cb == 0;

  f32x4 Ct[NXT];
#pragma unroll
  for (int xt = 0; xt < NXT; ++xt) {
    Ct[xt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.C0) {
      const float4 v4 = *reinterpret_cast<const float4*>(
          a.C0 + (bh * DK + xt * 16 + l16) * dv + c0 + wave * 16 + 4 * g);
      Ct[xt] = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
  }
  // n~ lives in column block 0 only, in the lanes of group 0 of each wave:
  // lane l16 holds x = 16 (wave XPW + p) + l16
  constexpr int XPW = NXT / 4;
  float nx[XPW];
#pragma unroll
  for (int p = 0; p < XPW; ++p)
    nx[p] = (a.C0 && g == 0) ? a.n0[bh * DK + (wave * XPW + p) * 16 + l16] : 0.0f;
  reinterpret_cast<uint2*>(sWD)[tid] = make_uint2(0u, 0u);
  float m = a.C0 ? a.m0[bh] : 0.0f;

  // v rows tid / 4, columns c0 + 16 (tid % 4) .. + 15 of a chunk
  const bf16_t* vrow = static_cast<const bf16_t*>(a.v) + (bh * T + (tid >> 2)) * dv + c0 + (tid & 3) * 16;
  uint4 nv0 = *reinterpret_cast<const uint4*>(vrow);
  uint4 nv1 = *reinterpret_cast<const uint4*>(vrow + 8);
  dma_k_chunk<DK>(a, bh * T, wave, lane, sK[0]);

  for (int c = 0; c <= nc; ++c) {
    // every load issued so far (k of chunk c, v) has landed; the previous
    // chunk's reads of sK[(c + 1) & 1], sWH, sWL and G are done
    wait_vm<0>();
    __syncthreads();
    // the stored state at boundary c: before a chunk as this workgroup's
    // swizzled bf16 tile (the reverse pass's LDS image), after the last
    // chunk in float32
    if (c < nc) {
      char* tile = reinterpret_cast<char*>(a.ws_Cb + ((bh * ncb + cb) * nc + c) * (DK * TVC));
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt)
        *reinterpret_cast<uint2*>(tile + swz(xt * 16 + l16, wave * 16 + 4 * g)) =
            make_uint2(pk2(Ct[xt][0], Ct[xt][1]), pk2(Ct[xt][2], Ct[xt][3]));
    } else {
      float* wsC = a.ws_CT + bh * DK * dv + c0 + wave * 16 + 4 * g;
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt)
        *reinterpret_cast<float4*>(wsC + static_cast<int64_t>(xt * 16 + l16) * dv) =
            make_float4(Ct[xt][0], Ct[xt][1], Ct[xt][2], Ct[xt][3]);
    }
    if (lead) {
      if (g == 0) {
#pragma unroll
        for (int p = 0; p < XPW; ++p) a.ws_n[(bh * nb + c) * DK + (wave * XPW + p) * 16 + l16] = nx[p];
      }
      if (tid == 0) a.ws_m[bh * nb + c] = m;
    }
    if (c == nc) break;
    const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
    const char* kc = sK[c & 1];
    if (c + 1 < nc) dma_k_chunk<DK>(a, tok0 + LC, wave, lane, sK[(c + 1) & 1]);
    if (wave == 0) gate_scan64(a, tok0, m, G);
    const uint4 v0 = nv0, v1 = nv1;
    if (c + 1 < nc) {
      nv0 = *reinterpret_cast<const uint4*>(vrow + static_cast<int64_t>(c + 1) * LC * dv);
      nv1 = *reinterpret_cast<const uint4*>(vrow + static_cast<int64_t>(c + 1) * LC * dv + 8);
    }
    __syncthreads();
    {
      const int j = tid >> 2, b0 = (tid & 3) * 16;
      const float wj = G.w[j];
      const float x[16] = {bf_lo(v0.x), bf_hi(v0.x), bf_lo(v0.y), bf_hi(v0.y), bf_lo(v0.z), bf_hi(v0.z),
                           bf_lo(v0.w), bf_hi(v0.w), bf_lo(v1.x), bf_hi(v1.x), bf_lo(v1.y), bf_hi(v1.y),
                           bf_lo(v1.z), bf_hi(v1.z), bf_lo(v1.w), bf_hi(v1.w)};
      uint32_t hp[8], lp[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float y0 = wj * x[e], y1 = wj * x[e + 1];
        const uint32_t h2 = pk2(y0, y1);
        hp[e / 2] = h2;
        lp[e / 2] = pk2(y0 - bf_lo(h2), y1 - bf_hi(h2));
      }
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        *reinterpret_cast<uint4*>(sWH + swz(j, b0 + 8 * h8)) = make_uint4(hp[4 * h8], hp[4 * h8 + 1], hp[4 * h8 + 2], hp[4 * h8 + 3]);
        *reinterpret_cast<uint4*>(sWL + swz(j, b0 + 8 * h8)) = make_uint4(lp[4 * h8], lp[4 * h8 + 1], lp[4 * h8 + 2], lp[4 * h8 + 3]);
      }
    }
    const float gL = G.g[LC - 1];
    if (lead && tid < LC) {   // the A operand of n~ += sum_j w_j k_j (hi and lo rows)
      const float wj = G.w[tid];
      const bf16_t hi = f2bf(wj);
      *reinterpret_cast<bf16_t*>(sWD + swz(0, tid)) = hi;
      *reinterpret_cast<bf16_t*>(sWD + swz(1, tid)) = f2bf(wj - bf2f(hi));
    }
    __syncthreads();
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt) Ct[xt] *= gL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 Ah = colfrag(sWH, 32 * ks, wave * 16, g, kr, kq);
      const bf16x8 Al = colfrag(sWL, 32 * ks, wave * 16, g, kr, kq);
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt) {
        const bf16x8 Bk = colfrag(wide(kc, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq);
        Ct[xt] = mfma16x16x32(Ah, Bk, Ct[xt]);
        Ct[xt] = mfma16x16x32(Al, Bk, Ct[xt]);
      }
    }
    if (lead) {   // n~ <- g_L n~ + K^T w for this wave's x tiles (D rows 0 + 1)
      f32x4 nacc[XPW];
#pragma unroll
      for (int p = 0; p < XPW; ++p) nacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Aw = rowfrag(sWD, l16, 32 * ks + 8 * g);
#pragma unroll
        for (int p = 0; p < XPW; ++p) {
          const int xt = wave * XPW + p;
          nacc[p] = mfma16x16x32(Aw, colfrag(wide(kc, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), nacc[p]);
        }
      }
#pragma unroll
      for (int p = 0; p < XPW; ++p) nx[p] = gL * nx[p] + (nacc[p][0] + nacc[p][1]);
    }
    m = G.m[LC - 1];
  }
}

template <int DK>
hipError_t launch_states_dk(const BwdArgs& a, hipStream_t st) {
  bwd_states_mfma_kernel<DK><<<static_cast<unsigned>(a.B * a.H * (a.dv / TVC)), NT4, 0, st>>>(a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const BwdArgs& a, hipStream_t st) {
  const unsigned wgs = static_cast<unsigned>(a.B * a.H * (a.dv / TVC));
  if (a.o_mode == O_BF16) bwd_rev_mfma_kernel<DK, bf16_t><<<wgs, NT4, 0, st>>>(a);
  else bwd_rev_mfma_kernel<DK, float><<<wgs, NT4, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool bwd_mfma_supported(const BwdArgs& a) {
  return a.qkv_bf16 && a.L == LC && a.T % LC == 0 && a.dv % TVC == 0 &&
         (a.dqk == 64 || a.dqk == 128 || a.dqk == 256);
}

hipError_t launch_bwd_states_mfma(const BwdArgs& a, hipStream_t st) {
  switch (a.dqk) {
    case 64: return launch_states_dk<64>(a, st);
    case 128: return launch_states_dk<128>(a, st);
    default: return launch_states_dk<256>(a, st);
  }
}

hipError_t launch_bwd_rev_mfma(const BwdArgs& a, hipStream_t st) {
  switch (a.dqk) {
    case 64: return launch_dk<64>(a, st);
    case 128: return launch_dk<128>(a, st);
    default: return launch_dk<256>(a, st);
  }
}

}  // namespace mlstm
