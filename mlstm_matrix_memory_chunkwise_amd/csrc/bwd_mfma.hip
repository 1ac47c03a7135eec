// State, reverse and dq/dk passes of the chunkwise backward on bf16 MFMA
// (gfx950): chunk 64, d_qk in {64, 128, 256}, d_v a multiple of 64, bf16
// q/k/v/h/dh.
//
// The same gradient as the float32 passes in bwd.hip (the derivative of the
// forward pass of the xLSTM post, llms.blog, section 3 "Associative Matrix
// Cell State" and "The Parallel Dual Form", with the running maximum of
// section 2 "The Normalizer State and Numerical Stabilization"), with every
// matrix product on 16x16x32 MFMAs.  Per chunk of 64 tokens, with the stored
// state (C~_s, n~_s, m_s) and the carried memory gradient dC, the reverse
// pass (one workgroup per head and 64 value columns, sequential over the
// chunks) forms
//
//   S = Q K^T,  DS = D (.) S              (masked; stored transposed, bf16;
//                                          row sums in float32)
//   r = sigmoid(o~) dh / den,  g r        (bf16 in LDS; r also to HBM)
//   dv^T = R^T DS + w (dC^T K^T)          (dC as a bf16 hi / lo pair)
//   dC^T <- g_L dC^T + (g R)^T Q,  dn <- g_L dn + sum_i g_i dnq_i q_i
//
// and stores, per chunk, the dC and dn it enters with (the gradient at the
// chunk's end) and dnq.  The dq/dk pass then runs on every (head, chunk,
// d_qk slice) at once, over all of d_v:
//
//   dS = R V^T,  W = D (.) (dS + dnq)     (float32 sum over d_v, bf16 W)
//   dq^T = g (C~_s R^T) + K^T W^T + g dnq n~_s
//   dk^T = w (dC V^T)   + Q^T W   + w dn
//
// so that no workgroup writes a partial sum over its own value columns.
//
// Operands are read from swizzled [rows][64] bf16 LDS tiles either as row
// fragments (8 consecutive columns, ds_read_b128) or as transposed column
// fragments (8 consecutive rows, two ds_read_b64_tr_b16), both in natural
// index order; the dq/dk pass reads its d_v-contracted operands straight
// from HBM as 16-byte fragments.  The memory gradient is carried transposed
// in float32 registers (dC^T tiles, one 16-column block per wave), which
// makes its bf16 copy a run of 4 consecutive columns per lane.  The products
// round their other operands to bf16 (accumulation stays float32); q, k, v
// are exact.  Vectors that meet a matrix in float32 precision (dn's g dnq,
// the state pass's w (.) V and w) enter as bf16 hi / lo pairs.
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

// the same from gate values already in registers (lane = token)
__device__ __forceinline__ void gate_scan64_v(float fpre, float ipre, int fgate_exp, float ms, Gate64& G) {
  const int lane = threadIdx.x & 63;
  const float lf = fgate_exp ? fpre : log_sigmoid(fpre);
  const float bc = scan_add(lf);
  const float u = ipre - bc;
  const float Mx = fmaxf(ms, scan_max(u));
  const float ML = __shfl(Mx, LC - 1, 64);
  G.u[lane] = u;
  G.M[lane] = Mx;
  G.m[lane] = bc + Mx;
  G.g[lane] = __expf(ms - Mx);
  G.w[lane] = __expf(u - ML);
}

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

constexpr int NT8 = 512;           // 8 waves

// The reverse pass: one workgroup of 8 waves per (head, 64 value columns),
// two roles.  Waves 0-3 ("score" waves, one query tile / 16 columns each)
// form everything of a chunk that does not depend on the carried dC: S, the
// denominators and dnq, r, g r and do~.  Waves 4-7 ("memory" waves, 16 value
// columns each) own dC^T in float32 registers; while the score waves work
// they store dC at the chunk's end to HBM and form w (.) (dC^T K^T) (into
// LDS); after the chunk's third barrier they update dC and dn while the score
// waves finish dv = R^T DS + w (.) (dC^T K^T).  Each SIMD runs one wave of
// each role, and the dC-only work of a chunk overlaps its score work.  The roles run separate loops with the same
// barrier sequence (one before the loop when dC1 is given, three per chunk,
// two after it), so that the registers of one role's values are free in the
// other's code.
template <int DK, typename TO>
__global__ __launch_bounds__(NT8, 1) void bwd_rev_mfma_kernel(BwdArgs a) {
  constexpr int NXT = DK / 16;      // 16-row tiles of x (d_qk)
  constexpr int XPW = NXT / 4;      // x tiles per memory wave in the dn product
  constexpr int NQT = DK / 64;
  constexpr int KH = DK / 64;       // 32-row blocks of x per half of d_qk
  __shared__ __align__(1024) char sQ[NQT * TB];
  __shared__ __align__(1024) char sK[NQT * TB];
  __shared__ __align__(1024) char sR[TB];
  __shared__ __align__(1024) char sGR[TB];
  __shared__ __align__(1024) char sDST[TB];   // (D (.) S)^T: [j][i]
  // [DK][64]: dC at the chunk's end (bf16), written by the memory waves at
  // the chunk's top.  Memory wave v then copies rows 16 KH v .. + 16 KH - 1
  // (bytes KH 2048 v ..) to HBM and reuses them for its transposes of dC (two
  // halves of [32 x][16 b] hi / lo tiles): every access after the second
  // barrier is private to one wave.
  __shared__ __align__(1024) char sCX[DK * 128];
  __shared__ __align__(1024) char sGD[16 * 128];   // rows 0, 1: g (.) dnq as bf16 hi / lo; rest 0
  __shared__ __align__(16) float sDVM[LC][TVC + 4];  // w (.) (dC^T K^T) as [token j][value column b]
  __shared__ float sN[DK], sDn[DK];
  __shared__ float sRs[LC];
  __shared__ float sBeta[LC];
  __shared__ Gate64 G;
  __shared__ float sRed[8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int rw = wave & 3;          // the wave's index within its role
  const int rtid = tid & (NT4 - 1); // the thread's index within its role
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

  for (int x = tid; x < DK; x += NT8) sDn[x] = a.dn1 ? a.dn1[bh * DK + x] : 0.0f;
  if (tid < 16 * 128 / 8) reinterpret_cast<uint2*>(sGD)[tid] = make_uint2(0u, 0u);

  // The chunk's q and k are loaded into the score waves' registers after
  // the previous chunk's third barrier: they are in flight while the memory
  // waves finish that chunk (the score waves are idle then), and land in LDS
  // at the next top.
  constexpr int NQK = LC * DK / 8 / NT4;
  // native vectors: HIP's uint4 struct would be copied through private memory
  u32x4 pq[NQK], pk[NQK];
  auto load_qk = [&](int cc) {
    const int64_t t0 = bh * T + static_cast<int64_t>(cc) * LC;
    const bf16_t* q = static_cast<const bf16_t*>(a.q) + t0 * DK;
    const bf16_t* k = static_cast<const bf16_t*>(a.k) + t0 * DK;
#pragma unroll
    for (int p = 0; p < NQK; ++p) {
      const int e = rtid + p * NT4;
      const int r = e / (DK / 8), col = (e % (DK / 8)) * 8;
      pq[p] = *reinterpret_cast<const u32x4*>(q + r * DK + col);
      pk[p] = *reinterpret_cast<const u32x4*>(k + r * DK + col);
    }
  };
  auto store_qk = [&]() {
#pragma unroll
    for (int p = 0; p < NQK; ++p) {
      const int e = rtid + p * NT4;
      const int r = e / (DK / 8), col = (e % (DK / 8)) * 8;
      *reinterpret_cast<u32x4*>(sQ + (col >> 6) * TB + swz(r, col & 63)) = pq[p];
      *reinterpret_cast<u32x4*>(sK + (col >> 6) * TB + swz(r, col & 63)) = pk[p];
    }
  };
  // dn at the chunk's end (column block 0), for the dq/dk pass
  auto store_dn = [&](int c) {
    if (lead) {
      for (int x = tid; x < DK; x += NT8) a.ws_dn[(bh * nc + c) * DK + x] = sDn[x];
    }
  };
  // the workgroup's sum of one value per wave, into *out (thread 0)
  auto wg_sum = [&](float part, float* out) {
    part = wave_sum(part);
    if (lane == 0) sRed[wave] = part;
    __syncthreads();
    if (tid == 0) {
      float s8 = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) s8 += sRed[w];
      *out = s8;
    }
  };
  if (wave < 4) {
    // ================= score waves
    // the small per-chunk inputs (gates, m, n~ at the chunk start, beta) are
    // read one chunk ahead into registers, so that no global latency sits
    // between a chunk's first barrier and its gate scan
    constexpr int NNR = (DK + NT4 - 1) / NT4;
    float pf_f, pf_i, pf_ms, pf_b, pf_n[NNR];
    auto prefetch_small = [&](int cc) {
      const int64_t t0 = bh * T + static_cast<int64_t>(cc) * LC;
      pf_f = a.f_pre[t0 + lane];
      pf_i = a.i_pre[t0 + lane];
      pf_ms = a.ws_m[bh * nb + cc];
      pf_b = a.ws_beta[t0 + (rtid & (LC - 1))];
#pragma unroll
      for (int r = 0; r < NNR; ++r) {
        const int x = rtid + r * NT4;
        pf_n[r] = x < DK ? a.ws_n[(bh * nb + cc) * DK + x] : 0.0f;
      }
    };
    prefetch_small(nc - 1);
    load_qk(nc - 1);
    // final-state term: <dn1, n~_T> (column block 0)
    if (a.dC1) {
      float part = 0.0f;
      if (lead) {
        for (int x = rtid; x < DK; x += NT4) part += a.dn1[bh * DK + x] * a.ws_n[(bh * nb + nc) * DK + x];
      }
      wg_sum(part, a.ws_kend + static_cast<int64_t>(cb) * BH + bh);   // barrier
    }
    for (int c = nc - 1; c >= 0; --c) {
      const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
      __syncthreads();   // (1)
      if (wave == 0) gate_scan64_v(pf_f, pf_i, a.fgate_exp, pf_ms, G);
#pragma unroll
      for (int r = 0; r < NNR; ++r) {
        const int x = rtid + r * NT4;
        if (x < DK) sN[x] = pf_n[r];
      }
      if (rtid < LC) sBeta[rtid] = pf_b;
      store_qk();
      store_dn(c);
      prefetch_small(c > 0 ? c - 1 : 0);   // (chunk 0 reads itself again: unused)
      // this thread's dh, h and o~ (row rtid / 4, 16 columns) for the r step,
      // loaded now so that their latency overlaps the score products
      uint4 pdh[2], ph[2], po[4];
      {
        const int64_t gi = (tok0 + (rtid >> 2)) * dv + c0 + (rtid & 3) * 16;
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
      __syncthreads();   // (2)
      // ---- S = Q K^T for query tile it = rw (all key tiles): D (.) S goes
      // to LDS transposed ([j][i]); its row sums stay inside the wave, so the
      // denominators and the r step below need no workgroup barrier
      {
        f32x4 acc[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const int x0 = 32 * ks;
          const bf16x8 A = rowfrag(wide(sQ, x0), rw * 16 + l16, (x0 & 63) + 8 * g);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            acc[jt] = mfma16x16x32(A, rowfrag(wide(sK, x0), jt * 16 + l16, (x0 & 63) + 8 * g), acc[jt]);
        }
        // lane: S[i = 16 rw + 4 g + e][j = 16 jt + l16]
        float Mi[4], rs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Mi[e] = G.M[rw * 16 + 4 * g + e];
          rs[e] = 0.0f;
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int j = jt * 16 + l16;
          const float uj = G.u[j];
          float ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ds[e] = j <= rw * 16 + 4 * g + e ? __expf(uj - Mi[e]) * acc[jt][e] : 0.0f;
            rs[e] += ds[e];
          }
          *reinterpret_cast<uint2*>(sDST + swz(j, rw * 16 + 4 * g)) = make_uint2(pk2(ds[0], ds[1]), pk2(ds[2], ds[3]));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int o = 8; o > 0; o >>= 1) rs[e] += __shfl_xor(rs[e], o, 64);   // over the 16 j lanes
        }
        if (l16 == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sRs[rw * 16 + 4 * g + e] = rs[e];
        }
      }
      // q . n~_s, the denominator and the normalizer gradient: the four
      // threads of token i = rtid / 4 (the query rows of this wave) each hold them
      float den;
      {
        const int i = rtid >> 2, qq = rtid & 3;
        float s = 0.0f;
        // thread qq takes the 16-byte chunks 4 it + qq of row i: the four
        // threads of a token read four chunks of one tile row at a time
#pragma unroll
        for (int it = 0; it < DK / 32; ++it) {
          const int x8 = 32 * it + 8 * qq;
          const uint4 v8 = lds_ld16(wide(sQ, 32 * it), swz(i, x8 & 63));
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
        if (qq == 0 && lead) {
          a.ws_dnq[tok0 + i] = dnq;
          // the A operand of dn += sum_i g_i dnq_i q_i (hi and lo rows)
          const float gd = G.g[i] * dnq;
          const bf16_t hi = f2bf(gd);
          *reinterpret_cast<bf16_t*>(sGD + swz(0, i)) = hi;
          *reinterpret_cast<bf16_t*>(sGD + swz(1, i)) = f2bf(gd - bf2f(hi));
        }
      }
      // ---- r and g r (bf16 to LDS; r also to HBM for the dq/dk pass) and
      // do~ (16 columns per thread)
      {
        const int i = rtid >> 2, b0 = (rtid & 3) * 16;
        const int64_t gi = (tok0 + i) * dv + c0 + b0;
        const float inv = 1.0f / den;
        const float gi_ = G.g[i];
        uint32_t rp[8], gp[8];
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const uint4 d8 = pdh[h8];
          float dhv[8] = {bf_lo(d8.x), bf_hi(d8.x), bf_lo(d8.y), bf_hi(d8.y),
                          bf_lo(d8.z), bf_hi(d8.z), bf_lo(d8.w), bf_hi(d8.w)};
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
          }
        }
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const u32x4 r4 = {rp[4 * h8], rp[4 * h8 + 1], rp[4 * h8 + 2], rp[4 * h8 + 3]};
          *reinterpret_cast<u32x4*>(sR + swz(i, b0 + 8 * h8)) = r4;
          *reinterpret_cast<u32x4*>(a.ws_R + gi + 8 * h8) = r4;
          *reinterpret_cast<uint4*>(sGR + swz(i, b0 + 8 * h8)) = make_uint4(gp[4 * h8], gp[4 * h8 + 1], gp[4 * h8 + 2], gp[4 * h8 + 3]);
        }
      }
      __syncthreads();   // (3)
      load_qk(c > 0 ? c - 1 : 0);   // (chunk 0 fetches itself again: in bounds, unused)
      // ---- dv^T = R^T DS + w (dC^T K^T) for value tile rw (the memory
      // waves' term from LDS)
      {
        f32x4 accA[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) accA[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 Ar = colfrag(sR, 32 * ks, rw * 16, g, kr, kq);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            accA[jt] = mfma16x16x32(Ar, rowfrag(sDST, jt * 16 + l16, 32 * ks + 8 * g), accA[jt]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int j = jt * 16 + l16;
          const float4 m4 = *reinterpret_cast<const float4*>(&sDVM[j][rw * 16 + 4 * g]);
          *reinterpret_cast<float4*>(a.d_v + (tok0 + j) * dv + c0 + rw * 16 + 4 * g) =
              make_float4(accA[jt][0] + m4.x, accA[jt][1] + m4.y, accA[jt][2] + m4.z, accA[jt][3] + m4.w);
        }
      }
    }
    __syncthreads();
    float part = 0.0f;
    if (lead) {
      for (int x = rtid; x < DK; x += NT4) {
        if (a.dn0) a.dn0[bh * DK + x] = sDn[x];
        if (a.C0) part += sDn[x] * a.n0[bh * DK + x];
      }
    }
    wg_sum(part, a.ws_dm0 + static_cast<int64_t>(cb) * BH + bh);   // barrier
  } else {
    // ================= memory waves
    // (their dC chain is the sequential critical path: issue ahead of the
    // score wave on the same SIMD; measured 0.5% faster per pass)
    __builtin_amdgcn_s_setprio(2);
    // carried dC^T: tile xt holds dC^T[b = 16 rw + 4 g + e][x = 16 xt + l16]
    f32x4 dCt[NXT];
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt) {
      dCt[xt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a.dC1) {
        const float4 v4 = *reinterpret_cast<const float4*>(
            a.dC1 + (bh * DK + xt * 16 + l16) * dv + c0 + rw * 16 + 4 * g);
        dCt[xt] = f32x4{v4.x, v4.y, v4.z, v4.w};
      }
    }
    // final-state term: <dC1, C~_T> over this workgroup's columns
    if (a.dC1) {
      float part = 0.0f;
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt) {
        const float4 c4 = *reinterpret_cast<const float4*>(
            a.ws_CT + (bh * DK + xt * 16 + l16) * dv + c0 + rw * 16 + 4 * g);
        part += (dCt[xt][0] * c4.x + dCt[xt][1] * c4.y) + (dCt[xt][2] * c4.z + dCt[xt][3] * c4.w);
      }
      wg_sum(part, nullptr);   // barrier (the score waves' thread 0 writes the sum)
    }
    char* tw = sCX + rw * (KH * 2048);
    // row x of a transposition tile sits at row x ^ 4 when x / 8 is odd: a
    // transposed read takes rows 8 g + 0..3 (or 4..7) in lane group g, and
    // this puts groups g and g + 1 on different halves of the banks
    auto trow = [](int x) { return x ^ (((x >> 3) & 1) << 2); };
    for (int c = nc - 1; c >= 0; --c) {
      const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
      __syncthreads();   // (1)
      // dC at this chunk's end (bf16, [x][b]) for its copy to HBM
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt)
        *reinterpret_cast<uint2*>(sCX + swz(xt * 16 + l16, rw * 16 + 4 * g)) =
            make_uint2(pk2(dCt[xt][0], dCt[xt][1]), pk2(dCt[xt][2], dCt[xt][3]));
      store_dn(c);
      __syncthreads();   // (2)
      // ---- this wave's rows of the dC tile to HBM, in the stored states'
      // tile order
      {
        u32x4* dst = reinterpret_cast<u32x4*>(a.ws_dCb + ((bh * ncb + cb) * nc + c) * (DK * TVC) + rw * (KH * 1024));
#pragma unroll
        for (int p = 0; p < KH * 2; ++p)
          dst[lane + 64 * p] = *reinterpret_cast<const u32x4*>(tw + 16 * (lane + 64 * p));
      }
      // ---- dC^T K^T for value tile rw: this wave's 16 value columns of the
      // carried dC (float32) enter as a bf16 (hi, lo) pair, transposed
      // through its rows of sCX half of d_qk at a time (a wave-level sync
      // before each half's writes, after the copy above or the first half's
      // reads, and between writes and reads).  A single bf16 copy of dC costs
      // up to ~2% of dv where the two terms of dv cancel.
      f32x4 accB[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) accB[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
          const int ks = hf * KH + kh;
#pragma unroll
          for (int t = 0; t < 2; ++t) {   // lane: dC^T[b = 4 g + e][x = 32 ks + 16 t + l16]
            const f32x4 v = dCt[2 * ks + t];
            const uint32_t h0 = pk2(v[0], v[1]), h1 = pk2(v[2], v[3]);
            const int off = kh * 2048 + trow(16 * t + l16) * 32 + g * 8;   // row x (32 bytes), columns b = 4 g ..
            *reinterpret_cast<uint2*>(tw + off) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(tw + 1024 + off) =
                make_uint2(pk2(v[0] - bf_lo(h0), v[1] - bf_hi(h0)), pk2(v[2] - bf_lo(h1), v[3] - bf_hi(h1)));
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
          const int x0 = 32 * (hf * KH + kh);
          // A[b = l16][x = 8 g + e]: transposed reads of rows 8 g + kr (+4), columns 4 kq
          const int r0 = kh * 2048 + trow(8 * g + kr) * 32 + 8 * kq;
          const int r1 = kh * 2048 + trow(8 * g + 4 + kr) * 32 + 8 * kq;
          const bf16x8 Ah = join(lds_tr(tw, r0), lds_tr(tw, r1));
          const bf16x8 Al = join(lds_tr(tw + 1024, r0), lds_tr(tw + 1024, r1));
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            const bf16x8 Bk = rowfrag(wide(sK, x0), jt * 16 + l16, (x0 & 63) + 8 * g);
            accB[jt] = mfma16x16x32(Ah, Bk, accB[jt]);
            accB[jt] = mfma16x16x32(Al, Bk, accB[jt]);
          }
        }
      }
      // lane: (dC^T K^T)^T[j = 16 jt + l16][b = 16 rw + 4 g + e], scaled by w_j
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = jt * 16 + l16;
        const float wj = G.w[j];
        *reinterpret_cast<float4*>(&sDVM[j][rw * 16 + 4 * g]) =
            make_float4(wj * accB[jt][0], wj * accB[jt][1], wj * accB[jt][2], wj * accB[jt][3]);
      }
      __syncthreads();   // (3)
      // ---- dC^T <- g_L dC^T + (g R)^T Q; in column block 0 also the
      // normalizer's sum_i g_i dnq_i q_i for this wave's x tiles (rows 0 + 1)
      f32x4 dnacc[XPW];
      const float gL = G.g[LC - 1];
#pragma unroll
      for (int xt = 0; xt < NXT; ++xt) dCt[xt] *= gL;
#pragma unroll
      for (int p = 0; p < XPW; ++p) dnacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Ag = colfrag(sGR, 32 * ks, rw * 16, g, kr, kq);
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt)
          dCt[xt] = mfma16x16x32(Ag, colfrag(wide(sQ, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), dCt[xt]);
        if (lead) {
          const bf16x8 Ad = rowfrag(sGD, l16, 32 * ks + 8 * g);
#pragma unroll
          for (int p = 0; p < XPW; ++p) {
            const int xt = rw * XPW + p;
            dnacc[p] = mfma16x16x32(Ad, colfrag(wide(sQ, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), dnacc[p]);
          }
        }
      }
      // ---- dn <- g_L dn + sum_i g_i dnq_i q_i (column block 0 only; sDn was
      // last read at this chunk's top, before the second barrier)
      if (lead && g == 0) {
#pragma unroll
        for (int p = 0; p < XPW; ++p) {
          const int x = (rw * XPW + p) * 16 + l16;
          sDn[x] = gL * sDn[x] + (dnacc[p][0] + dnacc[p][1]);
        }
      }
    }
    // ---- the initial state's gradients and dm0's share
    __syncthreads();
    float part = 0.0f;
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt) {
      const int64_t gi = (bh * DK + xt * 16 + l16) * dv + c0 + rw * 16 + 4 * g;
      if (a.dC0) *reinterpret_cast<float4*>(a.dC0 + gi) = make_float4(dCt[xt][0], dCt[xt][1], dCt[xt][2], dCt[xt][3]);
      if (a.C0) {
        const float4 c4 = *reinterpret_cast<const float4*>(a.C0 + gi);
        part += (dCt[xt][0] * c4.x + dCt[xt][1] * c4.y) + (dCt[xt][2] * c4.z + dCt[xt][3] * c4.w);
      }
    }
    wg_sum(part, nullptr);   // barrier (the score waves' thread 0 writes the sum)
  }
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

// Direct global -> LDS load of one chunk's k for the 8-wave state pass: the
// same tiles and lane layout as dma_k_chunk, DK / 64 instructions per wave.
template <int DK>
__device__ __forceinline__ void dma_k_chunk8(const BwdArgs& a, int64_t tok0, int wave, int lane, char* dst) {
  constexpr int PER_WAVE = DK / 64;   // (DK / 64 tiles) x (8 row groups) / 8 waves
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
// n~_{c+1} = g_L n~_c + K^T w.  Workgroup = (head, 64 value columns), 8
// waves, two per SIMD; the state is carried transposed in float32 registers
// (wave w: value columns 16 (w % 4)..+15, half of the d_qk rows by w / 4),
// w (.) V enters the MFMAs as a bf16 hi/lo pair (about 16 significant bits;
// k is exact), n~ on MFMA with w as a hi/lo pair (column block 0 only, which
// also writes n~ and m).  Every wave runs the gate scan itself (DPP scans),
// one chunk ahead: at chunk c it scans the gates of chunk c + 1 (loaded at
// the top of chunk c) and writes chunk c + 1's w (.) V and w into the LDS
// buffers of that chunk's parity, so the loop has one barrier per chunk.  k
// of the next chunk streams into the other half of a double-buffered LDS
// tile while the current one is used.
template <int DK>
__global__ __launch_bounds__(NT8, 1) void bwd_states_mfma_kernel(BwdArgs a) {
  constexpr int NXT = DK / 16;
  constexpr int NXH = NXT / 2;            // x tiles per wave
  constexpr int NXN = (NXT + 7) / 8;      // n~ x tiles per wave (column block 0)
  constexpr int NQT = DK / 64;
  __shared__ __align__(1024) char sK[2][NQT * TB];
  __shared__ __align__(1024) char sWH[2][TB];          // w (.) V, bf16 hi, by chunk parity
  __shared__ __align__(1024) char sWL[2][TB];          // ... and lo
  __shared__ __align__(1024) char sWD[2][16 * 128];    // rows 0, 1: w as bf16 hi / lo; rest 0

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int cg = wave & 3, rh = wave >> 2;
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

  // Ct[t]: C~^T[b = 16 cg + 4 g + e][x = 16 (rh NXH + t) + l16]
  f32x4 Ct[NXH];
#pragma unroll
  for (int t = 0; t < NXH; ++t) {
    Ct[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.C0) {
      const float4 v4 = *reinterpret_cast<const float4*>(
          a.C0 + (bh * DK + (rh * NXH + t) * 16 + l16) * dv + c0 + cg * 16 + 4 * g);
      Ct[t] = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
  }
  // n~ (column block 0): lane l16 of group 0 holds x = 16 (wave NXN + p) + l16
  float nx[NXN];
#pragma unroll
  for (int p = 0; p < NXN; ++p) {
    const int xt = wave * NXN + p;
    nx[p] = (a.C0 && g == 0 && xt < NXT) ? a.n0[bh * DK + xt * 16 + l16] : 0.0f;
  }
  for (int x = tid; x < 2 * 16 * 128 / 8; x += NT8) reinterpret_cast<uint2*>(&sWD[0][0])[x] = make_uint2(0u, 0u);
  float m = a.C0 ? a.m0[bh] : 0.0f;   // m before the chunk (every wave keeps it)

  // this thread's v: row tid / 8, columns c0 + 8 (tid % 8) .. + 7 of a chunk
  const int vj = tid >> 3, vb = (tid & 7) * 8;
  const bf16_t* vrow = static_cast<const bf16_t*>(a.v) + (bh * T + vj) * dv + c0 + vb;

  // Gate scan of the chunk at tok0 from its raw gates (this wave's copy):
  // w_j = exp(u_j - M_L) in lane j, g_L, and m after the chunk.
  struct Scan {
    float w, gL, m_after;
  };
  auto scan = [&](float fpre, float ipre, float ms) {
    const float lf = a.fgate_exp ? fpre : log_sigmoid(fpre);
    const float bc = scan_add(lf);
    const float u = ipre - bc;
    const float Mx = fmaxf(ms, scan_max(u));
    const float ML = __shfl(Mx, LC - 1, 64);
    Scan r;
    r.w = __expf(u - ML);
    r.gL = __shfl(__expf(ms - Mx), LC - 1, 64);
    r.m_after = __shfl(bc + Mx, LC - 1, 64);
    return r;
  };
  // w (.) V of this thread's row as a bf16 hi / lo pair into the buffers of
  // parity par; wave 0 also writes w itself (rows 0, 1 of sWD)
  auto split_wv = [&](const uint4 v8, float wlane, int par) {
    const float wj = __shfl(wlane, vj, 64);
    const float x[8] = {bf_lo(v8.x), bf_hi(v8.x), bf_lo(v8.y), bf_hi(v8.y),
                        bf_lo(v8.z), bf_hi(v8.z), bf_lo(v8.w), bf_hi(v8.w)};
    uint32_t hp[4], lp[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float y0 = wj * x[e], y1 = wj * x[e + 1];
      const uint32_t h2 = pk2(y0, y1);
      hp[e / 2] = h2;
      lp[e / 2] = pk2(y0 - bf_lo(h2), y1 - bf_hi(h2));
    }
    *reinterpret_cast<uint4*>(sWH[par] + swz(vj, vb)) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
    *reinterpret_cast<uint4*>(sWL[par] + swz(vj, vb)) = make_uint4(lp[0], lp[1], lp[2], lp[3]);
    if (lead && wave == 0) {   // the A operand of n~ += sum_j w_j k_j (hi and lo rows)
      const bf16_t hi = f2bf(wlane);
      *reinterpret_cast<bf16_t*>(sWD[par] + swz(0, lane)) = hi;
      *reinterpret_cast<bf16_t*>(sWD[par] + swz(1, lane)) = f2bf(wlane - bf2f(hi));
    }
  };

  // ---- prologue: k of chunk 0 in flight; chunk 0's scan and w (.) V
  dma_k_chunk8<DK>(a, bh * T, wave, lane, sK[0]);
  float gL, m_next;   // g_L of the current chunk, m after it
  {
    const Scan r = scan(a.f_pre[bh * T + lane], a.i_pre[bh * T + lane], m);
    gL = r.gL;
    m_next = r.m_after;
    split_wv(*reinterpret_cast<const uint4*>(vrow), r.w, 0);
  }

  for (int c = 0; c <= nc; ++c) {
    const int par = c & 1;
    // every load issued so far (k of chunk c) has landed, and every wave has
    // written chunk c's w (.) V and w and left the previous chunk's buffers
    wait_vm<0>();
    __syncthreads();
    // the stored state at boundary c: before a chunk as this workgroup's
    // swizzled bf16 tile (the reverse pass's LDS image), after the last
    // chunk in float32
    if (c < nc) {
      char* tile = reinterpret_cast<char*>(a.ws_Cb + ((bh * ncb + cb) * nc + c) * (DK * TVC));
#pragma unroll
      for (int t = 0; t < NXH; ++t)
        *reinterpret_cast<uint2*>(tile + swz((rh * NXH + t) * 16 + l16, cg * 16 + 4 * g)) =
            make_uint2(pk2(Ct[t][0], Ct[t][1]), pk2(Ct[t][2], Ct[t][3]));
    } else {
      float* wsC = a.ws_CT + bh * DK * dv + c0 + cg * 16 + 4 * g;
#pragma unroll
      for (int t = 0; t < NXH; ++t)
        *reinterpret_cast<float4*>(wsC + static_cast<int64_t>((rh * NXH + t) * 16 + l16) * dv) =
            make_float4(Ct[t][0], Ct[t][1], Ct[t][2], Ct[t][3]);
    }
    if (lead) {
      if (g == 0) {
#pragma unroll
        for (int p = 0; p < NXN; ++p) {
          const int xt = wave * NXN + p;
          if (xt < NXT) a.ws_n[(bh * nb + c) * DK + xt * 16 + l16] = nx[p];
        }
      }
      if (tid == 0) a.ws_m[bh * nb + c] = m;
    }
    if (c == nc) break;
    const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
    const char* kc = sK[par];
    // the next chunk: k into the other LDS half (its last reads were the
    // previous chunk's), its gates and this thread's v into registers
    const bool more = c + 1 < nc;
    if (more) dma_k_chunk8<DK>(a, tok0 + LC, wave, lane, sK[par ^ 1]);
    const int64_t tn = more ? tok0 + LC : tok0;   // (past the end: a harmless re-read)
    const float fpre_n = a.f_pre[tn + lane], ipre_n = a.i_pre[tn + lane];
    const uint4 vn = *reinterpret_cast<const uint4*>(vrow + (more ? static_cast<int64_t>(c + 1) * LC * dv : 0));

    // ---- C~ <- g_L C~ + K^T (w (.) V) for this wave's tiles
#pragma unroll
    for (int t = 0; t < NXH; ++t) Ct[t] *= gL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 Ah = colfrag(sWH[par], 32 * ks, cg * 16, g, kr, kq);
      const bf16x8 Al = colfrag(sWL[par], 32 * ks, cg * 16, g, kr, kq);
#pragma unroll
      for (int t = 0; t < NXH; ++t) {
        const int xt = rh * NXH + t;
        const bf16x8 Bk = colfrag(wide(kc, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq);
        Ct[t] = mfma16x16x32(Ah, Bk, Ct[t]);
        Ct[t] = mfma16x16x32(Al, Bk, Ct[t]);
      }
    }
    if (lead) {   // n~ <- g_L n~ + K^T w for this wave's x tiles (D rows 0 + 1)
      f32x4 nacc[NXN];
#pragma unroll
      for (int p = 0; p < NXN; ++p) nacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Aw = rowfrag(sWD[par], l16, 32 * ks + 8 * g);
#pragma unroll
        for (int p = 0; p < NXN; ++p) {
          const int xt = wave * NXN + p;
          if (xt < NXT)
            nacc[p] = mfma16x16x32(Aw, colfrag(wide(kc, xt * 16), 32 * ks, (xt * 16) & 63, g, kr, kq), nacc[p]);
        }
      }
#pragma unroll
      for (int p = 0; p < NXN; ++p) nx[p] = gL * nx[p] + (nacc[p][0] + nacc[p][1]);
    }
    // ---- the next chunk's scan and w (.) V (into the other parity)
    m = m_next;
    if (more) {
      const Scan r = scan(fpre_n, ipre_n, m);
      split_wv(vn, r.w, par ^ 1);
      gL = r.gL;
      m_next = r.m_after;
    }
  }
}

// dq and dk of one chunk over all of d_v, for every (head, chunk, d_qk slice)
// at once.  The reverse pass has stored, per chunk, r (bf16 [T][d_v]), the
// memory gradient at the chunk's end (dC, bf16 tiles in the state tiles'
// order), dn at the chunk's end and dnq; the state pass the boundary state
// C~_s and n~_s.  With g_i = exp(m_s - M_i), w_j = exp(u_j - M_L) and
// D_ij = exp(u_j - M_i) (j <= i) from the chunk's gate scan:
//
//   dq_i = g_i (C~_s r_i + dnq_i n~_s) + sum_j W_ij k_j
//   dk_j = w_j (dC v_j + dn)           + sum_i W_ij q_i
//   W_ij = D_ij (r_i . v_j + dnq_i)
//
// Workgroup = (head, chunk, XW rows x of d_qk), 4 waves; wave w owns the x
// tiles w XPW .. w XPW + XPW - 1 of the slice and, for W, the key tile j =
// 16 w .. 16 w + 15.  In the d_v contractions (C~_s R^T, dC V^T, V R^T)
// each wave reads its own C~_s and dC rows straight from HBM as 16-byte MFMA
// fragments, while r and v, which every wave needs whole, pass once per
// workgroup through LDS (each wave reading them itself doubled the L2
// requests and cost 0.33 ms per backward at d = 256, T = 8192).  The row
// scales g_i and w_j are applied to the float32 accumulators, after which the
// intra-chunk products add K^T W^T and Q^T W from the LDS copies of this
// slice of q and k.  The per-token dots q . dq and k . dk of the slice go to
// HBM for the per-head pass.
constexpr int QK_XW = 128;      // d_qk rows per workgroup of the dq/dk pass (at most)
constexpr int QK_OCC = 2;       // its workgroups per CU (waves per SIMD)

template <int DK>
__global__ __launch_bounds__(NT4, QK_OCC) void bwd_qk_mfma_kernel(BwdArgs a) {
  constexpr int XW = DK < QK_XW ? DK : QK_XW;   // d_qk rows per workgroup
  constexpr int NSPL = DK / XW;
  constexpr int XPW = XW / 64;              // 16-row x tiles per wave
  constexpr int NXQ = XW / 64;              // [64][64] tiles of the q (k) slice
  __shared__ __align__(1024) char sQ[NXQ * TB];
  __shared__ __align__(1024) char sK[NXQ * TB];
  __shared__ __align__(1024) char sW[TB];
  __shared__ __align__(1024) char sRV[2][2][TB];   // [step parity][r, v]: 64 columns of d_v
  __shared__ Gate64 G;
  __shared__ float sN[XW], sDn[XW];
  __shared__ float sDnq[LC];
  __shared__ float sDot[2][4][LC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int dv = static_cast<int>(a.dv);
  const int ncb = dv / TVC;
  const int64_t T = a.T;
  const int nc = static_cast<int>(T / LC);
  const int64_t nb = nc + 1;
  const int64_t BH = a.B * a.H;
  // workgroup -> (unit = head * nc + chunk, slice): with the unit count a
  // multiple of 8, the slices of one unit get ids equal mod 8 (one XCD), so
  // their shared r and v reads meet in one L2
  int64_t unit;
  int sp;
  {
    const int64_t w = blockIdx.x, nu = BH * nc;
    if (NSPL == 1) {
      unit = w;
      sp = 0;
    } else if (nu % 8 == 0) {
      const int64_t grp = w / (8 * NSPL), r = w % (8 * NSPL);
      sp = static_cast<int>(r / 8);
      unit = grp * 8 + r % 8;
    } else {
      unit = w / NSPL;
      sp = static_cast<int>(w % NSPL);
    }
  }
  const int64_t bh = unit / nc;
  const int c = static_cast<int>(unit % nc);
  const int64_t tok0 = bh * T + static_cast<int64_t>(c) * LC;
  const int xs = sp * XW;   // first d_qk row of the slice

  // ---- this slice of q and k into LDS (direct loads; waited for before
  // the barrier that precedes the intra-chunk products).  Load G of 8 * NXQ
  // per matrix fills rows 8 (G % 8) .. + 7 of tile G / 8; lane l writes
  // physical chunk l % 8 of row 8 (G % 8) + l / 8, which holds the logical
  // chunk (l % 8) ^ ((row / 2) % 8).
  {
    const bf16_t* q = static_cast<const bf16_t*>(a.q) + tok0 * DK + xs;
    const bf16_t* k = static_cast<const bf16_t*>(a.k) + tok0 * DK + xs;
    const int row8 = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int p = 0; p < 2 * NXQ; ++p) {
      const int Gi = wave * 2 * NXQ + p;          // 0 .. 8 NXQ - 1
      const int t = Gi >> 3, rg = Gi & 7;
      const int row = 8 * rg + row8;
      const int64_t off = static_cast<int64_t>(row) * DK + 64 * t + 8 * (pc ^ ((row >> 1) & 7));
      const uint32_t lq = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr(sQ + t * TB + rg * 1024))));
      const uint32_t lk = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr(sK + t * TB + rg * 1024))));
      dma16(q + off, lq);
      dma16(k + off, lk);
    }
  }
  if (wave == 0) gate_scan64(a, tok0, a.ws_m[bh * nb + c], G);
  for (int x = tid; x < XW; x += NT4) {
    sN[x] = a.ws_n[(bh * nb + c) * DK + xs + x];
    sDn[x] = a.ws_dn[(bh * nc + c) * DK + xs + x];
  }
  if (tid < LC) sDnq[tid] = a.ws_dnq[tok0 + tid];

  // ---- the d_v contractions, one MFMA k step (32 columns) at a time.
  // Fragments: lane (l16, g) holds columns b0 + 8 g .. + 7 of
  //   C~_s and dC rows x = xs + 16 (wave XPW + p) + l16  (A operands, HBM)
  //   r rows i = 16 it + l16, v rows j = 16 jt + l16      (B operands, LDS)
  //   v row 16 wave + l16                                 (A of V R^T, LDS)
  const char* Cst = reinterpret_cast<const char*>(a.ws_Cb);
  const char* dCt = reinterpret_cast<const char*>(a.ws_dCb);
  struct FragCD {
    u32x4 C[XPW], D[XPW];
  };
  struct FragRV {
    u32x4 R[4], V[4], Va;
  };
  auto load_cd = [&](int ks, FragCD& F) {
    const int b0 = 32 * ks;
    const int64_t tile = ((bh * ncb + (b0 >> 6)) * nc + c) * static_cast<int64_t>(DK * TVC * 2);
#pragma unroll
    for (int p = 0; p < XPW; ++p) {
      const int x = xs + 16 * (wave * XPW + p) + l16;
      const int off = swz(x, (b0 & 63) + 8 * g);
      F.C[p] = *reinterpret_cast<const u32x4*>(Cst + tile + off);
      F.D[p] = *reinterpret_cast<const u32x4*>(dCt + tile + off);
    }
  };
  // accQ[p][it]: dq^T[x = 16 (wave XPW + p) + 4 g + e][i = 16 it + l16]
  // accK[p][jt]: dk^T[x][j = 16 jt + l16]
  // accS[it]:    (R V^T)^T[j = 16 wave + 4 g + e][i = 16 it + l16]
  f32x4 accQ[XPW][4], accK[XPW][4], accS[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    accS[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < XPW; ++p) {
      accQ[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      accK[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  auto compute = [&](const FragCD& F, const FragRV& G) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 Br = __builtin_bit_cast(bf16x8, G.R[t]);
      const bf16x8 Bv = __builtin_bit_cast(bf16x8, G.V[t]);
      accS[t] = mfma16x16x32(__builtin_bit_cast(bf16x8, G.Va), Br, accS[t]);
#pragma unroll
      for (int p = 0; p < XPW; ++p) {
        accQ[p][t] = mfma16x16x32(__builtin_bit_cast(bf16x8, F.C[p]), Br, accQ[p][t]);
        accK[p][t] = mfma16x16x32(__builtin_bit_cast(bf16x8, F.D[p]), Bv, accK[p][t]);
      }
    }
  };
  {
    // 64 columns of d_v per step: this thread's share of the step's r and v
    // (rows e / 8, 16-byte chunk e % 8 of each [64][64] tile) is read into
    // registers one step ahead and written to the LDS buffer of the step's
    // parity at its top; C~_s and dC fragments (per wave) one step ahead in
    // registers.  One barrier per step: a buffer is rewritten two steps after
    // it was read, and every wave has passed the previous step's barrier.
    constexpr int NRV = 2 * LC * 64 / 8 / NT4;
    u32x4 rv[NRV];
    const bf16_t* rb = a.ws_R + tok0 * dv;
    const bf16_t* vb = static_cast<const bf16_t*>(a.v) + tok0 * dv;
    auto load_rv_regs = [&](int st) {
#pragma unroll
      for (int p = 0; p < NRV; ++p) {
        const int e = tid + p * NT4, mat = e >> 9, row = (e >> 3) & 63, ch = e & 7;
        rv[p] = *reinterpret_cast<const u32x4*>((mat ? vb : rb) + static_cast<int64_t>(row) * dv + 64 * st + 8 * ch);
      }
    };
    auto store_rv = [&](int par) {
#pragma unroll
      for (int p = 0; p < NRV; ++p) {
        const int e = tid + p * NT4, mat = e >> 9, row = (e >> 3) & 63, ch = e & 7;
        *reinterpret_cast<u32x4*>(sRV[par][mat] + swz(row, 8 * ch)) = rv[p];
      }
    };
    const int nst = dv / 64;
    FragCD Fa[2], Fb[2];
    load_rv_regs(0);
    load_cd(0, Fa[0]);
    load_cd(1, Fa[1]);
    for (int st = 0; st < nst; ++st) {
      const int par = st & 1;
      store_rv(par);
      if (st + 1 < nst) {
        load_rv_regs(st + 1);
        load_cd(2 * st + 2, Fb[0]);
        load_cd(2 * st + 3, Fb[1]);
      }
      __syncthreads();   // this step's r, v (and, at the first step, G, sN, sDn, sDnq)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        FragRV Gf;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Gf.R[t] = __builtin_bit_cast(u32x4, lds_ld16(sRV[par][0], swz(16 * t + l16, 32 * kk + 8 * g)));
          Gf.V[t] = __builtin_bit_cast(u32x4, lds_ld16(sRV[par][1], swz(16 * t + l16, 32 * kk + 8 * g)));
        }
        Gf.Va = __builtin_bit_cast(u32x4, lds_ld16(sRV[par][1], swz(16 * wave + l16, 32 * kk + 8 * g)));
        compute(Fa[kk], Gf);
      }
      Fa[0] = Fb[0];
      Fa[1] = Fb[1];
    }
  }

  // ---- W = D (.) (R V^T + dnq) for key tile j = 16 wave + 4 g + e (bf16,
  // [i][j] in LDS); the inter-chunk terms take their row scales
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = it * 16 + l16;
    const float Mi = G.M[i], dq_ = sDnq[i], gi_ = G.g[i], wi = G.w[i];
    float wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = wave * 16 + 4 * g + e;
      wv[e] = j <= i ? __expf(G.u[j] - Mi) * (accS[it][e] + dq_) : 0.0f;
    }
    *reinterpret_cast<uint2*>(sW + swz(i, wave * 16 + 4 * g)) = make_uint2(pk2(wv[0], wv[1]), pk2(wv[2], wv[3]));
#pragma unroll
    for (int p = 0; p < XPW; ++p) {
      accQ[p][it] *= gi_;
      accK[p][it] *= wi;   // here it is the key tile: w of key 16 it + l16
    }
  }
  wait_vm<0>();      // this thread's part of the q / k slice has landed
  __syncthreads();   // W and the slice are visible
  // ---- dq^T += K^T W^T,  dk^T += Q^T W  (contraction over the chunk's tokens)
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 Bw[4], Bwt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Bw[t] = rowfrag(sW, t * 16 + l16, 32 * ks + 8 * g);    // [k = j][n = i] = W[i][j]
      Bwt[t] = colfrag(sW, 32 * ks, t * 16, g, kr, kq);      // [k = i][n = j] = W[i][j]
    }
#pragma unroll
    for (int p = 0; p < XPW; ++p) {
      const int xl = 16 * (wave * XPW + p);
      const bf16x8 Ak = colfrag(wide(sK, xl), 32 * ks, xl & 63, g, kr, kq);
      const bf16x8 Aq = colfrag(wide(sQ, xl), 32 * ks, xl & 63, g, kr, kq);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        accQ[p][t] = mfma16x16x32(Ak, Bw[t], accQ[p][t]);
        accK[p][t] = mfma16x16x32(Aq, Bwt[t], accK[p][t]);
      }
    }
  }
  // ---- the normalizer terms, dq and dk to HBM, and the slice's dots
  float qd[4], kd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = t * 16 + l16;
    const float fq = G.g[i] * sDnq[i], fk = G.w[i];
    qd[t] = 0.0f;
    kd[t] = 0.0f;
#pragma unroll
    for (int p = 0; p < XPW; ++p) {
      const int xl = 16 * (wave * XPW + p) + 4 * g;
      float vq[4], vk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vq[e] = accQ[p][t][e] + fq * sN[xl + e];
        vk[e] = accK[p][t][e] + fk * sDn[xl + e];
      }
      const int64_t o = (tok0 + i) * DK + xs + xl;
      *reinterpret_cast<float4*>(a.d_q + o) = make_float4(vq[0], vq[1], vq[2], vq[3]);
      *reinterpret_cast<float4*>(a.d_k + o) = make_float4(vk[0], vk[1], vk[2], vk[3]);
      const uint2 q4 = *reinterpret_cast<const uint2*>(wide(sQ, xl) + swz(i, xl & 63));
      const uint2 k4 = *reinterpret_cast<const uint2*>(wide(sK, xl) + swz(i, xl & 63));
      qd[t] += (bf_lo(q4.x) * vq[0] + bf_hi(q4.x) * vq[1]) + (bf_lo(q4.y) * vq[2] + bf_hi(q4.y) * vq[3]);
      kd[t] += (bf_lo(k4.x) * vk[0] + bf_hi(k4.x) * vk[1]) + (bf_lo(k4.y) * vk[2] + bf_hi(k4.y) * vk[3]);
    }
    // over the four lane groups g (the x rows of each tile)
    qd[t] += __shfl_xor(qd[t], 16, 64);
    qd[t] += __shfl_xor(qd[t], 32, 64);
    kd[t] += __shfl_xor(kd[t], 16, 64);
    kd[t] += __shfl_xor(kd[t], 32, 64);
    if (g == 0) {
      sDot[0][wave][i] = qd[t];
      sDot[1][wave][i] = kd[t];
    }
  }
  __syncthreads();
  if (tid < 2 * LC) {   // wave 0: q . dq, wave 1: k . dk; and their sums over the chunk
    const int which = tid >> 6, i = tid & 63;
    const float s = (sDot[which][0][i] + sDot[which][1][i]) + (sDot[which][2][i] + sDot[which][3][i]);
    (which ? a.ws_kd : a.ws_qd)[sp * BH * T + tok0 + i] = s;
    const float tot = wave_sum(s);
    if (i == 0) a.ws_csum[(sp * BH * nc + unit) * 2 + which] = tot;
  }
}

// d~i and d log f per token, and dm0, one wave per (head, chunk).  From
// the dq/dk pass's per-token q . dq and k . dk (per d_qk slice) and their
// chunk sums, and the final-state term from the reverse pass:
//   d~i_t = k_t . dk_t
//   d log f_t = sum_{t' >= t} (q_t' . dq_t' - k_t' . dk_t') + <dC1, C~_T> + <dn1, n~_T>
// (the derivative of the cumulative log forget gates of the chunkwise form).
// The sum over the chunks after this one comes from their chunk sums; within
// the chunk, lane l takes token 63 - l, so a prefix sum over the lanes is the
// sum over the tokens at and after it.
__global__ __launch_bounds__(NT4) void bwd_gates64_kernel(BwdArgs a, int nspl, int ncb) {
  const int lane = threadIdx.x & 63;
  const int64_t T = a.T, BH = a.B * a.H;
  const int nc = static_cast<int>(T / LC);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * (NT4 / 64) + (threadIdx.x >> 6);
  if (unit >= BH * nc) return;   // (no barriers below)
  const int64_t bh = unit / nc;
  const int c = static_cast<int>(unit % nc);
  float carry = 0.0f;
  for (int c2 = c + 1 + lane; c2 < nc; c2 += 64) {
    for (int p = 0; p < nspl; ++p) {
      const float* cs = a.ws_csum + (p * BH * nc + bh * nc + c2) * 2;
      carry += cs[0] - cs[1];
    }
  }
  if (a.dC1) {
    for (int cb = lane; cb < ncb; cb += 64) carry += a.ws_kend[static_cast<int64_t>(cb) * BH + bh];
  }
  carry = wave_sum(carry);
  const int64_t t = bh * T + static_cast<int64_t>(c) * LC + (LC - 1 - lane);
  float qd = 0.0f, kd = 0.0f;
  for (int p = 0; p < nspl; ++p) {
    qd += a.ws_qd[p * BH * T + t];
    kd += a.ws_kd[p * BH * T + t];
  }
  a.d_i[t] = kd;
  const float after = carry + scan_add(qd - kd);
  a.d_f[t] = a.fgate_exp ? after : after * (1.0f - sigmoid_fast(a.f_pre[t]));
  if (a.dm0 && c == 0 && lane == 0) {
    float s = 0.0f;
    for (int cb = 0; cb < ncb; ++cb) s += a.ws_dm0[static_cast<int64_t>(cb) * BH + bh];
    a.dm0[bh] = s;
  }
}

template <int DK>
hipError_t launch_states_dk(const BwdArgs& a, hipStream_t st) {
  bwd_states_mfma_kernel<DK><<<static_cast<unsigned>(a.B * a.H * (a.dv / TVC)), NT8, 0, st>>>(a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const BwdArgs& a, hipStream_t st) {
  const unsigned wgs = static_cast<unsigned>(a.B * a.H * (a.dv / TVC));
  if (a.o_mode == O_BF16) bwd_rev_mfma_kernel<DK, bf16_t><<<wgs, NT8, 0, st>>>(a);
  else bwd_rev_mfma_kernel<DK, float><<<wgs, NT8, 0, st>>>(a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_qk_dk(const BwdArgs& a, hipStream_t st) {
  constexpr int NSPL = DK < QK_XW ? 1 : DK / QK_XW;
  const unsigned wgs = static_cast<unsigned>(a.B * a.H * (a.T / LC) * NSPL);
  bwd_qk_mfma_kernel<DK><<<wgs, NT4, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int bwd_qk_slices(const BwdArgs& a) { return a.dqk < QK_XW ? 1 : static_cast<int>(a.dqk / QK_XW); }

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

hipError_t launch_bwd_qk_mfma(const BwdArgs& a, hipStream_t st) {
  switch (a.dqk) {
    case 64: return launch_qk_dk<64>(a, st);
    case 128: return launch_qk_dk<128>(a, st);
    default: return launch_qk_dk<256>(a, st);
  }
}

hipError_t launch_bwd_gates_mfma(const BwdArgs& a, hipStream_t st) {
  const int64_t units = a.B * a.H * (a.T / LC);
  const unsigned wgs = static_cast<unsigned>((units + NT4 / 64 - 1) / (NT4 / 64));
  bwd_gates64_kernel<<<wgs, NT4, 0, st>>>(a, bwd_qk_slices(a), static_cast<int>(a.dv / TVC));
  return hipGetLastError();
}

}  // namespace mlstm
