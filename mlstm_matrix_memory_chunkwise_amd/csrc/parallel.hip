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
// (2) outputs: bf16 q/k/v with d_qk in {64, 128, 256} and d_v a multiple of
// 64 on MFMA (par_mfma_kernel below), everything else on the vector ALUs,
// one workgroup per (head, 64-query block, 16 value columns);
// (3) final state: the state-only chunk pass where it applies (bf16, T a
// multiple of 64), otherwise one thread per state element.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

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

// ---- outputs on bf16 MFMA.  One workgroup (4 waves) per (head, 64-query
// block, 64 value columns); wave w owns query tile w (16 queries).  Per key
// block of 64 (j0 = 0 .. i0), with the key and value tiles in LDS (global
// -> LDS loads one block ahead, double-buffered):
//   S^T = K Q^T for the wave's query tile and the 4 key tiles (MFMA),
//   P = S (.) D with D_ij = exp(u_j - M_i) (the exponent in float64),
//   masked to j <= i and j < T; its float32 row sums,
//   P to LDS (the wave's own query rows: written and read by the wave),
//   acc += P V (MFMA, V^T through the LDS transpose read).
// With an initial state, the readout q_i^T C~_0 runs once on MFMA with C~_0
// as a (high, remainder) bf16 pair, and q_i . n~_0 on the vector ALUs.
constexpr int PROW = 64 + 8;   // padded row of P (bf16)

template <int DQK, int OM>
__global__ __launch_bounds__(256, 1) void par_mfma_kernel(SeqArgs a, const double* ws) {
  using namespace mk;
  constexpr int NQT = DQK / 64;     // 64-wide d_qk tiles
  constexpr int NKS = DQK / 32;     // 32-wide k-steps over d_qk
  constexpr int TB = 64 * 128;      // bytes of a [64][64] bf16 tile
  __shared__ __align__(1024) char sQ[NQT * TB];
  __shared__ __align__(1024) char sK[2][NQT * TB];
  __shared__ __align__(1024) char sV[2][TB];
  __shared__ __align__(16) bf16_t sP[64 * PROW];
  __shared__ double sU[2][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int64_t bh = blockIdx.x;
  const int64_t T = a.T;
  const int dv = static_cast<int>(a.dv);
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int c0 = blockIdx.z * 64;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + bh * T * DQK;
  const bf16_t* k = static_cast<const bf16_t*>(a.k) + bh * T * DQK;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + bh * T * dv + c0;
  const double* U = ws + bh * 3 * T;
  const double* Mx = U + T;
  const double* Mm = Mx + T;

  // global -> LDS loads of a [64 rows][64 bf16] tile: one 1 KB instruction
  // per 8 rows (lane l: row 8 G + l / 8, physical chunk l % 8, which holds
  // the logical chunk (l % 8) ^ ((row / 2) % 8), the swz layout); rows past
  // T re-read row T - 1 (their values are masked)
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  auto load_tile = [&](const bf16_t* base, int64_t row0, int stride, char* dst, int G) {
    const int row = 8 * G + ld_r;
    int64_t r = row0 + row;
    if (r > T - 1) r = T - 1;
    dma16(base + r * stride + 8 * (ld_pc ^ ((row >> 1) & 7)), lds_addr(dst + G * 1024));
  };
  // a key block: NQT k tiles and one v tile, 8 (NQT + 1) instructions over
  // the 4 waves, and u of its keys
  auto load_block = [&](int64_t j0, int buf) {
#pragma unroll
    for (int x = 0; x < 2 * (NQT + 1); ++x) {
      const int item = wave * 2 * (NQT + 1) + x;   // 0 .. 8 (NQT + 1) - 1
      const int t = item >> 3, G = item & 7;
      if (t < NQT) load_tile(k + t * 64, j0, DQK, sK[buf] + t * TB, G);
      else load_tile(v, j0, dv, sV[buf], G);
    }
    if (tid < 64) sU[buf][tid] = U[j0 + tid < T ? j0 + tid : T - 1];
  };

  // the query block
#pragma unroll
  for (int x = 0; x < 2 * NQT; ++x) {
    const int item = wave * 2 * NQT + x;
    load_tile(q + (item >> 3) * 64, i0, DQK, sQ + (item >> 3) * TB, item & 7);
  }
  load_block(0, 0);

  const int iq = 16 * wave + l16;               // this lane's query (of the block)
  const int64_t ig = i0 + iq;
  const int64_t ic = ig < T ? ig : T - 1;
  const double Mi = Mx[ic];
  float rs = 0.0f;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblk = static_cast<int>(i0 / 64) + 1;
  for (int jb = 0; jb < nblk; ++jb) {
    const int buf = jb & 1;
    const int64_t j0 = static_cast<int64_t>(jb) * 64;
    wait_vm<0>();
    __syncthreads();   // block jb landed; every wave left block jb - 1's buffers
    if (jb + 1 < nblk) load_block(j0 + 64, buf ^ 1);
    // S^T of key tile kt and the wave's query tile
    f32x4 st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const char* Qt = sQ + (ks >> 1) * TB;
      const char* Kt = sK[buf] + (ks >> 1) * TB;
      const int col = 32 * (ks & 1) + 8 * g;
      const bf16x8 Bq = as_bf16x8(lds_ld16(Qt, swz(iq, col)));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st[kt] = mfma16x16x32(as_bf16x8(lds_ld16(Kt, swz(kt * 16 + l16, col))), Bq, st[kt]);
    }
    // P = S (.) D (lane: keys 16 kt + 4 g + e of query iq) and its row sums
    float part = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = kt * 16 + 4 * g + e;
        const int64_t j = j0 + jj;
        const float d = __expf(static_cast<float>(sU[buf][jj] - Mi));
        pe[e] = (j <= ig && j < T) ? st[kt][e] * d : 0.0f;
      }
      part += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      *reinterpret_cast<uint2*>(sP + iq * PROW + kt * 16 + 4 * g) = make_uint2(cvt2(pe[0], pe[1]), cvt2(pe[2], pe[3]));
    }
    rs += sum_groups(part);
    // P V (the P rows are this wave's own: written and read in order)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 Pf = as_bf16x8(*reinterpret_cast<const uint4*>(sP + iq * PROW + 32 * ks + 8 * g));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = ct * 16 + 4 * kq;
        const bf16x8 Vf = join(lds_tr(sV[buf], swz(32 * ks + 8 * g + kr, col)),
                               lds_tr(sV[buf], swz(32 * ks + 8 * g + 4 + kr, col)));
        acc[ct] = mfma16x16x32(Vf, Pf, acc[ct]);
      }
    }
  }

  // ---- the initial state's terms: g_i q_i^T C~_0 (MFMA, C~_0 as a high /
  // remainder bf16 pair) and g_i q_i . n~_0
  const double m0 = a.C0 ? static_cast<double>(a.m0[bh]) : 0.0;
  const float gi = static_cast<float>(exp(m0 - Mi));
  f32x4 ro[4];
  float qn = 0.0f;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) ro[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.C0) {
    const float* C0 = a.C0 + bh * static_cast<int64_t>(DQK) * dv + c0;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 Bq = as_bf16x8(lds_ld16(sQ + (ks >> 1) * TB, swz(iq, 32 * (ks & 1) + 8 * g)));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        // A[c = l16][d = 8 g + e] = C~_0[32 ks + 8 g + e][16 ct + l16]
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = C0[static_cast<int64_t>(32 * ks + 8 * g + e) * dv + 16 * ct + l16];
        bf16x8 hi, lo;
        cvt8_split(x, hi, lo);
        ro[ct] = mfma16x16x32(hi, Bq, ro[ct]);
        ro[ct] = mfma16x16x32(lo, Bq, ro[ct]);
      }
    }
    // q . n~_0: lane group g takes a quarter of d_qk
    const float* n0 = a.n0 + bh * DQK;
    float s4 = 0.0f;
#pragma unroll
    for (int x8 = g * (DQK / 4); x8 < (g + 1) * (DQK / 4); x8 += 8) {
      const uint4 q8 = lds_ld16(sQ + (x8 >> 6) * TB, swz(iq, x8 & 63));
      s4 += bf_lo(q8.x) * n0[x8] + bf_hi(q8.x) * n0[x8 + 1] + bf_lo(q8.y) * n0[x8 + 2] +
            bf_hi(q8.y) * n0[x8 + 3] + bf_lo(q8.z) * n0[x8 + 4] + bf_hi(q8.z) * n0[x8 + 5] +
            bf_lo(q8.w) * n0[x8 + 6] + bf_hi(q8.w) * n0[x8 + 7];
    }
    qn = sum_groups(s4);
  }
  if (ig >= T) return;
  // ---- h (lane: query iq, columns 16 ct + 4 g + e)
  const float den = fmaxf(fabsf(gi * qn + rs), static_cast<float>(exp(-Mm[ig])));
  const float inv = 1.0f / den;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int64_t oi = (bh * T + ig) * dv + c0 + 16 * ct + 4 * g;
    float hv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = (gi * ro[ct][e] + acc[ct][e]) * inv;
    if (OM == O_F32) {
      const float4 o4 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.o_pre) + oi);
      hv[0] *= sigmoidf_(o4.x); hv[1] *= sigmoidf_(o4.y); hv[2] *= sigmoidf_(o4.z); hv[3] *= sigmoidf_(o4.w);
    } else if (OM == O_BF16) {
      const uint2 o2 = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(a.o_pre) + oi);
      hv[0] *= sigmoidf_(bf_lo(o2.x)); hv[1] *= sigmoidf_(bf_hi(o2.x));
      hv[2] *= sigmoidf_(bf_lo(o2.y)); hv[3] *= sigmoidf_(bf_hi(o2.y));
    }
    *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.h) + oi) = make_uint2(cvt2(hv[0], hv[1]), cvt2(hv[2], hv[3]));
  }
}

bool par_mfma_supported(const SeqArgs& a) {
  return a.qkv_bf16 && (a.dqk == 64 || a.dqk == 128 || a.dqk == 256) && a.dv % 64 == 0 && a.T > 0;
}

template <int OM>
void launch_par_mfma(const SeqArgs& a, double* ws, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>((a.T + 63) / 64), static_cast<unsigned>(a.dv / 64));
  switch (a.dqk) {
    case 64: par_mfma_kernel<64, OM><<<grid, 256, 0, stream>>>(a, ws); break;
    case 128: par_mfma_kernel<128, OM><<<grid, 256, 0, stream>>>(a, ws); break;
    default: par_mfma_kernel<256, OM><<<grid, 256, 0, stream>>>(a, ws); break;
  }
}

template <typename TQ, int OM>
hipError_t launch_typed(const SeqArgs& a, double* ws, hipStream_t stream) {
  const unsigned BH = static_cast<unsigned>(a.B * a.H);
  par_scan_kernel<<<BH, 64, 0, stream>>>(a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (par_mfma_supported(a)) {
    launch_par_mfma<OM>(a, ws, stream);
  } else {
    dim3 g2(BH, static_cast<unsigned>((a.T + kQB - 1) / kQB), static_cast<unsigned>((a.dv + kTV - 1) / kTV));
    par_out_kernel<TQ, OM><<<g2, kThreads, 0, stream>>>(a, ws);
  }
  e = hipGetLastError();
  if (e != hipSuccess || !a.C1) return e;
  // the final state: the state-only chunk pass computes the same sum (with
  // its own rounding) far faster where it applies
  if (chunk_state_supported(a)) return launch_chunk_state(a, stream);
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
