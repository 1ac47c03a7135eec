// The states at the split points of a long sequence with few heads (d_qk
// 256), each from weighted products over the tokens before it.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form": the
// unrolled memory is a sum over tokens, C_T = sum_j (prod_{t>j} f_t) i_j v_j k_j^T
// (and n_T likewise with k_j), and section 2 "The Normalizer State and
// Numerical Stabilization": with the running maximum m_T written in closed
// form,
//   e_j = i~_j + sum_{t>j} log f_t,   m_T = max(m_0 + sum_t log f_t, max_j e_j),
// the stabilized state C~_T = C_T e^{-m_T} is
//   C~_T = g_0 C~_0 + K^T diag(w) V,  n~_T = g_0 n~_0 + K^T w,
//   w_j = exp(e_j - m_T) <= 1,        g_0 = exp(m_0 + sum_t log f_t - m_T) <= 1,
// which is the chunk update of the chunkwise kernels with the whole sequence
// as one chunk.  The recurrence m_t = max(log f_t + m_{t-1}, i~_t) unrolls to
// exactly this m_T, so the result equals the chunkwise state up to rounding.
// For several split points the tokens before the last one form Q equal
// summary segments.  Each segment gets its own summary from a zero state,
// normalized by its own largest e_j (e_j and that maximum taken within the
// segment).  The states at the segment ends follow in order from the
// associative combine of the chunk update,
//   m' = max(m + sum_seg log f, m_seg),
//   C~' = exp(m + sum_seg log f - m') C~ + exp(m_seg - m') C~_seg,
// every exponent <= 0.
//
// Design (CDNA4): the sum over tokens has no sequential dependency, so it is
// split over token segments as well as heads and value columns until the
// grid fills the GPU, and each workgroup accumulates a 256 x 128 block of
// C~ (four times the columns of the chunk kernels' state tiles, so each K^T
// fragment read from LDS feeds four times the MFMAs):
//   1. state_gsum_kernel: per block of 1024 tokens of a head, the sum of
//      log f (float64);
//   2. state_gexp_kernel: per block, e_j within its summary segment (float64
//      prefix sums over the segment's blocks before it and a block scan,
//      stored as float32) and the block's largest e_j;
//   3. state_gemm_kernel: per (head, 128 value columns, token segment; the
//      token segments nest in the summary segments), the summary segment's
//      largest e_j from the block maxima, w_j = exp(e_j - that maximum),
//      then K^T diag(w) V on bf16 MFMA (w V rounded to bf16, as in the chunk
//      kernels' update) and K^T w with w split into three bf16 terms (about
//      24 bits), written as partial sums;
//   4. state_scalars_kernel, state_scan_*: the combine factors of every
//      segment end, then the states there from the initial state and the
//      partial sums, in a fixed order (deterministic).
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int DQK = 256;
constexpr int L = 64;             // tokens per step of the product
constexpr int NKS = L / 32;
constexpr int TVG = 128;          // value columns per workgroup
constexpr int NTH = 512;
constexpr int NW = 8;
constexpr int D = 2;              // steps in flight
constexpr int NSLOT = D + 1;
constexpr int NB = 4 + 2 + 1;     // loads per wave per step: K (4 KB), V (2 KB), w (256 B)
constexpr int GT = 256;           // threads of the gate kernels
constexpr int GR = 4 * GT;        // tokens per gate block (4 per thread)
constexpr int kMaxSegments = 16;

struct GemmArgs {
  int64_t BH, Tp, Ts, dv;
  int S;                          // token segments (a multiple of Q)
  int Q;                          // summary segments
  int nbk;                        // gate blocks per head
  int bps;                        // gate blocks per summary segment
  const bf16_t* k;
  const bf16_t* v;
  const float* e;                 // e_j [BH][Tp]
  const double* psum;             // sum of log f per gate block [BH][nbk]
  const double* pmax;             // largest e_j per gate block [BH][nbk]
  float* part;                    // [S][BH][DQK][dv]
  float* npart;                   // [S][BH][DQK]
};

// sum log f and the largest e_j of summary segment k of one head, from the
// per-block figures (the same order everywhere: bitwise equal)
__device__ __forceinline__ void seg_scalars(const double* psum, const double* pmax, int nbk, int bps,
                                            int64_t bh, int k, double& total, double& emax) {
  total = 0.0;
  emax = -1.0e300;
  const int b1 = (k + 1) * bps < nbk ? (k + 1) * bps : nbk;
  for (int b = k * bps; b < b1; ++b) {
    total += psum[bh * nbk + b];
    emax = pmax[bh * nbk + b] > emax ? pmax[bh * nbk + b] : emax;
  }
}

// ---- 1., 2. gate weights.  Block b of a head covers tokens GR b .. GR b +
// GR - 1; thread t takes the four tokens GR b + 4 t .. + 3 (one 16-byte load
// per gate array).
__device__ __forceinline__ void gate_lf4(const SeqArgs& a, int64_t bh, int64_t j, double lf[4]) {
  const float4 f = *reinterpret_cast<const float4*>(a.f_pre + bh * a.Ts + j);
  lf[0] = static_cast<double>(log_forget_fast(f.x, a.fgate_exp));
  lf[1] = static_cast<double>(log_forget_fast(f.y, a.fgate_exp));
  lf[2] = static_cast<double>(log_forget_fast(f.z, a.fgate_exp));
  lf[3] = static_cast<double>(log_forget_fast(f.w, a.fgate_exp));
}

__global__ __launch_bounds__(GT) void state_gsum_kernel(SeqArgs a, double* psum, int nbk) {
  __shared__ double s_x[GT];
  const int64_t bh = blockIdx.x / nbk;
  const int b = blockIdx.x % nbk;
  const int tid = threadIdx.x;
  const int64_t j = static_cast<int64_t>(b) * GR + 4 * tid;
  double x = 0.0;
  if (j < a.T) {
    double lf[4];
    gate_lf4(a, bh, j, lf);
    x = (lf[0] + lf[1]) + (lf[2] + lf[3]);
  }
  s_x[tid] = x;
  __syncthreads();
  for (int h = GT / 2; h > 0; h >>= 1) {
    if (tid < h) s_x[tid] += s_x[tid + h];
    __syncthreads();
  }
  if (tid == 0) psum[bh * nbk + b] = s_x[0];
}

__global__ __launch_bounds__(GT) void state_gexp_kernel(SeqArgs a, const double* psum, float* e_out,
                                                        double* pmax, int nbk, int bps) {
  __shared__ double s_x[2][GT];
  const int64_t bh = blockIdx.x / nbk;
  const int b = blockIdx.x % nbk;
  const int tid = threadIdx.x;
  // sums over this block's summary segment: before it, and in all
  const int k0 = (b / bps) * bps, k1 = k0 + bps < nbk ? k0 + bps : nbk;
  double before = 0.0, total = 0.0;
  for (int k = k0; k < k1; ++k) {
    const double x = psum[bh * nbk + k];
    if (k < b) before += x;
    total += x;
  }
  const int64_t j = static_cast<int64_t>(b) * GR + 4 * tid;
  const bool live = j < a.T;
  double lf[4] = {0.0, 0.0, 0.0, 0.0};
  if (live) gate_lf4(a, bh, j, lf);
  // inclusive scan of the threads' sums over the block (Hillis-Steele)
  double x = (lf[0] + lf[1]) + (lf[2] + lf[3]);
  int p = 0;
  s_x[0][tid] = x;
  __syncthreads();
  for (int h = 1; h < GT; h <<= 1) {
    const double y = s_x[p][tid] + (tid >= h ? s_x[p][tid - h] : 0.0);
    p ^= 1;
    s_x[p][tid] = y;
    __syncthreads();
  }
  const double incl = s_x[p][tid];
  __syncthreads();
  // e_j = i~_j + sum_{j < t <= segment end} log f_t
  //     = i~_j + total - (sum_{segment start <= t <= j} log f_t)
  double run = before + incl - x;
  double emax = -1.0e300;
  if (live) {
    const float4 iv = *reinterpret_cast<const float4*>(a.i_pre + bh * a.Ts + j);
    const float ii[4] = {iv.x, iv.y, iv.z, iv.w};
    float ev[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      run += lf[q];
      const double e = static_cast<double>(ii[q]) + (total - run);
      ev[q] = static_cast<float>(e);
      emax = e > emax ? e : emax;
    }
    *reinterpret_cast<float4*>(e_out + bh * a.T + j) = make_float4(ev[0], ev[1], ev[2], ev[3]);
  }
  s_x[0][tid] = emax;
  __syncthreads();
  for (int h = GT / 2; h > 0; h >>= 1) {
    if (tid < h) s_x[0][tid] = s_x[0][tid + h] > s_x[0][tid] ? s_x[0][tid + h] : s_x[0][tid];
    __syncthreads();
  }
  if (tid == 0) pmax[bh * nbk + b] = s_x[0][0];
}

// ---- 3. partial K^T diag(w) V and K^T w of one (head, 128 columns, segment)
__global__ __launch_bounds__(NTH, 1) void state_gemm_kernel(GemmArgs a) {
  __shared__ __align__(1024) char sK[NSLOT][4][L * 128];   // 4 [64 x 64] bf16 sub-tiles of K
  __shared__ __align__(1024) char sV[NSLOT][2][L * 128];   // 2 [64 x 64] sub-tiles of the columns
  __shared__ __align__(256) float sOm[NSLOT][NW][L];        // w of the step, one copy per wave
  __shared__ __align__(16) bf16_t sW[NW / 2][4][L];         // w as three bf16 terms and a zero row
  __shared__ float s_mT;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int kr = l16 >> 2, kq = l16 & 3;
  const int sb = wave >> 1;      // rows 64 sb .. 64 sb + 63 of C~
  const int hc = wave & 1;       // columns 64 hc .. 64 hc + 63 of the workgroup's 128

  const int ncol = static_cast<int>(a.dv / TVG);
  const int64_t nblk = a.BH * ncol;
  const int seg = static_cast<int>(blockIdx.x / nblk);
  const int64_t rem = blockIdx.x % nblk;
  // the column blocks of one head on one XCD (block ids equal mod 8) when
  // the head count allows, so their shared K reads meet in one L2
  int64_t head;
  int vt;
  if (a.BH % 8 == 0) {
    const int64_t grp = rem / (8 * ncol), r = rem % (8 * ncol);
    vt = static_cast<int>(r / 8);
    head = grp * 8 + r % 8;
  } else {
    head = rem / ncol;
    vt = static_cast<int>(rem % ncol);
  }
  const int dv = static_cast<int>(a.dv);
  const int nsteps = static_cast<int>(a.Tp / L);
  const int spb = nsteps / a.S;
  const int c0 = seg * spb, c1 = c0 + spb;
  const int qseg = seg / (a.S / a.Q);      // the summary segment of these tokens
  const bool nwave = vt == 0 && hc == 0;   // this wave also forms K^T w for its rows

  const bf16_t* gk = a.k + head * a.Ts * DQK;
  const bf16_t* gv = a.v + head * a.Ts * dv + vt * TVG;
  const float* gw = a.e + head * a.Tp;
  if (tid == 0) {
    double total, emax;
    seg_scalars(a.psum, a.pmax, a.nbk, a.bps, head, qseg, total, emax);
    s_mT = static_cast<float>(emax);
  }

  // loads (per-lane byte offsets fixed, chunk bases wave-uniform): a 1 KB
  // load covers 8 rows of a [64 x 64] tile; lane l writes row 8G + l/8,
  // physical 16-byte chunk l%8, which holds logical chunk (l%8) ^ ((row/2)%8)
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  uint32_t koff[4], voff[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int item = wave * 4 + m;            // 0 .. 31
    const int sub = item / 8, G = item % 8;
    const int row = 8 * G + ld_r;
    koff[m] = static_cast<uint32_t>(2 * (row * DQK + sub * 64 + 8 * (ld_pc ^ ((row >> 1) & 7))));
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int item = wave * 2 + m;            // 0 .. 15
    const int sub = item / 8, G = item % 8;
    const int row = 8 * G + ld_r;
    voff[m] = static_cast<uint32_t>(2 * (row * dv + sub * 64 + 8 * (ld_pc ^ ((row >> 1) & 7))));
  }
  auto issue = [&](auto Sc, int c) {
    constexpr int S = decltype(Sc)::value;
    const int cc = c < c1 ? c : c1 - 1;      // past the segment: a harmless re-read
    const bf16_t* kb = gk + static_cast<int64_t>(cc) * L * DQK;
    const bf16_t* vb = gv + static_cast<int64_t>(cc) * L * dv;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int item = wave * 4 + m;
      dma16_s(kb, koff[m], lds_addr(sK[S][item / 8] + (item % 8) * 1024));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int item = wave * 2 + m;
      dma16_nt_s(vb, voff[m], lds_addr(sV[S][item / 8] + (item % 8) * 1024));
    }
    dma4_s(gw + static_cast<int64_t>(cc) * L, static_cast<uint32_t>(4 * lane),
           lds_addr(&sOm[S][wave][0]));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float nst[4] = {0.f, 0.f, 0.f, 0.f};
  if (nwave) sW[sb][3][lane] = 0;

  static_assert(D == 2 && NSLOT == 3, "the prologue and the unrolled loop assume two steps in flight");
  issue(wave_c<0>{}, c0);
  issue(wave_c<1>{}, c0 + 1);
  __syncthreads();
  const float mT = s_mT;

  // one step of 64 tokens in slot S (the loop is unrolled by the slots, so
  // every LDS address is a fixed per-lane offset)
  auto step = [&](auto Sc, int c) {
    constexpr int S = decltype(Sc)::value;
    // this step's loads were issued D steps ago; (D - 1) NB loads came after
    wait_vm<(D - 1) * NB>();
    __syncthreads();                            // the step's tiles are visible; slot S+2 is free
    issue(wave_c<(S + D) % NSLOT>{}, c + D);
    // w V in place: thread t scales the 16-byte chunk t % 8 of token row t / 8
    // in both column sub-tiles
    {
      const int row = tid >> 3, q = tid & 7;
      const float om = __expf(sOm[S][wave][row] - mT);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        uint4* p = reinterpret_cast<uint4*>(sV[S][sub] + row * 128 + q * 16);
        const uint4 x = *p;
        float f[8];
        f[0] = bf_lo(x.x) * om; f[1] = bf_hi(x.x) * om;
        f[2] = bf_lo(x.y) * om; f[3] = bf_hi(x.y) * om;
        f[4] = bf_lo(x.z) * om; f[5] = bf_hi(x.z) * om;
        f[6] = bf_lo(x.w) * om; f[7] = bf_hi(x.w) * om;
        *p = __builtin_bit_cast(uint4, cvt8(f));
      }
    }
    // w as three bf16 terms (A operand of K^T w: rows 4r + e hold term e)
    uint4 Wx[NKS];
    if (nwave) {
      split3_bf16(__expf(sOm[S][wave][lane] - mT), sW[sb][0][lane], sW[sb][1][lane], sW[sb][2][lane]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Wx[ks] = *reinterpret_cast<const uint4*>(&sW[sb][l16 & 3][32 * ks + 8 * g]);
    }
    __syncthreads();                            // w V is in place
    // K^T fragments of the wave's four row tiles: tile t holds the rows
    // 64 sb + 32 (t/2) + 8 g + 4 (t%2) + e (lane (g, c) of the A operand:
    // d_qk row 64 sb + 32 (t/2) + 8 (c/4) + 4 (t%2) + c%4, tokens 32 ks +
    // 8 g + 0..7)
    bf16x8 Kt[4][NKS], Vf[4][NKS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = 32 * (t >> 1) + 8 * kq + 4 * (t & 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Kt[t][ks] = join(lds_tr(sK[S][sb], swz(32 * ks + 8 * g + kr, col)),
                         lds_tr(sK[S][sb], swz(32 * ks + 8 * g + 4 + kr, col)));
    }
    // (w V) fragments of the wave's four column tiles: lane (g, c) holds
    // column 16 ct + c for tokens 32 ks + 8 g + 0..7
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Vf[ct][ks] = join(lds_tr(sV[S][hc], swz(32 * ks + 8 * g + kr, 16 * ct + 4 * kq)),
                          lds_tr(sV[S][hc], swz(32 * ks + 8 * g + 4 + kr, 16 * ct + 4 * kq)));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc[t][ct] = mfma16x16x32(Kt[t][ks], Vf[ct][ks], acc[t][ct]);
    if (nwave) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 ni = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ni = mfma16x16x32(as_bf16x8(Wx[ks]), Kt[t][ks], ni);
        nst[t] += (ni[0] + ni[1]) + ni[2];
      }
    }
  };
  for (int c = c0; c < c1; c += NSLOT) {
    step(wave_c<0>{}, c);
    if (c + 1 < c1) step(wave_c<1>{}, c + 1);
    if (c + 2 < c1) step(wave_c<2>{}, c + 2);
  }
  // no load may still be in flight when the workgroup ends
  wait_vm<0>();

  float* dst = a.part + (static_cast<int64_t>(seg) * a.BH + head) * DQK * a.dv + vt * TVG + 64 * hc;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 64 * sb + 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dst[static_cast<int64_t>(row) * dv + 16 * ct + l16] = acc[t][ct][e];
    }
  if (nwave && g == 0) {
    float* nd = a.npart + (static_cast<int64_t>(seg) * a.BH + head) * DQK;
#pragma unroll
    for (int t = 0; t < 4; ++t) nd[64 * sb + 32 * (t >> 1) + 8 * (l16 >> 2) + 4 * (t & 1) + (l16 & 3)] = nst[t];
  }
}

// ---- 4. the states at the segment ends.  Per head and segment k: with m
// before it (the initial m, or 0 for a zero state), m' = max(m + sum_k log f,
// m_k), fa = exp(m + sum_k log f - m'), fb = exp(m_k - m'); the state after
// segment k is fa * (state before) + fb * (segment k's summary).
__global__ __launch_bounds__(64) void state_scalars_kernel(const double* psum, const double* pmax,
                                                           int nbk, int bps, int Q, const float* m0,
                                                           float* fab, float* m_out,
                                                           int64_t m_kstride, int64_t BH) {
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  if (bh >= BH) return;
  double m = m0 ? static_cast<double>(m0[bh]) : 0.0;
  for (int k = 0; k < Q; ++k) {
    double total, emax;
    seg_scalars(psum, pmax, nbk, bps, bh, k, total, emax);
    const double md = m + total;
    const double mn = md > emax ? md : emax;
    fab[(bh * Q + k) * 2] = __expf(static_cast<float>(md - mn));
    fab[(bh * Q + k) * 2 + 1] = __expf(static_cast<float>(emax - mn));
    m_out[k * m_kstride + bh] = static_cast<float>(mn);
    m = mn;
  }
}

// C~: one float4 of one head per thread, the Q segment ends in order
__global__ __launch_bounds__(256) void state_scan_c_kernel(const float* part, const float* C0,
                                                           const float* fab, float* C_out,
                                                           int64_t c_kstride, int64_t BH,
                                                           int64_t per_head, int S, int Q) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // float4 index
  const int64_t n4 = BH * per_head / 4;
  if (i4 >= n4) return;
  const int64_t bh = (4 * i4) / per_head;
  const int spq = S / Q;
  float4 r = C0 ? reinterpret_cast<const float4*>(C0)[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < Q; ++k) {
    float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = k * spq; s < (k + 1) * spq; ++s) {
      const float4 x = reinterpret_cast<const float4*>(part)[s * n4 + i4];
      p.x += x.x; p.y += x.y; p.z += x.z; p.w += x.w;
    }
    const float fa = fab[(bh * Q + k) * 2], fb = fab[(bh * Q + k) * 2 + 1];
    r = make_float4(fa * r.x + fb * p.x, fa * r.y + fb * p.y, fa * r.z + fb * p.z, fa * r.w + fb * p.w);
    reinterpret_cast<float4*>(C_out + k * c_kstride)[i4] = r;
  }
}

__global__ __launch_bounds__(DQK) void state_scan_n_kernel(const float* npart, const float* n0,
                                                           const float* fab, float* n_out,
                                                           int64_t n_kstride, int64_t BH, int S, int Q) {
  const int64_t bh = blockIdx.x;
  const int r = threadIdx.x;
  const int spq = S / Q;
  float x = n0 ? n0[bh * DQK + r] : 0.0f;
  for (int k = 0; k < Q; ++k) {
    float p = 0.0f;
    for (int s = k * spq; s < (k + 1) * spq; ++s) p += npart[(s * BH + bh) * DQK + r];
    x = fab[(bh * Q + k) * 2] * x + fab[(bh * Q + k) * 2 + 1] * p;
    n_out[k * n_kstride + bh * DQK + r] = x;
  }
}

struct GemmLayout {
  size_t e, psum, pmax, fab, part, npart, end;
  int S, nbk, bps;
};

GemmLayout gemm_layout(const SeqArgs& a, int Q) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  GemmLayout l{};
  const int64_t BH = a.B * a.H;
  const int64_t groups = BH * (a.dv / TVG);
  const int64_t nsteps = a.T / L;
  int S = Q;
  while (S < kMaxSegments && groups * (2 * S) <= 256 && nsteps % (2 * S) == 0 && nsteps / (2 * S) >= 8)
    S *= 2;
  l.S = S;
  l.nbk = static_cast<int>((a.T + GR - 1) / GR);
  l.bps = Q == 1 ? l.nbk : static_cast<int>(a.T / Q / GR);
  l.e = 0;
  l.psum = up(l.e + 4 * static_cast<size_t>(BH * a.T));
  l.pmax = up(l.psum + 8 * static_cast<size_t>(BH) * l.nbk);
  l.fab = up(l.pmax + 8 * static_cast<size_t>(BH) * l.nbk);
  l.part = up(l.fab + 8 * static_cast<size_t>(BH) * Q);
  l.npart = up(l.part + 4 * static_cast<size_t>(S) * BH * DQK * a.dv);
  l.end = up(l.npart + 4 * static_cast<size_t>(S) * BH * DQK);
  return l;
}

}  // namespace

bool state_gemm_supported(const SeqArgs& a, int Q) {
  if (!(a.qkv_bf16 && a.dqk == DQK && a.dv % TVG == 0 && a.T % L == 0 && a.t0 == 0 && a.Ts % 4 == 0 &&
        Q >= 1 && Q <= kMaxSegments))
    return false;
  if (a.T < 8 * L * Q) return false;
  // several summary segments: whole gate blocks and whole 64-token steps each
  return Q == 1 || (a.T % Q == 0 && (a.T / Q) % GR == 0);
}

size_t state_gemm_workspace(const SeqArgs& a, int Q) { return gemm_layout(a, Q).end; }

hipError_t launch_state_gemm(const SeqArgs& a, int Q, float* C_out, float* n_out, float* m_out,
                             void* workspace, hipStream_t stream) {
  const GemmLayout l = gemm_layout(a, Q);
  char* w = static_cast<char*>(workspace);
  const int64_t BH = a.B * a.H;
  float* ev = reinterpret_cast<float*>(w + l.e);
  double* psum = reinterpret_cast<double*>(w + l.psum);
  double* pmax = reinterpret_cast<double*>(w + l.pmax);
  float* fab = reinterpret_cast<float*>(w + l.fab);
  float* part = reinterpret_cast<float*>(w + l.part);
  float* npart = reinterpret_cast<float*>(w + l.npart);
  const unsigned ngb = static_cast<unsigned>(BH * l.nbk);
  state_gsum_kernel<<<dim3(ngb), dim3(GT), 0, stream>>>(a, psum, l.nbk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  state_gexp_kernel<<<dim3(ngb), dim3(GT), 0, stream>>>(a, psum, ev, pmax, l.nbk, l.bps);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmArgs g{};
  g.BH = BH; g.Tp = a.T; g.Ts = a.Ts; g.dv = a.dv; g.S = l.S; g.Q = Q; g.nbk = l.nbk; g.bps = l.bps;
  g.k = static_cast<const bf16_t*>(a.k);
  g.v = static_cast<const bf16_t*>(a.v);
  g.e = ev; g.psum = psum; g.pmax = pmax;
  g.part = part; g.npart = npart;
  const unsigned nwg = static_cast<unsigned>(BH * (a.dv / TVG) * l.S);
  state_gemm_kernel<<<dim3(nwg), dim3(NTH), 0, stream>>>(g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  state_scalars_kernel<<<dim3(static_cast<unsigned>((BH + 63) / 64)), dim3(64), 0, stream>>>(
      psum, pmax, l.nbk, l.bps, Q, a.C0 ? a.m0 : nullptr, fab, m_out, BH, BH);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_head = DQK * a.dv;
  const int64_t n4 = BH * per_head / 4;
  state_scan_c_kernel<<<dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, stream>>>(
      part, a.C0, fab, C_out, BH * per_head, BH, per_head, l.S, Q);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  state_scan_n_kernel<<<dim3(static_cast<unsigned>(BH)), dim3(DQK), 0, stream>>>(
      npart, a.C0 ? a.n0 : nullptr, fab, n_out, BH * DQK, BH, l.S, Q);
  return hipGetLastError();
}

}  // namespace mlstm
