// State-only chunkwise pass: the state (C~, n~, m) after T tokens of every
// head, from a given initial state, with no outputs.  It carries the state
// across the first half of a long sequence so that the forward kernels can
// run both halves at once (see the sequence split in api.hip).
//
// Method: xLSTM post (llms.blog), section 3 "Associative Matrix Cell State"
// (C_t = f_t C_{t-1} + i_t v_t k_t^T, n_t = f_t n_{t-1} + i_t k_t) with the
// running maximum of section 2 "The Normalizer State and Numerical
// Stabilization", applied a chunk of 64 tokens at a time as in section 3 "The
// Parallel Dual Form" split at chunk boundaries: with chunk-local cumulative
// log forget gates b_j and u_j = i~_j - b_j,
//   M = max(m_s, max_j u_j),  g_L = exp(m_s - M),  w_j = exp(u_j - M),
//   C~ <- g_L C~ + K^T diag(w) V,  n~ <- g_L n~ + K^T w,  m <- b_L + M.
// The result does not depend on the chunk length beyond rounding.
//
// Design (CDNA4): one workgroup of 8 waves per (head, 32 value columns): the
// pass runs where the forward's grid leaves compute units idle, so it uses
// twice as many workgroups.  Wave w keeps 16 columns (w % 2) of C~ for a
// quarter of the d_qk rows (w / 2) in float32 registers with a lazy scale
// (C~ = sig * acc, as in the forward kernels), and the n~ rows of half of its
// row tiles; two waves share each SIMD, so one wave's LDS and MFMA latencies
// overlap the other's work.  Every wave loads an eighth of each chunk's K
// tile and of the 64-column V block that holds the workgroup's columns (and
// its own copy of the next chunk's gates), global -> LDS through a ring of 3
// chunk slots, two chunks ahead; one barrier per chunk publishes a slot.
// Every wave runs the gate scan itself (DPP scans, so no gate values cross
// waves), one chunk ahead: the scan of chunk c + 1 depends only on its gates
// and on m after chunk c, so it runs beside chunk c's products instead of
// before them.  The update K^T (w V) runs on bf16 MFMA with the K^T fragments
// read with the LDS transpose read; the n~ increment K^T w on MFMA with w
// split into three bf16 terms (about 24 bits), as in the forward kernel.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int NW = 8;
constexpr int NTH = 512;
constexpr int TV = 32;            // value columns per workgroup
constexpr int L = 64;             // tokens per chunk
constexpr int NKS = L / 32;       // 32-token MFMA k-steps
constexpr int SUBT = L * 128;     // one [64 tokens x 64] bf16 tile (128-byte rows)
constexpr int D = 2;              // chunks in flight
constexpr int NSLOT = D + 1;

template <int DQK>
__global__ __launch_bounds__(NTH, 1) void chunk_state_kernel(SeqArgs a) {
  constexpr int NSUB = DQK / 64;          // 64-wide d_qk sub-tiles of K
  constexpr int NCTW = DQK / 64;          // 16-row C~ tiles per wave (a quarter of the rows)
  constexpr int NB_K = NSUB;              // 1 KB K loads per wave per chunk
  constexpr int NB = NB_K + 1 + 2;        // + one V load and the wave's two gate loads
  __shared__ __align__(1024) char sK[NSLOT][NSUB][SUBT];
  __shared__ __align__(1024) char sV[NSLOT][SUBT];
  __shared__ __align__(256) float sG[NSLOT][NW][2][L];   // raw gates, one copy per wave
  // per slot: w as three bf16 terms + a zero row, and w / sig' (the update's
  // scale); wave-private
  __shared__ __align__(16) bf16_t sW[NSLOT][NW][4][L];
  __shared__ __align__(16) float sWv[NSLOT][NW][L];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int cgw = wave & 1;               // 16-column group
  const int rq = wave >> 1;               // quarter of the d_qk rows

  const int nvt = static_cast<int>(a.dv / TV);
  const int64_t nhead = a.B * a.H;
  int64_t head;
  int vt;
  {
    // the column tiles of one head on one XCD (block ids equal mod 8), so
    // their shared K reads meet in one L2
    const int64_t w = blockIdx.x;
    if (nhead % 8 == 0) {
      const int64_t grp = w / (8 * nvt), r = w % (8 * nvt);
      vt = static_cast<int>(r / 8);
      head = grp * 8 + r % 8;
    } else {
      head = w / nvt;
      vt = static_cast<int>(w % nvt);
    }
  }
  const int dv = static_cast<int>(a.dv);
  const int64_t Ts = a.Ts;
  const int nchunks = static_cast<int>(a.T / L);
  const int vcol = 32 * (vt & 1) + 16 * cgw;      // this wave's columns in the 64-column V block
  const int b0w = 64 * (vt >> 1) + vcol;          // ... and in the head
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * Ts * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * Ts * dv + 64 * (vt >> 1);
  const float* gi = a.i_pre + head * Ts;
  const float* gf = a.f_pre + head * Ts;

  // ---- loads: an eighth of the K tile and of the V block of chunk c, and
  // this wave's own copy of the gates of chunk c + 1.  A 1 KB load covers 8
  // rows of a [64 x 64] tile: lane l writes row 8G + l/8, physical 16-byte
  // chunk l%8, which holds the logical chunk (l%8) ^ ((row/2)%8) (the swz
  // layout).  Each load takes a wave-uniform chunk base (SGPRs) and a fixed
  // per-lane byte offset, so no lane computes a 64-bit address per chunk.
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  uint32_t koff[NB_K];
#pragma unroll
  for (int m = 0; m < NB_K; ++m) {
    const int item = wave * NB_K + m;             // 0 .. 8 NSUB - 1
    const int sb = item / 8, G = item % 8;
    const int row = 8 * G + ld_r;
    koff[m] = static_cast<uint32_t>(2 * (row * DQK + sb * 64 + 8 * (ld_pc ^ ((row >> 1) & 7))));
  }
  const uint32_t voff = static_cast<uint32_t>(
      2 * ((8 * wave + ld_r) * dv + 8 * (ld_pc ^ (((8 * wave + ld_r) >> 1) & 7))));
  const uint32_t goff = static_cast<uint32_t>(4 * lane);
  auto issue_gates = [&](auto Sg, int c) {
    constexpr int S = decltype(Sg)::value;
    const int cc = c < nchunks ? c : nchunks - 1;   // past the end: a harmless re-read
    dma4_s(gi + static_cast<int64_t>(cc) * L, goff, lds_addr(&sG[S][wave][0][0]));
    dma4_s(gf + static_cast<int64_t>(cc) * L, goff, lds_addr(&sG[S][wave][1][0]));
  };
  // chunk c into slot S (= c % NSLOT), and the gates of chunk c + 1
  auto issue_chunk = [&](auto Sc, int c) {
    constexpr int S = decltype(Sc)::value;
    const int cc = c < nchunks ? c : nchunks - 1;
    const bf16_t* kb = gk + static_cast<int64_t>(cc) * L * DQK;
#pragma unroll
    for (int m = 0; m < NB_K; ++m) {
      const int item = wave * NB_K + m;
      const int sb = item / 8, G = item % 8;
      dma16_s(kb, koff[m], lds_addr(sK[S][sb] + G * 1024));
    }
    dma16_s(gv + static_cast<int64_t>(cc) * L * dv, voff, lds_addr(sV[S] + wave * 1024));
    issue_gates(wave_c<(S + 1) % NSLOT>{}, c + 1);
  };

  // ---- state.  The wave's C~ tiles are the 16-row tiles T = rq NCTW + t
  // (t = 0 .. NCTW-1) of the d_qk rows, all in the K sub-tile T / 4; tile T
  // holds the rows 32 (T/2) + 8 g + 4 (T%2) + e (the row order in which the
  // update's output lands, see the K^T fragments below).
  auto arow_of = [&](int t, int e) {
    const int T = rq * NCTW + t;
    return 32 * (T >> 1) + 8 * g + 4 * (T & 1) + e;
  };
  f32x4 cacc[NCTW];
#pragma unroll
  for (int t = 0; t < NCTW; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      cacc[t][e] = a.C0 ? a.C0[(head * DQK + arow_of(t, e)) * dv + b0w + l16] : 0.0f;
  }
  // n~: the wave keeps the rows of its tiles T with T % 2 == cgw (so each
  // tile's rows are kept by one wave); lane l holds the row 32 (T/2) +
  // 8 (l16/4) + 4 (T%2) + l16%4 of tile T (the column order of the K^T
  // fragment used as the B operand below)
  auto n_tile = [&](int t) { return ((rq * NCTW + t) & 1) == cgw; };
  auto nrow_of = [&](int t) {
    const int T = rq * NCTW + t;
    return 32 * (T >> 1) + 8 * (l16 >> 2) + 4 * (T & 1) + (l16 & 3);
  };
  float nst[NCTW];
#pragma unroll
  for (int t = 0; t < NCTW; ++t) nst[t] = (a.C0 && n_tile(t)) ? a.n0[head * DQK + nrow_of(t)] : 0.0f;
  float m_s = a.C0 ? a.m0[head] : 0.0f;
  float sig = 1.0f;
#pragma unroll
  for (int s = 0; s < NSLOT; ++s) sW[s][wave][3][lane] = 0;
  // the initial-state loads complete here, before any load of the ring:
  // otherwise the compiler, which does not see the asm loads, waits for every
  // outstanding load (vmcnt(0), a drain of the ring) at the first use of the
  // state inside the chunk loop
  wait_vm<0>();

  // Gate scan of chunk c (this wave's copy, slot S = c % NSLOT; lane j =
  // token j): writes w (three terms) and w / sig' into the wave's buffers of
  // slot S, and returns g_L and whether the accumulators take the scale,
  // advancing m and sig to their values after the chunk.
  auto scan = [&](auto Sc, float& gL, bool& renorm) {
    constexpr int S = decltype(Sc)::value;
    const float xi = sG[S][wave][0][lane];
    const float lf = log_forget_fast(sG[S][wave][1][lane], a.fgate_exp);
    const float bcum = scan_add(lf);
    const float u = xi - bcum;
    const float Mx = fmaxf(m_s, scan_max(u));
    const float ML = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Mx), L - 1));
    const float bL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bcum), L - 1));
    gL = __expf(m_s - ML);
    const float wj = __expf(u - ML);
    // lazy scale: C~_new = g_L C~ + K^T (w V) = sig' (acc + K^T ((w / sig') V)),
    // sig' = g_L sig; when sig' gets tiny the accumulators take g_L sig
    renorm = gL * sig < 0x1p-64f;
    const float sig_new = renorm ? 1.0f : gL * sig;
    split3_bf16(wj, sW[S][wave][0][lane], sW[S][wave][1][lane], sW[S][wave][2][lane]);
    sWv[S][wave][lane] = wj * __builtin_amdgcn_rcpf(sig_new);
    m_s = bL + ML;
    sig = sig_new;
  };

  // ---- prologue: the gates of chunk 0, then chunks 0 .. D-1 (with the
  // gates of chunks 1 .. D) in flight; chunk 0's scan once its gates land
  static_assert(D == 2 && NSLOT == 3, "the prologue and the unrolled loop assume two chunks in flight");
  issue_gates(wave_c<0>{}, 0);
  issue_chunk(wave_c<0>{}, 0);
  issue_chunk(wave_c<1>{}, 1);
  wait_vm<D * NB>();
  // gL, renorm: chunk c's, from its scan; sig_prev, m_prev: the scale and
  // m before chunk c while it is processed (after it, once the loop ends)
  float gL = 1.0f, sig_prev = 1.0f, m_prev = m_s;
  bool renorm = false;
  scan(wave_c<0>{}, gL, renorm);

  const int kr = l16 >> 2, kq = l16 & 3;
  // one chunk; the slot S = c % NSLOT is a compile-time constant (the loop
  // is unrolled by NSLOT), so every LDS address is a fixed per-lane offset
  auto chunk_step = [&](auto Sc, int c) {
    constexpr int S = decltype(Sc)::value;
    // chunk c's loads (and the gates of chunk c + 1) were issued D chunks
    // ago; (D - 1) NB loads of this wave came after them
    wait_vm<(D - 1) * NB>();
    __syncthreads();
    issue_chunk(wave_c<(S + D) % NSLOT>{}, c + D);   // into the slot of chunk c - 1, which every wave has left

    // w (three terms) as the A operand of the n~ increment, and w / sig' for
    // this lane's tokens 32 ks + 8 g + 0..7 (wave-private LDS, written by the
    // scan of this chunk one iteration earlier)
    uint4 Wx[NKS];
    bf16x8 wVf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      Wx[ks] = *reinterpret_cast<const uint4*>(&sW[S][wave][l16 & 3][32 * ks + 8 * g]);
      const float4 w0 = *reinterpret_cast<const float4*>(&sWv[S][wave][32 * ks + 8 * g]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sWv[S][wave][32 * ks + 8 * g + 4]);
      // V^T fragment of this wave's 16 columns: lane (g, c) gets column c
      // for tokens 32 ks + 8 g + 0..7
      const int col = vcol + 4 * kq;
      const uint2 lo = lds_tr(sV[S], swz(32 * ks + 8 * g + kr, col));
      const uint2 hi = lds_tr(sV[S], swz(32 * ks + 8 * g + 4 + kr, col));
      float xw[8];
      xw[0] = bf_lo(lo.x) * w0.x; xw[1] = bf_hi(lo.x) * w0.y;
      xw[2] = bf_lo(lo.y) * w0.z; xw[3] = bf_hi(lo.y) * w0.w;
      xw[4] = bf_lo(hi.x) * w1.x; xw[5] = bf_hi(hi.x) * w1.y;
      xw[6] = bf_lo(hi.y) * w1.z; xw[7] = bf_hi(hi.y) * w1.w;
      wVf[ks] = cvt8(xw);
    }
    if (renorm) {
      const float f = gL * sig_prev;
#pragma unroll
      for (int t = 0; t < NCTW; ++t) cacc[t] *= f;
    }
    const float gLc = gL;

    // ---- update of the wave's tiles.  The A operand of C~ tile T (sub-tile
    // sb = T/4, tl = T%4) is the K^T fragment: lane (g, c) holds the d_qk row
    // 64 sb + 32 (tl/2) + 8 (c/4) + 4 (tl%2) + c%4 for tokens 32 ks + 8 g +
    // 0..7 (two transposed reads of 4 tokens each).  As a B operand the same
    // fragment gives the n~ increment of those rows, with the three terms of
    // w in rows 4r..4r+2 of the A operand: D[4r + e][c] is term e of
    // (K^T w)[row c].
#pragma unroll
    for (int t = 0; t < NCTW; ++t) {
      const int T = rq * NCTW + t;
      const char* Kb = sK[S][T >> 2];
      const int tl = T & 3;
      const int col = 32 * (tl >> 1) + 8 * kq + 4 * (tl & 1);
      uint2 Klo[NKS], Khi[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Klo[ks] = lds_tr(Kb, swz(32 * ks + 8 * g + kr, col));
        Khi[ks] = lds_tr(Kb, swz(32 * ks + 8 * g + 4 + kr, col));
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        cacc[t] = mfma16x16x32(join(Klo[ks], Khi[ks]), wVf[ks], cacc[t]);
      if (n_tile(t)) {
        f32x4 ni = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          ni = mfma16x16x32(as_bf16x8(Wx[ks]), join(Klo[ks], Khi[ks]), ni);
        nst[t] = gLc * nst[t] + ((ni[0] + ni[1]) + ni[2]);
      }
    }
    // ---- the next chunk's gate scan (its gates landed with this chunk's
    // loads); it reads nothing this chunk's products write
    sig_prev = sig;
    m_prev = m_s;
    scan(wave_c<(S + 1) % NSLOT>{}, gL, renorm);
  };
  for (int c = 0; c < nchunks; c += NSLOT) {
    chunk_step(wave_c<0>{}, c);
    if (c + 1 < nchunks) chunk_step(wave_c<1>{}, c + 1);
    if (c + 2 < nchunks) chunk_step(wave_c<2>{}, c + 2);
  }
  // no LDS load may still be in flight when the workgroup ends
  wait_vm<0>();
  __syncthreads();

  // ---- final state (sig_prev, m_prev: after the last chunk; the scan past
  // the end changed only values that are not used)
#pragma unroll
  for (int t = 0; t < NCTW; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a.C1[(head * DQK + arow_of(t, e)) * dv + b0w + l16] = cacc[t][e] * sig_prev;
  }
  if (vt == 0) {
    if (g == 0) {
#pragma unroll
      for (int t = 0; t < NCTW; ++t)
        if (n_tile(t)) a.n1[head * DQK + nrow_of(t)] = nst[t];
    }
    if (tid == 0) a.m1[head] = m_prev;
  }
}

}  // namespace

bool chunk_state_supported(const SeqArgs& a) {
  return a.qkv_bf16 && (a.dqk == 64 || a.dqk == 128 || a.dqk == 256) && a.dv % 64 == 0 &&
         a.T % L == 0 && a.T > 0;
}

hipError_t launch_chunk_state(const SeqArgs& a, hipStream_t stream) {
  const unsigned nwg = static_cast<unsigned>(a.B * a.H * (a.dv / TV));
  switch (a.dqk) {
    case 64: chunk_state_kernel<64><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    case 128: chunk_state_kernel<128><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
    default: chunk_state_kernel<256><<<dim3(nwg), dim3(NTH), 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace mlstm
