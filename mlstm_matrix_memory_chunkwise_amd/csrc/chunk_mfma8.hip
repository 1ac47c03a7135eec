// Fused chunkwise mLSTM forward, bf16 MFMA, chunk 64, two waves per SIMD.
//
// Method: xLSTM post (llms.blog), section 3 "The Parallel Dual Form" inside
// chunks of 64 tokens, the state of "Associative Matrix Cell State" carried
// between chunks, the running maximum of section 2 "The Normalizer State and
// Numerical Stabilization".  The chunk algebra is the same as in
// chunk_mfma.hip:
//   u_j = i~_j - b_j,  M_i = max(m_s, max_{j<=i} u_j),  m_i = b_i + M_i
//   D_ij = exp(u_j - M_i),  g_i = exp(m_s - M_i),  w_j = exp(u_j - M_L)
//   h_i = sigmoid(o~_i) (.) (g_i q_i^T C~_s + sum_j D_ij (q_i.k_j) v_j)
//         / max(|g_i q_i.n~_s + sum_j D_ij (q_i.k_j)|, exp(-m_i))
//   C~ <- g_L C~ + K^T diag(w) V,  n~ <- g_L n~ + K^T w.
//
// Work split (the reason for this kernel).  With one wave per SIMD every
// LDS-read latency before an MFMA is exposed.  Here a workgroup has 8 waves
// for the same 64 value columns: wave w owns columns 16 (w % 4) .. +15 and,
// of every 64-row d_qk slice, the 32 rows of k-step h = w / 4.  The two
// waves on a SIMD (w and w + 4) therefore always have independent work.  Per
// d_qk slice each wave does its half of the readout C~^T Q^T, of the score
// tiles S^T = K Q^T and of q.n~ (partial sums over its 32 rows), and the
// state update of its own 32 rows of C~.  Once per chunk the partial sums
// meet in LDS: the two waves of a column group each finish half of the query
// tiles, and the score tiles are finished by alternating owners.
//
// Loads, layouts and the lazily scaled state (C~ = sig * acc) are as in
// chunk_mfma.hip: all loop loads are global->LDS DMA from asm with explicit
// compile-time vmcnt waits, tiles are row-major with swizzled 16-byte chunks,
// token-contracted operands come from ds_read_b64_tr_b16.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mlstm {
namespace {

using namespace mk;

constexpr int NW = 8;        // waves per workgroup
constexpr int NTH = 512;
constexpr int TV = 64;       // value columns per workgroup
constexpr int AS = 64;       // d_qk slice (stage) width
constexpr int L = 64;        // chunk
constexpr int NT = L / 16;   // 16-token tiles
constexpr int NKS = L / 32;  // 32-token k-steps
constexpr int NTILES = NT * (NT + 1) / 2;
constexpr int TILE = L * 128;   // one [64 x 64] bf16 tile
constexpr int PROW = L + 8;

template <int DQK, int OM>
struct C8 {
  static constexpr int NS = DQK / AS;
  static constexpr int D = 3 < NS ? 3 : NS;         // stages in flight
  static constexpr int NSLOT = D + 1;
  static constexpr int VSLOT = (D <= NS - 1) ? 1 : 2;
  static constexpr int OROW = (OM == O_BF16) ? 128 : 256;
  static constexpr int OTILE = (OM == O_NONE) ? 16 : L * OROW;
  static constexpr int NB_QK = 2 * TILE / 1024 / NW;   // 2
  static constexpr int NB_V = TILE / 1024 / NW;        // 1
  static constexpr int NB_O = (OM == O_NONE) ? 0 : L * OROW / 1024 / NW;
  static constexpr int NB_G = 2;
  static constexpr int NB_X = NB_O + NB_G;
  static_assert(DQK % AS == 0 && NS <= 4, "d_qk must be 64, 128, 192 or 256");
};

template <int DQK, int OM>
__global__ __launch_bounds__(NTH, 1) void chunk_mfma8_kernel(SeqArgs a) {
  using C = C8<DQK, OM>;
  __shared__ __align__(1024) char sRing[C::NSLOT][2][TILE];   // [slot][q|k]
  __shared__ __align__(1024) char sV[C::VSLOT][TILE];
  __shared__ __align__(1024) char sO[C::OTILE];
  __shared__ __align__(16) bf16_t sP[L * PROW];
  __shared__ __align__(16) float sSx[NTILES][64][4];          // score partials
  __shared__ __align__(16) float sOx[4][NT][64][4];           // readout partials
  // per chunk parity: u, M, g, w, exp(-m), w / sig'
  __shared__ __align__(16) float sGate[2][6][L];
  __shared__ float sRs[NW][L];
  __shared__ float sQn[2][L];
  __shared__ __align__(16) float sN[DQK];
  __shared__ float sNp[DQK];   // n~ increments over the chunk's second k-step
  __shared__ __align__(256) float sGin[2][2][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int cg = wave & 3;     // column group
  const int hh = wave >> 2;    // k-step half of every d_qk slice

  const int nvt = static_cast<int>(a.dv / TV);
  const int64_t nhead = a.B * a.H;
  int64_t head;
  int vt;
  {
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
  const int64_t T = a.T, Ts = a.Ts;   // tokens per head; token stride between heads
  const int nchunks = static_cast<int>(T / L);
  const int b0w = vt * TV + cg * 16;

  const bf16_t* gq = static_cast<const bf16_t*>(a.q) + head * Ts * DQK;
  const bf16_t* gk = static_cast<const bf16_t*>(a.k) + head * Ts * DQK;
  const bf16_t* gv = static_cast<const bf16_t*>(a.v) + head * Ts * dv + vt * TV;
  const float* gi = a.i_pre + head * Ts;
  const float* gf = a.f_pre + head * Ts;
  bf16_t* gh = static_cast<bf16_t*>(a.h) + head * Ts * dv + b0w + 4 * g;

  // ---- state: C~ rows of k-step half hh of every slice (tile pair 2s + hh)
  f32x4 cacc[C::NS][2];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int arow = 32 * (2 * s + hh) + 8 * g + 4 * e2 + e;
        cacc[s][e2][e] = a.C0 ? a.C0[(head * DQK + arow) * dv + b0w + l16] : 0.0f;
      }
    }
  }
  if (tid < DQK) sN[tid] = a.C0 ? a.n0[head * DQK + tid] : 0.0f;
  float m_s = a.C0 ? a.m0[head] : 0.0f;

  // ---- loads
  const int ld_r = lane >> 3, ld_pc = lane & 7;
  int qk_off[C::NB_QK];
#pragma unroll
  for (int m = 0; m < C::NB_QK; ++m) {
    const int Gr = (wave * C::NB_QK + m) % (L / 8);
    const int row = 8 * Gr + ld_r;
    qk_off[m] = row * DQK + 8 * (ld_pc ^ ((row >> 1) & 7));
  }
  const int v_row = 8 * wave + ld_r;
  const int v_off = v_row * dv + 8 * (ld_pc ^ ((v_row >> 1) & 7));
  auto issue_stage = [&](int x) {
    const int cx = x / C::NS, sx = x % C::NS;
    const int cc = cx < nchunks ? cx : nchunks - 1;    // past the end: harmless re-read
    char* slot = sRing[x % C::NSLOT][0];
    const int64_t base = static_cast<int64_t>(cc) * L * DQK + sx * AS;
#pragma unroll
    for (int m = 0; m < C::NB_QK; ++m) {
      const int G = wave * C::NB_QK + m;
      const int mat = G / (L / 8);
      dma16((mat ? gk : gq) + base + qk_off[m], lds_addr(slot + mat * TILE + (G % (L / 8)) * 1024));
    }
    if (sx == 0)
      dma16(gv + static_cast<int64_t>(cc) * L * dv + v_off, lds_addr(sV[cx % C::VSLOT] + wave * 1024));
  };
  auto issue_chunk_extras = [&](int c) {
    if (OM != O_NONE) {
      constexpr int RPI = 1024 / C::OROW;
      constexpr int NCH = C::OROW / 16;
#pragma unroll
      for (int m = 0; m < C::NB_O; ++m) {
        const int G = wave * C::NB_O + m;
        const int row = RPI * G + lane / NCH;
        const int pc = lane % NCH;
        const int lc = (OM == O_F32) ? (pc ^ (row & 15)) : (pc ^ ((row >> 1) & 7));
        const int64_t r = head * Ts + static_cast<int64_t>(c) * L + row;
        const char* src = (OM == O_F32)
            ? reinterpret_cast<const char*>(static_cast<const float*>(a.o_pre) + r * dv + vt * TV + 4 * lc)
            : reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.o_pre) + r * dv + vt * TV + 8 * lc);
        dma16(src, lds_addr(sO + G * 1024));
      }
    }
    const int cn = (c + 2 < nchunks) ? c + 2 : nchunks - 1;
    dma4(gi + static_cast<int64_t>(cn) * L + lane, lds_addr(&sGin[c & 1][0][0]));
    dma4(gf + static_cast<int64_t>(cn) * L + lane, lds_addr(&sGin[c & 1][1][0]));
  };

  // Gate scan of one chunk (wave 0), DPP scans; returns m after the chunk.
  // sg is the state scale before the chunk; the update weights are stored
  // already divided by the scale after it (the same expression as the loop).
  auto scan_gates = [&](int par, float ms, float sg) {
    const float lf = log_forget_fast(sGin[par][1][lane], a.fgate_exp);
    const float bcum = scan_add(lf);
    const float u = sGin[par][0][lane] - bcum;
    const float Mx = fmaxf(ms, scan_max(u));
    const float ML = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Mx), L - 1));
    const float bL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bcum), L - 1));
    const float gv = __expf(ms - Mx);
    const float wv = __expf(u - ML);
    const float gLn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv), L - 1));
    const float sg_new = gLn * sg < 0x1p-64f ? 1.0f : gLn * sg;
    sGate[par][0][lane] = u;
    sGate[par][1][lane] = Mx;
    sGate[par][2][lane] = gv;
    sGate[par][3][lane] = wv;
    sGate[par][4][lane] = __expf(-(bcum + Mx));
    sGate[par][5][lane] = wv * (1.0f / sg_new);
    return bL + ML;
  };

  // ---- prologue
#pragma unroll
  for (int x = 0; x < C::D; ++x) issue_stage(x);
  dma4(gi + lane, lds_addr(&sGin[0][0][0]));
  dma4(gf + lane, lds_addr(&sGin[0][1][0]));
  dma4(gi + (nchunks > 1 ? L : 0) + lane, lds_addr(&sGin[1][0][0]));
  dma4(gf + (nchunks > 1 ? L : 0) + lane, lds_addr(&sGin[1][1][0]));
  wait_vm<0>();
  float m_next = 0.0f;
  if (wave == 0) m_next = scan_gates(0, m_s, 1.0f);
  __syncthreads();
  float sig = 1.0f;   // C~ = sig * cacc

  f32x4 outT[NT];
  f32x4 sacc[3];
  bf16x8 Vf[NKS];
  bf16x8 wVf[NKS];
  float nn[C::NS];
  float qnp = 0.0f;

  for (int c = 0; c < nchunks; ++c) {
    const int par = c & 1;
    const float gL = sGate[par][2][L - 1];
    const bool renorm = gL * sig < 0x1p-64f;
    const float sig_new = renorm ? 1.0f : gL * sig;

#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const int x = c * C::NS + s;
      if (x < C::D) wait_vm<0>();
      else wait_stage<C::NS, C::D, C::NB_QK, C::NB_V, C::NB_X>(s);
      __syncthreads();
      issue_stage(x + C::D);
      if (s == 0) issue_chunk_extras(c);
      const char* Qb = sRing[x % C::NSLOT][0];
      const char* Kb = sRing[x % C::NSLOT][1];

      if (s == 0) {
        const char* Vb = sV[c % C::VSLOT];
        const int vr = l16 >> 2, vq = l16 & 3;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int col = cg * 16 + 4 * vq;
          const uint2 lo = lds_tr(Vb, swz(32 * ks + 8 * g + vr, col));
          const uint2 hi = lds_tr(Vb, swz(32 * ks + 8 * g + 4 + vr, col));
          Vf[ks] = join(lo, hi);
          const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][5][32 * ks + 8 * g]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][5][32 * ks + 8 * g + 4]);
          float xw[8];
          xw[0] = bf_lo(lo.x) * w0.x; xw[1] = bf_hi(lo.x) * w0.y;
          xw[2] = bf_lo(lo.y) * w0.z; xw[3] = bf_hi(lo.y) * w0.w;
          xw[4] = bf_lo(hi.x) * w1.x; xw[5] = bf_hi(hi.x) * w1.y;
          xw[6] = bf_lo(hi.y) * w1.z; xw[7] = bf_hi(hi.y) * w1.w;
          wVf[ks] = cvt8(xw);
        }
#pragma unroll
        for (int it = 0; it < NT; ++it) outT[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 3; ++k) sacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        qnp = 0.0f;
      }

      // ---- this wave's k-step (rows 32 hh .. +31 of the slice)
      const int P = 2 * s + hh;   // C~ tile pair
      float ca[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ca[e] = cacc[s][0][e];
        ca[4 + e] = cacc[s][1][e];
      }
      // C~ as a (high, remainder) pair of bf16 operands (see cvt8_split)
      bf16x8 A_hi, A_lo;
      cvt8_split(ca, A_hi, A_lo);
      uint4 Qf[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        Qf[it] = lds_ld16(Qb, swz(it * 16 + l16, 32 * hh + 8 * g));
        outT[it] = mfma16x16x32(A_hi, as_bf16x8(Qf[it]), outT[it]);
        outT[it] = mfma16x16x32(A_lo, as_bf16x8(Qf[it]), outT[it]);
      }
      const float4 n0v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g]);
      const float4 n1v = *reinterpret_cast<const float4*>(&sN[32 * P + 8 * g + 4]);
      for_wave<NW>(wave, [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
        constexpr int CG = W & 3;
        // q . n~ for query tile CG over this wave's rows
        qnp += bf_lo(Qf[CG].x) * n0v.x + bf_hi(Qf[CG].x) * n0v.y +
               bf_lo(Qf[CG].y) * n0v.z + bf_hi(Qf[CG].y) * n0v.w +
               bf_lo(Qf[CG].z) * n1v.x + bf_hi(Qf[CG].z) * n1v.y +
               bf_lo(Qf[CG].w) * n1v.z + bf_hi(Qf[CG].w) * n1v.w;
        // score tiles n = CG, CG+4, CG+8 over this wave's k-step
#pragma unroll
        for (int it = 0; it < NT; ++it) {
#pragma unroll
          for (int jt = 0; jt <= it; ++jt) {
            const int n = it * (it + 1) / 2 + jt;
            if (n % 4 == CG) {
              const uint4 Kf = lds_ld16(Kb, swz(jt * 16 + l16, 32 * (W >> 2) + 8 * g));
              sacc[n / 4] = mfma16x16x32(as_bf16x8(Kf), as_bf16x8(Qf[it]), sacc[n / 4]);
            }
          }
        }
      });

      // ---- state update of this wave's 32 rows.  n~ increment: the four
      // waves of a half split its 2 row tiles x 2 token k-steps (tile W & 1,
      // k-step (W & 3) / 2); the two k-step partials of a row meet in LDS.
      if (renorm) {
        const float f = gL * sig;
        cacc[s][0] *= f;
        cacc[s][1] *= f;
      }
      const int kr = l16 >> 2, kq = l16 & 3;
      float npart = 0.0f;
      for_wave<NW>(wave, [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
        constexpr int H = W >> 2;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int col = 32 * H + 8 * kq + 4 * e2;
            const uint2 lo = lds_tr(Kb, swz(32 * ks + 8 * g + kr, col));
            const uint2 hi = lds_tr(Kb, swz(32 * ks + 8 * g + 4 + kr, col));
            cacc[s][e2] = mfma16x16x32(join(lo, hi), wVf[ks], cacc[s][e2]);
            if (e2 == (W & 1) && ks == ((W & 3) >> 1)) {
              const float4 w0 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g]);
              const float4 w1 = *reinterpret_cast<const float4*>(&sGate[par][3][32 * ks + 8 * g + 4]);
              npart += bf_lo(lo.x) * w0.x + bf_hi(lo.x) * w0.y + bf_lo(lo.y) * w0.z + bf_hi(lo.y) * w0.w +
                       bf_lo(hi.x) * w1.x + bf_hi(hi.x) * w1.y + bf_lo(hi.y) * w1.z + bf_hi(hi.y) * w1.w;
            }
          }
        }
      });
      nn[s] = sum_groups(npart);
    }

    // ================= end of chunk
    wait_vm<C::NB_G + loads_after_chunk_extras<C::NS, C::D, C::NB_QK, C::NB_V>()>();
    const float m_cur = m_next;
    if (wave == 0) m_next = scan_gates(par ^ 1, m_cur, sig_new);

    // partial sums out: q.n~, n~ increments of the second k-step, score tiles
    // finished by the other half, readout tiles finished by the other half
    // (query tile it is finished by half it/2)
    if (cg >= 2 && g == 0) {
#pragma unroll
      for (int s = 0; s < C::NS; ++s)
        sNp[s * AS + 32 * hh + 8 * (l16 >> 2) + 4 * (cg & 1) + (l16 & 3)] = nn[s];
    }
    {
      const float qv = sum_groups(qnp);
      if (g == 0) sQn[hh][cg * 16 + l16] = qv;
    }
    for_wave<NW>(wave, [&](auto Wc) {
      constexpr int W = decltype(Wc)::value;
      constexpr int CG = W & 3, H = W >> 2;
#pragma unroll
      for (int n = CG; n < NTILES; n += 4)
        if (((n / 4) & 1) != H)
          *reinterpret_cast<f32x4*>(&sSx[n][lane][0]) = sacc[n / 4];
#pragma unroll
      for (int it = 0; it < NT; ++it)
        if (it / 2 != H) *reinterpret_cast<f32x4*>(&sOx[CG][it][lane][0]) = outT[it];
    });
    __syncthreads();

    // n~ of the next chunk (waves with cg < 2 finish the rows of tile 2 hh + cg
    // of each slice: first k-step here, second from LDS)
    if (cg < 2 && g == 0) {
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int arow = s * AS + 32 * hh + 8 * (l16 >> 2) + 4 * cg + (l16 & 3);
        sN[arow] = gL * sN[arow] + (nn[s] + sNp[arow]);
      }
    }
    // finish this wave's score tiles: P = S (.) D, row sums
    float rsp[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) rsp[it] = 0.0f;
    for_wave<NW>(wave, [&](auto Wc) {
      constexpr int W = decltype(Wc)::value;
      constexpr int CG = W & 3, H = W >> 2;
#pragma unroll
      for (int it = 0; it < NT; ++it) {
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
          const int n = it * (it + 1) / 2 + jt;
          if (n % 4 == CG && ((n / 4) & 1) == H) {
            const f32x4 other = *reinterpret_cast<const f32x4*>(&sSx[n][lane][0]);
            const f32x4 S = sacc[n / 4] + other;
            const int i = it * 16 + l16;
            const float Mi = sGate[par][1][i];
            const float4 uj = *reinterpret_cast<const float4*>(&sGate[par][0][jt * 16 + 4 * g]);
            const float ujv[4] = {uj.x, uj.y, uj.z, uj.w};
            float pe[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = jt * 16 + 4 * g + e;
              const float pv = S[e] * __expf(ujv[e] - Mi);
              pe[e] = (jt < it || j <= i) ? pv : 0.0f;
            }
            rsp[it] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
            *reinterpret_cast<uint2*>(sP + i * PROW + jt * 16 + 4 * g) =
                make_uint2(cvt2(pe[0], pe[1]), cvt2(pe[2], pe[3]));
            if (jt == it && (it & 1) == 0)
              *reinterpret_cast<uint2*>(sP + i * PROW + (jt + 1) * 16 + 4 * g) = make_uint2(0u, 0u);
          }
        }
      }
    });
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const float r = sum_groups(rsp[it]);
      if (g == 0) sRs[wave][it * 16 + l16] = r;
    }
    __syncthreads();

    // ---- outputs of this wave's query tiles it = 2 hh, 2 hh + 1
    for_wave<NW>(wave, [&](auto Wc) {
      constexpr int W = decltype(Wc)::value;
      constexpr int CG = W & 3, H = W >> 2;
#pragma unroll
      for (int it = 2 * H; it < 2 * H + 2; ++it) {
        const int i = it * 16 + l16;
        const f32x4 other = *reinterpret_cast<const f32x4*>(&sOx[CG][it][lane][0]);
        const float gi_ = sGate[par][2][i];
        f32x4 o = (outT[it] + other) * (gi_ * sig);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if (32 * ks <= it * 16 + 15) {
            const uint4 Pf = *reinterpret_cast<const uint4*>(sP + i * PROW + 32 * ks + 8 * g);
            o = mfma16x16x32(Vf[ks], as_bf16x8(Pf), o);
          }
        }
        float rs = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) rs += sRs[w2][i];
        const float qn = sQn[0][i] + sQn[1][i];
        const float den = fmaxf(fabsf(gi_ * qn + rs), sGate[par][4][i]);
        const float inv = __builtin_amdgcn_rcpf(den);
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = o[e] * inv;
        if (OM != O_NONE) {
          float ov[4];
          if (OM == O_F32) {
            const float4 o4 = *reinterpret_cast<const float4*>(sO + i * 256 + 16 * ((CG * 4 + g) ^ (i & 15)));
            ov[0] = o4.x; ov[1] = o4.y; ov[2] = o4.z; ov[3] = o4.w;
          } else {
            const uint2 o2 = *reinterpret_cast<const uint2*>(sO + swz(i, CG * 16 + 4 * g));
            ov[0] = bf_lo(o2.x); ov[1] = bf_hi(o2.x); ov[2] = bf_lo(o2.y); ov[3] = bf_hi(o2.y);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] *= sigmoid_fast(ov[e]);
        }
        *reinterpret_cast<uint2*>(gh + (static_cast<int64_t>(c) * L + i) * dv) =
            make_uint2(cvt2(hv[0], hv[1]), cvt2(hv[2], hv[3]));
      }
    });
    m_s = m_cur;
    sig = sig_new;
  }
  wait_vm<0>();
  __syncthreads();

  if (a.C1) {
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int arow = 32 * (2 * s + hh) + 8 * g + 4 * e2 + e;
          a.C1[(head * DQK + arow) * dv + b0w + l16] = cacc[s][e2][e] * sig;
        }
      }
    }
    if (vt == 0) {
      if (tid < DQK) a.n1[head * DQK + tid] = sN[tid];
      if (tid == 0) a.m1[head] = m_s;
    }
  }
}

template <int DQK, int OM>
hipError_t launch_shape(const SeqArgs& a, hipStream_t stream) {
  const unsigned nwg = static_cast<unsigned>(a.B * a.H * (a.dv / TV));
  chunk_mfma8_kernel<DQK, OM><<<dim3(nwg), dim3(NTH), 0, stream>>>(a);
  return hipGetLastError();
}

template <int OM>
hipError_t launch_D(const SeqArgs& a, hipStream_t stream) {
  switch (a.dqk) {
    case 64: return launch_shape<64, OM>(a, stream);
    case 128: return launch_shape<128, OM>(a, stream);
    default: return launch_shape<256, OM>(a, stream);
  }
}

}  // namespace

bool chunk_mfma8_supported(const SeqArgs& a, int64_t chunk) {
  return a.qkv_bf16 && (a.dqk == 64 || a.dqk == 128 || a.dqk == 256) && a.dv % TV == 0 &&
         chunk == L && a.T % L == 0;
}

hipError_t launch_chunk_mfma8(const SeqArgs& a, hipStream_t stream) {
  switch (a.o_mode) {
    case O_F32: return launch_D<O_F32>(a, stream);
    case O_BF16: return launch_D<O_BF16>(a, stream);
    default: return launch_D<O_NONE>(a, stream);
  }
}

}  // namespace mlstm
