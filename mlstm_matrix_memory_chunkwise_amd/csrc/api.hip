// C ABI of the mLSTM library: argument checks, kernel selection, status codes.
// Every check runs on the host before anything is enqueued.  No HIP call is
// made before the checks pass, so invalid calls are rejected on hosts without
// a GPU too.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/mlstm.h"
#include "kernels.hpp"

#include <mutex>

// Fixed device scratch of mlstm_fwd_chunkwise_noalloc, for callers that cannot
// allocate.  Every GPU the library runs on holds one copy of this array (in
// its own memory, at its own address) until the process ends.  In host code
// `scratch` names a host-side stand-in, never a device address: the address
// of a device's copy comes from hipGetSymbolAddress, looked up once per
// device with that device current (scratch_address below), and only that
// address is handed to kernels.  Calls on one GPU share its copy, so calls
// that overlap in time on one GPU race; what the kernels read from it they
// first write in the same call (the state carried from the matrix-core
// kernel to the tail kernel), so nothing needs clearing between calls.
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`; the stream (NULL: the
// null stream of the current device) must belong to the current device.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace {

thread_local char g_detail[512] = "";

mlstm_status_t fail(mlstm_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}

mlstm_status_t ok() {
  g_detail[0] = '\0';
  return MLSTM_OK;
}

struct Buf {
  const char* name;
  const void* p;
  size_t bytes;
  size_t align;  // alignment the kernels need (vector accesses: 16; scalars: 4)
};

bool overlaps(const Buf& x, const Buf& y) {
  if (!x.p || !y.p || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const Buf& b) { return (reinterpret_cast<uintptr_t>(b.p) & (b.align - 1)) == 0; }

size_t dsize(int32_t dt) { return dt == MLSTM_BF16 ? 2 : 4; }

mlstm_status_t check_problem(const mlstm_problem_t* p, bool need_T) {
  if (!p) return fail(MLSTM_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->B < 0 || p->H < 0 || p->d_qk <= 0 || p->d_v <= 0 || (need_T && p->T < 0))
    return fail(MLSTM_ERR_INVALID_ARG,
                "sizes must be non-negative and d_qk, d_v positive (B=%lld H=%lld T=%lld d_qk=%lld d_v=%lld)",
                (long long)p->B, (long long)p->H, (long long)p->T, (long long)p->d_qk,
                (long long)p->d_v);
  if (p->qkv_dtype != MLSTM_F32 && p->qkv_dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown qkv_dtype %d", p->qkv_dtype);
  if (p->o_dtype != MLSTM_F32 && p->o_dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown o_dtype %d", p->o_dtype);
  if (p->fgate != MLSTM_FGATE_SIGMOID && p->fgate != MLSTM_FGATE_EXP)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown fgate %d", p->fgate);
  if (p->reserved != 0) return fail(MLSTM_ERR_INVALID_ARG, "reserved field must be 0");
  // grid-size and 32-bit index limits of the kernels
  if (p->B * p->H > (int64_t)1 << 24)
    return fail(MLSTM_ERR_UNSUPPORTED, "B*H=%lld exceeds 2^24", (long long)(p->B * p->H));
  if (p->d_qk % 16 != 0 || p->d_v % 16 != 0 || p->d_qk > 512 || p->d_v > 512)
    return fail(MLSTM_ERR_UNSUPPORTED, "d_qk=%lld d_v=%lld: need multiples of 16, at most 512",
                (long long)p->d_qk, (long long)p->d_v);
  if (need_T && p->T > ((int64_t)1 << 31) - 1)
    return fail(MLSTM_ERR_UNSUPPORTED, "T=%lld exceeds 2^31-1", (long long)p->T);
  return MLSTM_OK;
}

// Shared checks of the two whole-sequence entry points.
mlstm_status_t check_seq(const mlstm_problem_t* p, const void* q, const void* k, const void* v,
                         const float* i_pre, const float* f_pre, const void* o_pre,
                         const float* C0, const float* n0, const float* m0, void* h,
                         float* C1, float* n1, float* m1, mlstm::SeqArgs* out) {
  mlstm_status_t s = check_problem(p, true);
  if (s != MLSTM_OK) return s;
  if (!q || !k || !v || !i_pre || !f_pre || !h)
    return fail(MLSTM_ERR_INVALID_ARG, "q, k, v, i_pre, f_pre and h are required");
  const int in_state = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
  if (in_state != 0 && in_state != 3)
    return fail(MLSTM_ERR_INVALID_ARG, "initial state must be all of C0, n0, m0 or none");
  const int out_state = (C1 != nullptr) + (n1 != nullptr) + (m1 != nullptr);
  if (out_state != 0 && out_state != 3)
    return fail(MLSTM_ERR_INVALID_ARG, "final state must be all of C1, n1, m1 or none");
  const size_t BH = (size_t)(p->B * p->H), T = (size_t)p->T;
  const size_t dqk = (size_t)p->d_qk, dv = (size_t)p->d_v, sq = dsize(p->qkv_dtype);
  const Buf bufs[] = {
      {"q", q, BH * T * dqk * sq, 16},      {"k", k, BH * T * dqk * sq, 16},
      {"v", v, BH * T * dv * sq, 16},       {"i_pre", i_pre, BH * T * 4, 4},
      {"f_pre", f_pre, BH * T * 4, 4},      {"o_pre", o_pre, BH * T * dv * dsize(p->o_dtype), 16},
      {"C0", C0, BH * dqk * dv * 4, 16},    {"n0", n0, BH * dqk * 4, 4},
      {"m0", m0, BH * 4, 4},                {"h", h, BH * T * dv * sq, 16},
      {"C1", C1, BH * dqk * dv * 4, 16},    {"n1", n1, BH * dqk * 4, 4},
      {"m1", m1, BH * 4, 4},
  };
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", bufs[i].name, bufs[i].align);
  // outputs (h, C1, n1, m1 = indices 9..12) must not overlap any input or each other
  for (int o = 9; o < nb; ++o)
    for (int i = 0; i < nb; ++i)
      if (i != o && overlaps(bufs[o], bufs[i]))
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
  mlstm::SeqArgs a;
  a.B = p->B; a.H = p->H; a.T = p->T; a.dqk = p->d_qk; a.dv = p->d_v;
  a.Ts = p->T; a.t0 = 0;
  a.qkv_bf16 = p->qkv_dtype == MLSTM_BF16;
  a.o_mode = o_pre ? (p->o_dtype == MLSTM_BF16 ? mlstm::O_BF16 : mlstm::O_F32) : mlstm::O_NONE;
  a.fgate_exp = p->fgate == MLSTM_FGATE_EXP;
  a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
  a.C0 = C0; a.n0 = n0; a.m0 = m0; a.h = h; a.C1 = C1; a.n1 = n1; a.m1 = m1;
  *out = a;
  return MLSTM_OK;
}

// The workspace (`need` bytes) of a whole-sequence call must not overlap any
// tensor argument.
mlstm_status_t check_seq_workspace(const mlstm_problem_t* p, const void* q, const void* k,
                                   const void* v, const float* i_pre, const float* f_pre,
                                   const void* o_pre, const float* C0, const float* n0,
                                   const float* m0, const void* h, const float* C1,
                                   const float* n1, const float* m1, const void* workspace,
                                   size_t need) {
  const Buf ws{"workspace", workspace, need, 16};
  const size_t BH = (size_t)(p->B * p->H), T = (size_t)p->T, sq = dsize(p->qkv_dtype);
  const Buf all[] = {
      {"q", q, BH * T * p->d_qk * sq, 16}, {"k", k, BH * T * p->d_qk * sq, 16},
      {"v", v, BH * T * p->d_v * sq, 16},  {"i_pre", i_pre, BH * T * 4, 4},
      {"f_pre", f_pre, BH * T * 4, 4},
      {"o_pre", o_pre, BH * T * p->d_v * dsize(p->o_dtype), 16},
      {"C0", C0, BH * p->d_qk * p->d_v * 4, 16}, {"n0", n0, BH * p->d_qk * 4, 4},
      {"m0", m0, BH * 4, 4},               {"h", h, BH * T * p->d_v * sq, 16},
      {"C1", C1, BH * p->d_qk * p->d_v * 4, 16}, {"n1", n1, BH * p->d_qk * 4, 4},
      {"m1", m1, BH * 4, 4}};
  for (const Buf& b : all)
    if (overlaps(ws, b)) return fail(MLSTM_ERR_INVALID_ARG, "workspace overlaps %s", b.name);
  return MLSTM_OK;
}

mlstm_status_t check_chunk(const mlstm_problem_t* p, int64_t chunk) {
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
    return fail(MLSTM_ERR_UNSUPPORTED, "chunk=%lld: supported chunks are 16, 32, 64, 128",
                (long long)chunk);
  return MLSTM_OK;
}

mlstm::SeqArgs problem_args(const mlstm_problem_t* p) {
  mlstm::SeqArgs a{};
  a.B = p->B; a.H = p->H; a.T = p->T; a.dqk = p->d_qk; a.dv = p->d_v;
  a.Ts = p->T; a.t0 = 0;
  a.qkv_bf16 = p->qkv_dtype == MLSTM_BF16;
  return a;
}

// Shapes the backward pass covers.
mlstm_status_t check_bwd_shape(const mlstm_problem_t* p, int64_t chunk) {
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(MLSTM_ERR_UNSUPPORTED, "backward: chunk=%lld: supported chunks are 16, 32, 64",
                (long long)chunk);
  if (chunk == 64) {
    if (p->qkv_dtype != MLSTM_BF16 || p->d_v % 64 != 0 ||
        (p->d_qk != 64 && p->d_qk != 128 && p->d_qk != 256))
      return fail(MLSTM_ERR_UNSUPPORTED,
                  "backward chunk 64 needs bf16 q/k/v, d_v a multiple of 64 and d_qk 64, 128 "
                  "or 256 (got d_qk=%lld, d_v=%lld)", (long long)p->d_qk, (long long)p->d_v);
    return MLSTM_OK;
  }
  const int64_t tv = p->d_v % 32 == 0 ? 32 : 16;
  if (p->d_qk > 256 || p->d_qk % (256 / tv) != 0)
    return fail(MLSTM_ERR_UNSUPPORTED,
                "backward: d_qk=%lld: need at most 256 and a multiple of %lld (d_v=%lld)",
                (long long)p->d_qk, (long long)(256 / tv), (long long)p->d_v);
  return MLSTM_OK;
}

mlstm::BwdArgs bwd_problem_args(const mlstm_problem_t* p, int64_t chunk) {
  mlstm::BwdArgs a{};
  a.B = p->B; a.H = p->H; a.T = p->T; a.dqk = p->d_qk; a.dv = p->d_v;
  a.qkv_bf16 = p->qkv_dtype == MLSTM_BF16;
  a.fgate_exp = p->fgate == MLSTM_FGATE_EXP;
  a.L = static_cast<int>(chunk);
  return a;
}

mlstm_status_t device_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MLSTM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// dst <- src (`bytes`, a multiple of 4), or zeros when src is NULL; nothing
// when dst is NULL.  Zeros come from a fill kernel, not a memset node.
hipError_t copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t st) {
  if (!dst || bytes == 0) return hipSuccess;
  if (src) return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
  const int64_t words = static_cast<int64_t>(bytes / 4);
  return mlstm::launch_fill_words(static_cast<uint32_t*>(dst), 1, words, 0, words, 0u, st);
}

// A state triple/quadruple given all-or-none; the copies of an empty
// sequence's pass-through state must not overlap their sources.
struct StateBufs {
  const char* names[4];
  const void* in[4];
  void* out[4];
  size_t bytes[4];
  int n;
};

mlstm_status_t pass_state(const StateBufs& sb, const char* what, hipStream_t st) {
  int nin = 0, nout = 0;
  for (int i = 0; i < sb.n; ++i) {
    nin += sb.in[i] != nullptr;
    nout += sb.out[i] != nullptr;
  }
  if (nin != 0 && nin != sb.n)
    return fail(MLSTM_ERR_INVALID_ARG, "%s: initial state must be given whole or not at all", what);
  if (nout != 0 && nout != sb.n)
    return fail(MLSTM_ERR_INVALID_ARG, "%s: final state must be given whole or not at all", what);
  for (int i = 0; i < sb.n; ++i) {
    const size_t al = 4;   // copied or filled as 32-bit words only
    if ((sb.in[i] && (reinterpret_cast<uintptr_t>(sb.in[i]) & (al - 1))) ||
        (sb.out[i] && (reinterpret_cast<uintptr_t>(sb.out[i]) & (al - 1))))
      return fail(MLSTM_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", what, sb.names[i], al);
    for (int j = 0; j < sb.n; ++j) {
      const Buf o{sb.names[i], sb.out[i], sb.bytes[i], 4};
      if (overlaps(o, Buf{"in", sb.in[j], sb.bytes[j], 4}) ||
          (j != i && overlaps(o, Buf{"out", sb.out[j], sb.bytes[j], 4})))
        return fail(MLSTM_ERR_INVALID_ARG, "%s: final state %s overlaps another state buffer", what,
                    sb.names[i]);
    }
  }
  hipError_t e = hipSuccess;
  for (int i = 0; i < sb.n && e == hipSuccess; ++i) e = copy_or_zero(sb.out[i], sb.in[i], sb.bytes[i], st);
  return device_status(e, what);
}

// A whole-sequence call with B*H = 0 does nothing; with T = 0 its final
// state is its initial state (zeros without one).
mlstm_status_t seq_empty(const mlstm_problem_t* p, const float* C0, const float* n0,
                         const float* m0, float* C1, float* n1, float* m1, void* stream) {
  const size_t BH = (size_t)(p->B * p->H), dqk = (size_t)p->d_qk, dv = (size_t)p->d_v;
  if (BH == 0) return ok();
  const StateBufs sb{{"C1", "n1", "m1", ""}, {C0, n0, m0, nullptr}, {C1, n1, m1, nullptr},
                     {BH * dqk * dv * 4, BH * dqk * 4, BH * 4, 0}, 3};
  return pass_state(sb, "empty sequence", static_cast<hipStream_t>(stream));
}

bool seq_is_empty(const mlstm_problem_t* p) { return p->B * p->H == 0 || p->T == 0; }

// How a chunkwise call runs.  When T is not a multiple of the chunk and an
// MFMA kernel covers the shape, that kernel runs the first Tm = T - (T % chunk)
// tokens and leaves its final state (C~, n~, m) in the workspace; the VALU
// kernel continues from that state over the last T % chunk tokens, as one
// shorter chunk.  Otherwise a single kernel runs the whole sequence (the VALU
// kernel takes a shorter last chunk by itself).
//
// Sequence split.  The MFMA kernels run one workgroup per (head, 64 value
// columns) through the whole sequence, so a problem with few heads leaves
// most of the 256 compute units idle.  When that grid has at most
// kSplitGroups workgroups and the sequence is long, the call instead splits
// the sequence into P = 2, 4, 8 or 16 equal segments (the most that still fit the
// compute units and leave at least kSplitMinTokens per segment):
//   1. computes the exact states at the P - 1 split points: from weighted
//      products over the tokens before them (state_gemm.hip) where that
//      covers the shape, else (P = 2 only) with the state-only chunk
//      recurrence over the first half (chunk_state.hip);
//   2. runs the MFMA kernel once over all segments at the same time: segment
//      s of head h is laid out in memory exactly like head P h + s of a
//      problem with P H heads of T / P tokens, whose initial states are the
//      caller's (or zero) for s = 0 and the state from step 1 otherwise;
//   3. copies the final states of the last segments out.
// The states of the P H segment-heads live in the workspace.
constexpr int64_t kSplitGroups = 128;      // half the compute units of an MI355X
constexpr int64_t kSplitCUs = 256;         // the grid of all segments fits these
constexpr int64_t kSplitMinTokens = 2048;  // per segment

// One block of float32 states for n heads: C~ [n][d_qk][d_v], then n~ [n][d_qk],
// then m [n], each 256-byte aligned, from byte offset `at`.
struct StateBlock {
  size_t C, n, m, end;
};
StateBlock state_block(size_t at, size_t nheads, size_t dqk, size_t dv) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  StateBlock b;
  b.C = up(at);
  b.n = up(b.C + 4 * nheads * dqk * dv);
  b.m = up(b.n + 4 * nheads * dqk);
  b.end = up(b.m + 4 * nheads);
  return b;
}

struct FwdPlan {
  bool mfma;        // an MFMA kernel runs tokens 0 .. Tm-1
  bool tail;        // then the VALU kernel runs tokens Tm .. T-1
  int64_t Tm;
  size_t mid_off;   // byte offset of the carried state in the workspace
  bool split;       // the sequence split above (no tail)
  int P;            // its segment count
  StateBlock s_in;  // initial states of the P B H segment-heads
  StateBlock s_out; // their final states
  StateBlock s_mid; // the states at the P - 1 split points of the B H heads
  bool state_gemm;  // step 1 of the split as weighted products
  size_t sg_off;    // their scratch
  size_t need;      // workspace bytes
};

// cap: the most workspace a split may take (the fixed scratch of the
// no-allocation entry point); with less, fewer segments or none.
FwdPlan fwd_plan(const mlstm::SeqArgs& a, int64_t chunk, size_t cap = SIZE_MAX) {
  FwdPlan f{};
  f.Tm = a.T - a.T % chunk;
  mlstm::SeqArgs m = a;
  m.T = f.Tm;
  f.mfma = f.Tm > 0 && mlstm::chunk_mfma_supported(m, chunk);
  f.tail = f.mfma && f.Tm < a.T;
  const size_t mfma_ws = f.mfma ? mlstm::chunk_mfma_workspace(m, chunk) : 0;
  f.mid_off = (mfma_ws + 255) / 256 * 256;
  const size_t BH = static_cast<size_t>(a.B * a.H);
  const size_t dqk = static_cast<size_t>(a.dqk), dv = static_cast<size_t>(a.dv);
  const size_t mid = f.tail ? 4 * BH * (dqk * dv + dqk + 1) : 0;
  f.need = f.tail ? f.mid_off + mid : mfma_ws;
  if (f.mfma && !f.tail) {
    const int64_t unit = chunk > 64 ? chunk : 64;   // segments of whole chunks and of 64 tokens
    const int64_t grid = a.B * a.H * (a.dv / 64);
    for (int P = 16; P >= 2 && !f.split; P /= 2) {
      if (grid > kSplitGroups || grid * P > kSplitCUs || a.T % (P * unit) != 0 ||
          a.T / P < kSplitMinTokens)
        continue;
      mlstm::SeqArgs seg = a;
      seg.T = a.T / P;
      seg.H = P * a.H;
      if (!mlstm::chunk_mfma_supported(seg, chunk)) continue;
      mlstm::SeqArgs before = a;       // tokens before the last split point
      before.T = a.T / P * (P - 1);
      bool gemm = mlstm::state_gemm_supported(before, P - 1);
      const bool recur = P == 2 && mlstm::chunk_state_supported(seg);
      if (!gemm && !recur) continue;
      const StateBlock s_in = state_block(f.mid_off, P * BH, dqk, dv);
      const StateBlock s_out = state_block(s_in.end, P * BH, dqk, dv);
      const StateBlock s_mid = state_block(s_out.end, (P - 1) * BH, dqk, dv);
      size_t need = s_mid.end + (gemm ? mlstm::state_gemm_workspace(before, P - 1) : 0);
      if (need > cap && gemm && recur) {   // the chunk recurrence needs no scratch of its own
        gemm = false;
        need = s_mid.end;
      }
      if (need > cap) continue;   // fewer segments need less scratch
      f.split = true;
      f.P = P;
      f.state_gemm = gemm;
      f.s_in = s_in;
      f.s_out = s_out;
      f.s_mid = s_mid;
      f.sg_off = s_mid.end;
      f.need = need;
    }
  }
  return f;
}

// Copies `width` bytes per head from n heads of src (pitch spitch) to dst
// (pitch dpitch), or fills them with zeros when src is NULL.
hipError_t copy_heads(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                      size_t nheads, hipStream_t st) {
  if (src)
    return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, nheads, hipMemcpyDeviceToDevice, st);
  return mlstm::launch_fill_words(static_cast<uint32_t*>(dst), static_cast<int64_t>(nheads),
                                  static_cast<int64_t>(dpitch / 4), 0,
                                  static_cast<int64_t>(width / 4), 0u, st);
}

// The sequence split (see fwd_plan) on a checked call.
hipError_t run_split(const mlstm::SeqArgs& a, int64_t chunk, const FwdPlan& f, void* workspace,
                     hipStream_t st) {
  char* w = static_cast<char*>(workspace);
  const int P = f.P;
  const size_t BH = static_cast<size_t>(a.B * a.H);
  const size_t dqk = static_cast<size_t>(a.dqk), dv = static_cast<size_t>(a.dv);
  const size_t cB = 4 * dqk * dv, nB = 4 * dqk;   // bytes of one head's C~, n~
  char* inC = w + f.s_in.C;
  char* inN = w + f.s_in.n;
  char* inM = w + f.s_in.m;
  float* midC = reinterpret_cast<float*>(w + f.s_mid.C);
  float* midN = reinterpret_cast<float*>(w + f.s_mid.n);
  float* midM = reinterpret_cast<float*>(w + f.s_mid.m);
  // 1. the states at the split points T/P, 2T/P, .. (block k of the mid
  // states: the state at (k + 1) T/P of every head)
  mlstm::SeqArgs p1 = a;
  p1.T = a.T / P * (P - 1);   // tokens before the last split point (heads T apart)
  hipError_t e;
  if (f.state_gemm) {
    e = mlstm::launch_state_gemm(p1, P - 1, midC, midN, midM, w + f.sg_off, st);
  } else {
    p1.C1 = midC; p1.n1 = midN; p1.m1 = midM;   // (P = 2: the first half)
    e = mlstm::launch_chunk_state(p1, st);
  }
  // initial states of the segment-heads: P h <- the caller's (or zero),
  // P h + s <- the state at s T/P
  if (e == hipSuccess) e = copy_heads(inC, P * cB, a.C0, cB, cB, BH, st);
  if (e == hipSuccess) e = copy_heads(inN, P * nB, a.n0, nB, nB, BH, st);
  if (e == hipSuccess) e = copy_heads(inM, P * 4, a.m0, 4, 4, BH, st);
  for (int s = 1; s < P && e == hipSuccess; ++s) {
    const size_t k = static_cast<size_t>(s - 1);
    e = copy_heads(inC + s * cB, P * cB, reinterpret_cast<char*>(midC) + k * BH * cB, cB, cB, BH, st);
    if (e == hipSuccess)
      e = copy_heads(inN + s * nB, P * nB, reinterpret_cast<char*>(midN) + k * BH * nB, nB, nB, BH, st);
    if (e == hipSuccess)
      e = copy_heads(inM + s * 4, P * 4, reinterpret_cast<char*>(midM) + k * BH * 4, 4, 4, BH, st);
  }
  if (e != hipSuccess) return e;
  // 2. all segments at once, as P H heads of T/P tokens
  mlstm::SeqArgs p2 = a;
  p2.H = P * a.H;
  p2.T = a.T / P;
  p2.Ts = a.T / P;
  p2.C0 = reinterpret_cast<float*>(inC);
  p2.n0 = reinterpret_cast<float*>(inN);
  p2.m0 = reinterpret_cast<float*>(inM);
  const bool out = a.C1 != nullptr;
  p2.C1 = out ? reinterpret_cast<float*>(w + f.s_out.C) : nullptr;
  p2.n1 = out ? reinterpret_cast<float*>(w + f.s_out.n) : nullptr;
  p2.m1 = out ? reinterpret_cast<float*>(w + f.s_out.m) : nullptr;
  e = mlstm::launch_chunk_mfma(p2, chunk, nullptr, st);
  if (e != hipSuccess || !out) return e;
  // 3. the final state is that of the last segments
  const size_t last = static_cast<size_t>(P - 1);
  e = copy_heads(a.C1, cB, w + f.s_out.C + last * cB, P * cB, cB, BH, st);
  if (e == hipSuccess) e = copy_heads(a.n1, nB, w + f.s_out.n + last * nB, P * nB, nB, BH, st);
  if (e == hipSuccess) e = copy_heads(a.m1, 4, w + f.s_out.m + last * 4, P * 4, 4, BH, st);
  return e;
}

// Backward of a sequence whose length T is not a multiple of the chunk: the
// pass runs on copies padded to Tp = ceil(T / chunk) chunks, placed at the
// front of the workspace.  A padding token leaves the memory as it is
// (log f = 0: f~ = 1e4 for the sigmoid gate, 0 for the exponential one;
// i = 0: i~ = -1e4) and has q = k = v = h = dh = o~ = 0, so it adds nothing
// to any gradient, and dC1, dn1 given at Tp are the gradients at T.  The
// gradients of the first T tokens are copied out afterwards.
struct BwdPad {
  int64_t Tp;
  enum { Q, K, V, I, F, O, H, DH, DQ, DK, DV, DI, DF, DO, N };
  size_t off[N];
  size_t row[N];    // bytes per token
  size_t bytes;     // 0: no padding
};

BwdPad bwd_pad_plan(const mlstm_problem_t* p, int64_t chunk) {
  BwdPad b{};
  b.Tp = (p->T + chunk - 1) / chunk * chunk;
  if (b.Tp == p->T) return b;
  const size_t sq = dsize(p->qkv_dtype), so = dsize(p->o_dtype);
  const size_t dqk = (size_t)p->d_qk, dv = (size_t)p->d_v;
  const size_t rows[BwdPad::N] = {dqk * sq, dqk * sq, dv * sq, 4, 4, dv * so, dv * sq, dv * sq,
                                  dqk * 4, dqk * 4, dv * 4, 4, 4, dv * 4};
  size_t at = 0;
  for (int i = 0; i < BwdPad::N; ++i) {
    b.row[i] = rows[i];
    b.off[i] = at;
    at += (static_cast<size_t>(p->B * p->H) * b.Tp * rows[i] + 255) / 256 * 256;
  }
  b.bytes = at;
  return b;
}

mlstm::BwdArgs bwd_padded_args(const mlstm_problem_t* p, int64_t chunk, const BwdPad& pad) {
  mlstm::BwdArgs a = bwd_problem_args(p, chunk);
  a.T = pad.Tp;
  return a;
}

// Backward of an empty sequence: dC0 = dC1, dn0 = dn1 and
// dm0 = <dC1, C~0> + <dn1, n~0>, with zeros for what is not given.
mlstm_status_t bwd_empty(const mlstm_problem_t* p, int64_t chunk, const float* C0,
                         const float* n0, const float* m0, const float* dC1, const float* dn1,
                         float* dC0, float* dn0, float* dm0, void* stream) {
  const int in_state = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
  if (in_state != 0 && in_state != 3)
    return fail(MLSTM_ERR_INVALID_ARG, "initial state must be all of C0, n0, m0 or none");
  if ((dC1 != nullptr) != (dn1 != nullptr))
    return fail(MLSTM_ERR_INVALID_ARG, "final-state gradient must be both of dC1, dn1 or none");
  const size_t BH = (size_t)(p->B * p->H), dqk = (size_t)p->d_qk, dvv = (size_t)p->d_v;
  const Buf bufs[] = {
      {"C0", C0, BH * dqk * dvv * 4, 4}, {"n0", n0, BH * dqk * 4, 4}, {"m0", m0, BH * 4, 4},
      {"dC1", dC1, BH * dqk * dvv * 4, 4}, {"dn1", dn1, BH * dqk * 4, 4},
      {"dC0", dC0, BH * dqk * dvv * 4, 4}, {"dn0", dn0, BH * dqk * 4, 4}, {"dm0", dm0, BH * 4, 4}};
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not 4-byte aligned", bufs[i].name);
  for (int o = 5; o < nb; ++o)
    for (int i = 0; i < nb; ++i)
      if (i != o && overlaps(bufs[o], bufs[i]))
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
  mlstm::BwdArgs a = bwd_problem_args(p, chunk);
  a.C0 = C0; a.n0 = n0; a.m0 = m0; a.dC1 = dC1; a.dn1 = dn1;
  a.dC0 = dC0; a.dn0 = dn0; a.dm0 = dm0;
  return device_status(mlstm::launch_bwd_empty(a, static_cast<hipStream_t>(stream)),
                       "backward of an empty sequence");
}


// The chunkwise forward pass behind both entry points.  With fixed_scratch
// the workspace is the library's own device array (below) instead of the
// caller's (workspace, workspace_bytes are then ignored); every check still
// runs before the first HIP call.
mlstm_status_t fwd_chunkwise(const mlstm_problem_t* p, int64_t chunk, const void* q,
                             const void* k, const void* v, const float* i_pre,
                             const float* f_pre, const void* o_pre, const float* C0,
                             const float* n0, const float* m0, void* h, float* C1, float* n1,
                             float* m1, void* workspace, size_t workspace_bytes,
                             bool fixed_scratch, void* stream) {
  if (p && check_problem(p, true) == MLSTM_OK && seq_is_empty(p)) {
    const mlstm_status_t sc = check_chunk(p, chunk);
    if (sc != MLSTM_OK) return sc;
    return seq_empty(p, C0, n0, m0, C1, n1, m1, stream);
  }
  mlstm::SeqArgs a;
  mlstm_status_t s = check_seq(p, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1, &a);
  if (s != MLSTM_OK) return s;
  s = check_chunk(p, chunk);
  if (s != MLSTM_OK) return s;
  const FwdPlan f = fwd_plan(a, chunk, fixed_scratch ? kScratchBytes : SIZE_MAX);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fixed_scratch) {
    if (f.need > kScratchBytes)
      return fail(MLSTM_ERR_UNSUPPORTED,
                  "this problem needs %zu bytes of scratch; the fixed scratch of "
                  "mlstm_fwd_chunkwise_noalloc holds %zu (use mlstm_fwd_chunkwise with a workspace)",
                  f.need, kScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (f.need > 0) {   // the first HIP call of this path
      const hipError_t e = scratch_address(st, &workspace);
      if (e != hipSuccess) return device_status(e, "fixed scratch");
      workspace_bytes = kScratchBytes;
    }
  } else {
    if (workspace_bytes < f.need || (f.need > 0 && !workspace))
      return fail(MLSTM_ERR_INVALID_ARG, "workspace of %zu bytes given, %zu needed",
                  workspace_bytes, f.need);
    if (f.need > 0 && !aligned16(workspace))
      return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    s = check_seq_workspace(p, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1, workspace,
                            f.need);
    if (s != MLSTM_OK) return s;
  }
  if (!f.mfma) return device_status(mlstm::launch_chunk_valu(a, chunk, st), "chunkwise (valu)");
  if (f.split) return device_status(run_split(a, chunk, f, workspace, st), "chunkwise (split)");
  if (!f.tail)
    return device_status(mlstm::launch_chunk_mfma(a, chunk, workspace, st), "chunkwise (mfma)");
  const size_t BH = static_cast<size_t>(a.B * a.H);
  float* midC = reinterpret_cast<float*>(static_cast<char*>(workspace) + f.mid_off);
  float* midn = midC + BH * a.dqk * a.dv;
  float* midm = midn + BH * a.dqk;
  mlstm::SeqArgs head = a;   // tokens 0 .. Tm-1 on MFMA, state into the workspace
  head.T = f.Tm;
  head.C1 = midC; head.n1 = midn; head.m1 = midm;
  s = device_status(mlstm::launch_chunk_mfma(head, chunk, workspace, st), "chunkwise (mfma)");
  if (s != MLSTM_OK) return s;
  mlstm::SeqArgs tail = a;   // tokens Tm .. T-1 from that state
  tail.t0 = f.Tm;
  tail.C0 = midC; tail.n0 = midn; tail.m0 = midm;
  return device_status(mlstm::launch_chunk_valu(tail, chunk, st), "chunkwise tail (valu)");
}

}  // namespace

extern "C" {

const char* mlstm_version(void) { return "mlstm-gfx950 0.1.0"; }

const char* mlstm_status_string(mlstm_status_t s) {
  switch (s) {
    case MLSTM_OK: return "ok";
    case MLSTM_ERR_INVALID_ARG: return "invalid argument";
    case MLSTM_ERR_UNSUPPORTED: return "unsupported problem";
    case MLSTM_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* mlstm_last_error_detail(void) { return g_detail; }

mlstm_status_t mlstm_fwd_chunkwise_workspace_bytes(const mlstm_problem_t* p, int64_t chunk,
                                                   size_t* bytes) {
  if (!bytes) return fail(MLSTM_ERR_INVALID_ARG, "bytes is NULL");
  mlstm_status_t s = check_problem(p, true);
  if (s != MLSTM_OK) return s;
  s = check_chunk(p, chunk);
  if (s != MLSTM_OK) return s;
  *bytes = fwd_plan(problem_args(p), chunk).need;
  return ok();
}

mlstm_status_t mlstm_fwd_chunkwise(const mlstm_problem_t* p, int64_t chunk, const void* q,
                                   const void* k, const void* v, const float* i_pre,
                                   const float* f_pre, const void* o_pre, const float* C0,
                                   const float* n0, const float* m0, void* h, float* C1,
                                   float* n1, float* m1, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return fwd_chunkwise(p, chunk, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1,
                       workspace, workspace_bytes, false, stream);
}

mlstm_status_t mlstm_fwd_chunkwise_noalloc(const mlstm_problem_t* p, int64_t chunk,
                                           const void* q, const void* k, const void* v,
                                           const float* i_pre, const float* f_pre,
                                           const void* o_pre, const float* C0, const float* n0,
                                           const float* m0, void* h, float* C1, float* n1,
                                           float* m1, void* stream) {
  return fwd_chunkwise(p, chunk, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1,
                       nullptr, 0, true, stream);
}

mlstm_status_t mlstm_bwd_chunkwise_workspace_bytes(const mlstm_problem_t* p, int64_t chunk,
                                                   size_t* bytes) {
  if (!bytes) return fail(MLSTM_ERR_INVALID_ARG, "bytes is NULL");
  mlstm_status_t s = check_problem(p, true);
  if (s != MLSTM_OK) return s;
  s = check_bwd_shape(p, chunk);
  if (s != MLSTM_OK) return s;
  if (seq_is_empty(p)) {
    *bytes = 0;
    return ok();
  }
  const BwdPad pad = bwd_pad_plan(p, chunk);
  *bytes = pad.bytes + mlstm::bwd_workspace(bwd_padded_args(p, chunk, pad), nullptr);
  return ok();
}

mlstm_status_t mlstm_bwd_chunkwise(const mlstm_problem_t* p, int64_t chunk, const void* q,
                                   const void* k, const void* v, const float* i_pre,
                                   const float* f_pre, const void* o_pre, const float* C0,
                                   const float* n0, const float* m0, const void* h,
                                   const void* dh, const float* dC1, const float* dn1,
                                   float* dq, float* dk, float* dv, float* di, float* df,
                                   float* d_o, float* dC0, float* dn0, float* dm0,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  mlstm_status_t s = check_problem(p, true);
  if (s != MLSTM_OK) return s;
  s = check_bwd_shape(p, chunk);
  if (s != MLSTM_OK) return s;
  if (p->B * p->H == 0) return ok();
  if (p->T == 0) return bwd_empty(p, chunk, C0, n0, m0, dC1, dn1, dC0, dn0, dm0, stream);
  if (!q || !k || !v || !i_pre || !f_pre || !h || !dh || !dq || !dk || !dv || !di || !df)
    return fail(MLSTM_ERR_INVALID_ARG,
                "q, k, v, i_pre, f_pre, h, dh, dq, dk, dv, di and df are required");
  const int in_state = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
  if (in_state != 0 && in_state != 3)
    return fail(MLSTM_ERR_INVALID_ARG, "initial state must be all of C0, n0, m0 or none");
  if ((dC1 != nullptr) != (dn1 != nullptr))
    return fail(MLSTM_ERR_INVALID_ARG, "final-state gradient must be both of dC1, dn1 or none");
  if ((o_pre != nullptr) != (d_o != nullptr))
    return fail(MLSTM_ERR_INVALID_ARG, "d_o is required exactly when o_pre is given");
  const size_t BH = (size_t)(p->B * p->H), T = (size_t)p->T;
  const size_t dqk = (size_t)p->d_qk, dvv = (size_t)p->d_v, sq = dsize(p->qkv_dtype);
  // chunk 64 reads and writes the [.., d_v] arrays 16 bytes at a time
  const size_t va = chunk == 64 ? 16 : 4;
  const Buf bufs[] = {
      {"q", q, BH * T * dqk * sq, 16},      {"k", k, BH * T * dqk * sq, 16},
      {"v", v, BH * T * dvv * sq, 16},      {"i_pre", i_pre, BH * T * 4, 4},
      {"f_pre", f_pre, BH * T * 4, 4},      {"o_pre", o_pre, BH * T * dvv * dsize(p->o_dtype), va},
      {"C0", C0, BH * dqk * dvv * 4, va},   {"n0", n0, BH * dqk * 4, 4},
      {"m0", m0, BH * 4, 4},                {"h", h, BH * T * dvv * sq, 16},
      {"dh", dh, BH * T * dvv * sq, 16},    {"dC1", dC1, BH * dqk * dvv * 4, va},
      {"dn1", dn1, BH * dqk * 4, 4},
      // outputs from here (index 13 on)
      {"dq", dq, BH * T * dqk * 4, 16},     {"dk", dk, BH * T * dqk * 4, 16},
      {"dv", dv, BH * T * dvv * 4, va},     {"di", di, BH * T * 4, 4},
      {"df", df, BH * T * 4, 4},            {"d_o", d_o, BH * T * dvv * 4, va},
      {"dC0", dC0, BH * dqk * dvv * 4, va}, {"dn0", dn0, BH * dqk * 4, 4},
      {"dm0", dm0, BH * 4, 4},
  };
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", bufs[i].name, bufs[i].align);
  for (int o = 13; o < nb; ++o)
    for (int i = 0; i < nb; ++i)
      if (i != o && overlaps(bufs[o], bufs[i]))
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
  const BwdPad pad = bwd_pad_plan(p, chunk);
  mlstm::BwdArgs a = bwd_padded_args(p, chunk, pad);
  const size_t need = pad.bytes + mlstm::bwd_workspace(a, nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(MLSTM_ERR_INVALID_ARG, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                need);
  if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const Buf ws{"workspace", workspace, need, 16};
  for (int i = 0; i < nb; ++i)
    if (overlaps(ws, bufs[i])) return fail(MLSTM_ERR_INVALID_ARG, "workspace overlaps %s", bufs[i].name);
  a.o_mode = o_pre ? (p->o_dtype == MLSTM_BF16 ? mlstm::O_BF16 : mlstm::O_F32) : mlstm::O_NONE;
  a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
  a.C0 = C0; a.n0 = n0; a.m0 = m0; a.h = h; a.dh = dh; a.dC1 = dC1; a.dn1 = dn1;
  a.d_q = dq; a.d_k = dk; a.d_v = dv; a.d_i = di; a.d_f = df; a.d_o = d_o;
  a.dC0 = dC0; a.dn0 = dn0; a.dm0 = dm0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pad.bytes == 0)
    return device_status(mlstm::launch_bwd(a, workspace, st), "chunkwise backward");

  // padded copies: rows of T tokens copied, tokens T .. Tp-1 filled
  char* w = static_cast<char*>(workspace);
  const int64_t BHr = p->B * p->H, Tr = p->T, Tp = pad.Tp;
  auto at = [&](int i) { return static_cast<void*>(w + pad.off[i]); };
  const float fpad = p->fgate == MLSTM_FGATE_EXP ? 0.0f : 1.0e4f, ipad = -1.0e4f;
  const void* src[BwdPad::DQ] = {q, k, v, i_pre, f_pre, o_pre, h, dh};
  hipError_t e = hipSuccess;
  for (int i = 0; i < BwdPad::DQ && e == hipSuccess; ++i) {
    if (!src[i]) continue;
    const size_t r = pad.row[i];
    e = hipMemcpy2DAsync(at(i), Tp * r, src[i], Tr * r, Tr * r, BHr, hipMemcpyDeviceToDevice, st);
    float fill = 0.0f;
    if (i == BwdPad::I) fill = ipad;
    if (i == BwdPad::F) fill = fpad;
    uint32_t word;
    std::memcpy(&word, &fill, 4);
    if (e == hipSuccess)
      e = mlstm::launch_fill_words(static_cast<uint32_t*>(at(i)), BHr, Tp * r / 4, Tr * r / 4,
                                   (Tp - Tr) * r / 4, word, st);
  }
  if (e != hipSuccess) return device_status(e, "chunkwise backward (padding)");
  a.q = at(BwdPad::Q); a.k = at(BwdPad::K); a.v = at(BwdPad::V);
  a.i_pre = static_cast<const float*>(at(BwdPad::I));
  a.f_pre = static_cast<const float*>(at(BwdPad::F));
  a.o_pre = o_pre ? at(BwdPad::O) : nullptr;
  a.h = at(BwdPad::H); a.dh = at(BwdPad::DH);
  a.d_q = static_cast<float*>(at(BwdPad::DQ)); a.d_k = static_cast<float*>(at(BwdPad::DK));
  a.d_v = static_cast<float*>(at(BwdPad::DV)); a.d_i = static_cast<float*>(at(BwdPad::DI));
  a.d_f = static_cast<float*>(at(BwdPad::DF));
  a.d_o = d_o ? static_cast<float*>(at(BwdPad::DO)) : nullptr;
  s = device_status(mlstm::launch_bwd(a, w + pad.bytes, st), "chunkwise backward");
  if (s != MLSTM_OK) return s;
  void* dst[BwdPad::N] = {};
  dst[BwdPad::DQ] = dq; dst[BwdPad::DK] = dk; dst[BwdPad::DV] = dv;
  dst[BwdPad::DI] = di; dst[BwdPad::DF] = df; dst[BwdPad::DO] = d_o;
  for (int i = BwdPad::DQ; i < BwdPad::N && e == hipSuccess; ++i) {
    if (!dst[i]) continue;
    const size_t r = pad.row[i];
    e = hipMemcpy2DAsync(dst[i], Tr * r, at(i), Tp * r, Tr * r, BHr, hipMemcpyDeviceToDevice, st);
  }
  return device_status(e, "chunkwise backward (copy out)");
}

mlstm_status_t mlstm_groupnorm_ogate(int64_t B, int64_t H, int64_t T, int64_t d_v,
                                     mlstm_dtype_t h_dtype, mlstm_dtype_t o_dtype,
                                     const void* h, const void* o_pre,
                                     const float* gamma, const float* beta, float eps,
                                     void* y, void* stream) {
  if (B < 0 || H < 0 || T < 0 || d_v <= 0)
    return fail(MLSTM_ERR_INVALID_ARG,
                "sizes must be non-negative and d_v positive (B=%lld H=%lld T=%lld d_v=%lld)",
                (long long)B, (long long)H, (long long)T, (long long)d_v);
  if ((h_dtype != MLSTM_F32 && h_dtype != MLSTM_BF16) || (o_dtype != MLSTM_F32 && o_dtype != MLSTM_BF16))
    return fail(MLSTM_ERR_INVALID_ARG, "unknown dtype (h %d, o %d)", h_dtype, o_dtype);
  if (B * H * T == 0) return ok();   // no rows
  if (!h || !y) return fail(MLSTM_ERR_INVALID_ARG, "h and y are required");
  if (!(eps >= 0.0f) || eps == __builtin_inff())
    return fail(MLSTM_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (d_v % 4 != 0 || d_v > 1024)
    return fail(MLSTM_ERR_UNSUPPORTED, "d_v=%lld: need a multiple of 4, at most 1024", (long long)d_v);
  // at most 2^32 rows keeps the grid (4 rows or more per workgroup) below 2^31 workgroups
  if (B * H * T > ((int64_t)1 << 32))
    return fail(MLSTM_ERR_UNSUPPORTED, "B*H*T=%lld exceeds 2^32", (long long)(B * H * T));
  const size_t n = (size_t)(B * H * T * d_v), sh = dsize(h_dtype), so = dsize(o_dtype);
  // rows move in 16-byte pieces
  const Buf bufs[] = {
      {"h", h, n * sh, 16},         {"o_pre", o_pre, n * so, 16},
      {"gamma", gamma, (size_t)(H * d_v) * 4, 16}, {"beta", beta, (size_t)(H * d_v) * 4, 16},
      {"y", y, n * sh, 16},
  };
  for (const Buf& b : bufs)
    if (b.p && !aligned(b))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", b.name, b.align);
  for (int i = 1; i < 4; ++i)
    if (overlaps(bufs[4], bufs[i])) return fail(MLSTM_ERR_INVALID_ARG, "y overlaps %s", bufs[i].name);
  if (y != h && overlaps(bufs[4], bufs[0]))
    return fail(MLSTM_ERR_INVALID_ARG, "y overlaps h without being h");
  mlstm::GnArgs a{};
  a.rows = B * H * T; a.H = H; a.T = T; a.dv = (int)d_v;
  a.h_bf16 = h_dtype == MLSTM_BF16; a.o_bf16 = o_dtype == MLSTM_BF16; a.eps = eps;
  a.h = h; a.o_pre = o_pre; a.gamma = gamma; a.beta = beta; a.y = y;
  return device_status(mlstm::launch_groupnorm_ogate(a, static_cast<hipStream_t>(stream)),
                       "groupnorm_ogate");
}

mlstm_status_t mlstm_causal_conv1d(int64_t B, int64_t T, int64_t C, int64_t K,
                                   mlstm_dtype_t dtype, const void* x, const float* w,
                                   const float* bias, const float* state_in, void* y,
                                   float* state_out, void* stream) {
  if (B < 0 || T < 0 || C <= 0 || K <= 0)
    return fail(MLSTM_ERR_INVALID_ARG,
                "sizes must be non-negative and C, K positive (B=%lld T=%lld C=%lld K=%lld)",
                (long long)B, (long long)T, (long long)C, (long long)K);
  if (dtype != MLSTM_F32 && dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (B == 0) return ok();
  if (T == 0) {   // no tokens: the carried window passes through
    if (K > 8) return fail(MLSTM_ERR_UNSUPPORTED, "K=%lld: at most 8", (long long)K);
    const size_t ns = (size_t)(B * (K - 1) * C) * 4;
    const StateBufs sb{{"state_out", "", "", ""}, {state_in, nullptr, nullptr, nullptr},
                       {state_out, nullptr, nullptr, nullptr}, {ns, 0, 0, 0}, 1};
    return pass_state(sb, "causal conv with T = 0", static_cast<hipStream_t>(stream));
  }
  if (!x || !w || !y) return fail(MLSTM_ERR_INVALID_ARG, "x, w and y are required");
  if (K > 8) return fail(MLSTM_ERR_UNSUPPORTED, "K=%lld: at most 8", (long long)K);
  const int64_t ve = dtype == MLSTM_BF16 ? 8 : 4;
  if (C % ve != 0)
    return fail(MLSTM_ERR_UNSUPPORTED, "C=%lld: need a multiple of %lld", (long long)C, (long long)ve);
  if (B * T * C > ((int64_t)1 << 40))
    return fail(MLSTM_ERR_UNSUPPORTED, "B*T*C=%lld too large", (long long)(B * T * C));
  const size_t n = (size_t)(B * T * C), sx = dsize(dtype), ns = (size_t)(B * (K - 1) * C) * 4;
  const Buf bufs[] = {
      {"x", x, n * sx, 16},            {"w", w, (size_t)(C * K) * 4, 4},
      {"bias", bias, (size_t)C * 4, 4}, {"state_in", state_in, ns, 4},
      // outputs from here (index 4 on)
      {"y", y, n * sx, 16},            {"state_out", state_out, ns, 4},
  };
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", bufs[i].name, bufs[i].align);
  for (int o = 4; o < nb; ++o)
    for (int i = 0; i < nb; ++i)
      if (i != o && overlaps(bufs[o], bufs[i]))
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
  mlstm::ConvArgs a{};
  a.B = B; a.T = T; a.C = C; a.K = (int)K; a.x_bf16 = dtype == MLSTM_BF16;
  a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = y; a.state_out = state_out;
  return device_status(mlstm::launch_causal_conv(a, static_cast<hipStream_t>(stream)),
                       "causal_conv1d");
}

mlstm_status_t mlstm_slstm_fwd(const mlstm_slstm_problem_t* p, const void* wx, const float* R,
                               const float* c0, const float* n0, const float* m0,
                               const float* h0, void* h, float* c1, float* n1, float* m1,
                               float* h1, void* stream) {
  if (!p) return fail(MLSTM_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->B < 0 || p->NH < 0 || p->T < 0 || p->DH <= 0)
    return fail(MLSTM_ERR_INVALID_ARG,
                "sizes must be non-negative and DH positive (B=%lld NH=%lld T=%lld DH=%lld)",
                (long long)p->B, (long long)p->NH, (long long)p->T, (long long)p->DH);
  if (p->x_dtype != MLSTM_F32 && p->x_dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown x_dtype %d", p->x_dtype);
  if (p->fgate != MLSTM_FGATE_SIGMOID && p->fgate != MLSTM_FGATE_EXP)
    return fail(MLSTM_ERR_INVALID_ARG, "unknown fgate %d", p->fgate);
  if (p->B * p->NH == 0) return ok();
  if (p->T == 0) {   // no steps: the final state is the initial one (zeros without it)
    const size_t stb = (size_t)(p->B * p->NH * p->DH) * 4;
    const StateBufs sb{{"c1", "n1", "m1", "h1"}, {c0, n0, m0, h0}, {c1, n1, m1, h1},
                       {stb, stb, stb, stb}, 4};
    return pass_state(sb, "sLSTM with T = 0", static_cast<hipStream_t>(stream));
  }
  if (!wx || !R || !h) return fail(MLSTM_ERR_INVALID_ARG, "wx, R and h are required");
  const int in_state = (c0 != nullptr) + (n0 != nullptr) + (m0 != nullptr) + (h0 != nullptr);
  if (in_state != 0 && in_state != 4)
    return fail(MLSTM_ERR_INVALID_ARG, "initial state must be all of c0, n0, m0, h0 or none");
  const int out_state = (c1 != nullptr) + (n1 != nullptr) + (m1 != nullptr) + (h1 != nullptr);
  if (out_state != 0 && out_state != 4)
    return fail(MLSTM_ERR_INVALID_ARG, "final state must be all of c1, n1, m1, h1 or none");
  if (p->DH != 16 && p->DH != 32 && p->DH != 64 && p->DH != 128)
    return fail(MLSTM_ERR_UNSUPPORTED, "DH=%lld: supported 16, 32, 64, 128", (long long)p->DH);
  if (p->B * p->NH > ((int64_t)1 << 31) - 1 || p->T > ((int64_t)1 << 40))
    return fail(MLSTM_ERR_UNSUPPORTED, "B*NH or T too large");
  const size_t BH = (size_t)(p->B * p->NH), T = (size_t)p->T, DH = (size_t)p->DH;
  const size_t sx = dsize(p->x_dtype), st = BH * DH * 4;
  const Buf bufs[] = {
      {"wx", wx, BH * T * 4 * DH * sx, sx}, {"R", R, (size_t)p->NH * 4 * DH * DH * 4, 16},
      {"c0", c0, st, 4}, {"n0", n0, st, 4}, {"m0", m0, st, 4}, {"h0", h0, st, 4},
      // outputs from here (index 6 on)
      {"h", h, BH * T * DH * sx, sx},
      {"c1", c1, st, 4}, {"n1", n1, st, 4}, {"m1", m1, st, 4}, {"h1", h1, st, 4},
  };
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", bufs[i].name, bufs[i].align);
  for (int o = 6; o < nb; ++o)
    for (int i = 0; i < nb; ++i)
      if (i != o && overlaps(bufs[o], bufs[i]))
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
  mlstm::SlstmArgs a{};
  a.B = p->B; a.NH = p->NH; a.T = p->T; a.DH = (int)p->DH;
  a.x_bf16 = p->x_dtype == MLSTM_BF16; a.fgate_exp = p->fgate == MLSTM_FGATE_EXP;
  a.wx = wx; a.R = R; a.c0 = c0; a.n0 = n0; a.m0 = m0; a.h0 = h0;
  a.h = h; a.c1 = c1; a.n1 = n1; a.m1 = m1; a.h1 = h1;
  return device_status(mlstm::launch_slstm(a, static_cast<hipStream_t>(stream)), "slstm_fwd");
}

mlstm_status_t mlstm_fwd_parallel_workspace_bytes(const mlstm_problem_t* p, size_t* bytes) {
  if (!bytes) return fail(MLSTM_ERR_INVALID_ARG, "bytes is NULL");
  mlstm_status_t s = check_problem(p, true);
  if (s != MLSTM_OK) return s;
  *bytes = mlstm::parallel_workspace(problem_args(p));
  return ok();
}

mlstm_status_t mlstm_fwd_parallel(const mlstm_problem_t* p, const void* q, const void* k,
                                  const void* v, const float* i_pre, const float* f_pre,
                                  const void* o_pre, const float* C0, const float* n0,
                                  const float* m0, void* h, float* C1, float* n1, float* m1,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (p && check_problem(p, true) == MLSTM_OK && seq_is_empty(p))
    return seq_empty(p, C0, n0, m0, C1, n1, m1, stream);
  mlstm::SeqArgs a;
  mlstm_status_t s = check_seq(p, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1, &a);
  if (s != MLSTM_OK) return s;
  const size_t need = mlstm::parallel_workspace(a);
  if (!workspace || workspace_bytes < need)
    return fail(MLSTM_ERR_INVALID_ARG, "workspace of %zu bytes given, %zu needed",
                workspace_bytes, need);
  if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  s = check_seq_workspace(p, q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C1, n1, m1, workspace,
                          need);
  if (s != MLSTM_OK) return s;
  return device_status(mlstm::launch_parallel(a, workspace, static_cast<hipStream_t>(stream)),
                       "parallel");
}

mlstm_status_t mlstm_step(const mlstm_problem_t* p, const void* q, const void* k, const void* v,
                          const float* i_pre, const float* f_pre, const void* o_pre,
                          const float* C_in, const float* n_in, const float* m_in,
                          float* C_out, float* n_out, float* m_out, void* h, void* stream) {
  mlstm_status_t s = check_problem(p, false);
  if (s != MLSTM_OK) return s;
  if (p->B * p->H == 0) return ok();   // no heads: nothing to do
  if (!q || !k || !v || !i_pre || !f_pre || !C_in || !n_in || !m_in || !C_out || !n_out ||
      !m_out || !h)
    return fail(MLSTM_ERR_INVALID_ARG,
                "q, k, v, i_pre, f_pre, C_in, n_in, m_in, C_out, n_out, m_out and h are required");
  const size_t BH = (size_t)(p->B * p->H), dqk = (size_t)p->d_qk, dv = (size_t)p->d_v;
  const size_t sq = dsize(p->qkv_dtype);
  const Buf bufs[] = {
      {"q", q, BH * dqk * sq, 4},     {"k", k, BH * dqk * sq, 4},
      {"v", v, BH * dv * sq, 16},     {"i_pre", i_pre, BH * 4, 4},
      {"f_pre", f_pre, BH * 4, 4},    {"o_pre", o_pre, BH * dv * dsize(p->o_dtype), 4},
      {"C_in", C_in, BH * dqk * dv * 4, 16}, {"n_in", n_in, BH * dqk * 4, 4},
      {"m_in", m_in, BH * 4, 4},      {"C_out", C_out, BH * dqk * dv * 4, 16},
      {"n_out", n_out, BH * dqk * 4, 4}, {"m_out", m_out, BH * 4, 4},
      {"h", h, BH * dv * sq, 4},
  };
  const int nb = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < nb; ++i)
    if (bufs[i].p && !aligned(bufs[i]))
      return fail(MLSTM_ERR_INVALID_ARG, "%s is not %zu-byte aligned", bufs[i].name, bufs[i].align);
  // outputs 9..12: an output may equal its own input exactly (in place), nothing else
  for (int o = 9; o < nb; ++o) {
    for (int i = 0; i < nb; ++i) {
      if (i == o || !overlaps(bufs[o], bufs[i])) continue;
      const bool same_state = (o <= 11) && (i == o - 3) && bufs[o].p == bufs[i].p;
      if (!same_state)
        return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
    }
  }
  mlstm::StepArgs a;
  a.B = p->B; a.H = p->H; a.dqk = p->d_qk; a.dv = p->d_v;
  a.qkv_bf16 = p->qkv_dtype == MLSTM_BF16;
  a.o_mode = o_pre ? (p->o_dtype == MLSTM_BF16 ? mlstm::O_BF16 : mlstm::O_F32) : mlstm::O_NONE;
  a.fgate_exp = p->fgate == MLSTM_FGATE_EXP;
  a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
  a.C_in = C_in; a.n_in = n_in; a.m_in = m_in; a.C_out = C_out; a.n_out = n_out;
  a.m_out = m_out; a.h = h;
  return device_status(mlstm::launch_step(a, static_cast<hipStream_t>(stream)), "step");
}

}  // extern "C"
