/*
 * mlstm.h -- C ABI of the MI355X (gfx950) mLSTM matrix-memory cell forward pass.
 *
 * The method (xLSTM post, llms.blog, "xLSTM: How Exponential Gating and Matrix
 * Memory Scale Recurrent Neural Networks"):
 *   - section 3, "Associative Matrix Cell State": memory update
 *     C_t = f_t C_{t-1} + i_t v_t k_t^T, normalizer n_t = f_t n_{t-1} + i_t k_t,
 *     retrieval h~_t = C_t q_t / max(n_t^T q_t, 1), output h_t = o_t (.) h~_t,
 *     with i_t = exp(i~_t) and f_t = exp(f~_t) or sigmoid(f~_t);
 *   - section 2, "The Normalizer State and Numerical Stabilization": the running
 *     maximum m_t = max(log f_t + m_{t-1}, i~_t) and the stabilized factors
 *     exp(log f_t + m_{t-1} - m_t), exp(i~_t - m_t);
 *   - section 3, "The Parallel Dual Form": the same outputs from the decay
 *     matrix S and H = ((Q K^T) (.) S) V, evaluated chunk by chunk with a
 *     carried state (chunkwise) or over the whole sequence at once (parallel).
 *
 * State convention.  The state is the stabilized triple (C~, n~, m) with the
 * true memory C = C~ e^m and n = n~ e^m.  C~ is stored [d_qk][d_v] (the
 * transpose of the page's v k^T, so the readout is q^T C~).  The output is
 *   h_t = sigmoid(o~_t) (.) (q_t^T C~_t) / max(|n~_t . q_t|, exp(-m_t)),
 * which equals the page's retrieval with |n^T q| in the denominator.  The
 * final m is the value of the sequential recurrence; (C~ e^{-c}, n~ e^{-c},
 * m + c) is the same memory, so compare states after rescaling to one m.
 * k is expected pre-scaled by 1/sqrt(d_qk); q is used as given.
 *
 * Layouts.  Every tensor is dense row-major (C order) with the shapes below.
 * B = batch, H = heads, T = tokens.  q, k: [B,H,T,d_qk]; v, o~, h:
 * [B,H,T,d_v]; i~, f~: [B,H,T]; C~: [B,H,d_qk,d_v]; n~: [B,H,d_qk]; m: [B,H].
 * The decode step drops the T axis.  q, k, v and h have dtype qkv_dtype; o~
 * has o_dtype; gates and state are float32.
 *
 * Memory and ownership.  Every pointer is a DEVICE pointer owned by the caller.
 * q, k, v, o~, h and C~ must be 16-byte aligned (the kernels use 16-byte
 * vector accesses on them; mlstm_step needs this only for v and C~); every
 * other pointer needs 4-byte alignment.  The library allocates nothing and keeps no
 * state between calls except a per-thread error string (and the fixed device
 * scratch of mlstm_fwd_chunkwise_noalloc); it is reentrant.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream); the library never synchronizes.  Argument checks run on the host
 * before anything is enqueued; a failed check enqueues nothing.  A launch
 * failure returns MLSTM_ERR_DEVICE; faults during execution surface at the
 * caller's next synchronization.  NaN or Inf in the inputs propagate to the
 * outputs without an error code.  Supported range: |m| <= 80 (exp(-m) stays
 * finite in float32).
 *
 * Empty inputs.  Sizes may be 0 (negative sizes, and zero head or feature
 * dimensions, are MLSTM_ERR_INVALID_ARG).  With no heads (B*H = 0), or no
 * rows for the group normalization, a call returns MLSTM_OK and enqueues
 * nothing.  With T = 0 the per-token pointers may be NULL and nothing is
 * computed for them: a final state that is asked for equals the initial state
 * (zeros without one; for the convolution, the carried window), and the
 * backward gives dC0 = dC1, dn0 = dn1 (zeros without them) and
 * dm0 = <dC1, C~0> + <dn1, n~0> (zero without an initial state).  Those
 * copies are enqueued on `stream` like any other work.
 */
#ifndef MLSTM_H
#define MLSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLSTM_OK = 0,
  MLSTM_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, misaligned or
                                overlapping buffers, partial state, bad enum,
                                workspace too small */
  MLSTM_ERR_UNSUPPORTED = 2, /* valid but not implemented: d not a multiple of
                                16 or above 512, chunk not in {16,32,64,128},
                                backward shapes without a kernel */
  MLSTM_ERR_DEVICE = 3       /* a HIP call or kernel launch failed */
} mlstm_status_t;

typedef enum { MLSTM_F32 = 0, MLSTM_BF16 = 1 } mlstm_dtype_t;

/* Forget gate: log f = logsigmoid(f~) (sigmoid gate) or log f = f~ (exp gate). */
typedef enum { MLSTM_FGATE_SIGMOID = 0, MLSTM_FGATE_EXP = 1 } mlstm_fgate_t;

typedef struct {
  int64_t B, H, T;    /* T is ignored by mlstm_step */
  int64_t d_qk, d_v;  /* head dims of q/k and of v/h */
  int32_t qkv_dtype;  /* mlstm_dtype_t of q, k, v and h */
  int32_t o_dtype;    /* mlstm_dtype_t of o~ (ignored when o~ is NULL) */
  int32_t fgate;      /* mlstm_fgate_t */
  int32_t reserved;   /* must be 0 */
} mlstm_problem_t;

/*
 * Chunkwise forward pass (section 3, "The Parallel Dual Form", evaluated one
 * chunk of `chunk` tokens at a time: the decay matrix inside a chunk, the
 * carried state between chunks).  Result does not depend on `chunk` beyond
 * rounding.
 *   q, k, v, i_pre, f_pre, h: required.
 *   o_pre: NULL means o = 1 (no output gate).
 *   C0, n0, m0: all NULL (zero state, m0 = 0) or all set.
 *   C1, n1, m1: all NULL (final state not written) or all set.
 *   State outputs must not overlap state inputs; h must not overlap any input.
 *   workspace: device scratch of at least the size given by
 *   mlstm_fwd_chunkwise_workspace_bytes (may be NULL when that size is 0);
 *   it must not overlap any other argument.
 * Any T >= 0 is accepted (T = 0: see "Empty inputs" above).  When T is not
 * a multiple of `chunk`, the last T % chunk tokens form one shorter chunk:
 * on the bf16 matrix-core path they run on the float32 vector kernel,
 * continuing from the state the first T - T % chunk tokens leave in the
 * workspace (B*H*(d_qk*d_v + d_qk + 1) floats).  A long sequence with few
 * heads (at most 128 matrix-core workgroups of 64 value columns) is split
 * into P = 16, 8, 4 or 2 equal segments: the largest P whose P-fold grid fits 256
 * compute units, with T a multiple of P chunks (and of 64 P) and at least
 * 2048 tokens per segment; P above 2 needs d_qk 256 and d_v a multiple of
 * 128.  The states at the P - 1 split points are computed first, then all
 * segments run at once.  Its workspace holds (3P - 1)*B*H states and, at
 * d_qk 256 with d_v a multiple of 128, the token segments' partial sums of
 * those states (at most 30 states per head) and per-token gate weights.
 * mlstm_fwd_chunkwise_workspace_bytes gives the size in every case.
 * Returns MLSTM_OK or an error code; on error, mlstm_last_error_detail()
 * describes it.
 */
mlstm_status_t mlstm_fwd_chunkwise(const mlstm_problem_t* p, int64_t chunk,
                                   const void* q, const void* k, const void* v,
                                   const float* i_pre, const float* f_pre,
                                   const void* o_pre, const float* C0,
                                   const float* n0, const float* m0, void* h,
                                   float* C1, float* n1, float* m1,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace needed by mlstm_fwd_chunkwise for this problem (bytes). */
mlstm_status_t mlstm_fwd_chunkwise_workspace_bytes(const mlstm_problem_t* p,
                                                   int64_t chunk, size_t* bytes);

/*
 * mlstm_fwd_chunkwise without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * mlstm_fwd_chunkwise computes, with the same kernels, and allocates nothing:
 * where that call needs a workspace (T not a multiple of `chunk` on the bf16
 * matrix-core path, or the split of a long sequence with few heads), it uses a fixed
 * device array of 64 MiB that the library holds on every GPU it runs on
 * until the process ends.
 *   Arguments, layouts and rules: as mlstm_fwd_chunkwise.  `stream` must
 *   belong to the current device (NULL: its null stream).
 *   Where the sequence split would need more than 64 MiB, it takes a form
 *   that fits: fewer segments, the state at the split point by the chunk
 *   recurrence instead of the weighted products, or no split; the result
 *   then equals mlstm_fwd_chunkwise's up to rounding instead of bit for bit.  A problem that still needs more than 64 MiB of workspace
 *   (a long tail state) returns MLSTM_ERR_UNSUPPORTED
 *   (mlstm_fwd_chunkwise_workspace_bytes gives the size) and enqueues nothing.
 *   Calls on one GPU share that GPU's array: calls whose execution overlaps
 *   on one GPU (on two streams, or from two threads) race on it and must be
 *   ordered by the caller.  Nothing in the array needs clearing between
 *   calls.
 */
mlstm_status_t mlstm_fwd_chunkwise_noalloc(const mlstm_problem_t* p, int64_t chunk,
                                           const void* q, const void* k, const void* v,
                                           const float* i_pre, const float* f_pre,
                                           const void* o_pre, const float* C0,
                                           const float* n0, const float* m0, void* h,
                                           float* C1, float* n1, float* m1, void* stream);

/*
 * Parallel (quadratic) forward pass (section 3, "The Parallel Dual Form":
 * H = ((Q K^T) (.) S) V over the whole sequence, plus the decayed initial
 * state).  Same arguments and rules as mlstm_fwd_chunkwise without `chunk`.
 * Cost grows as T^2; meant for short sequences and as a cross-check.
 */
mlstm_status_t mlstm_fwd_parallel(const mlstm_problem_t* p, const void* q,
                                  const void* k, const void* v,
                                  const float* i_pre, const float* f_pre,
                                  const void* o_pre, const float* C0,
                                  const float* n0, const float* m0, void* h,
                                  float* C1, float* n1, float* m1,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Workspace needed by mlstm_fwd_parallel for this problem (bytes). */
mlstm_status_t mlstm_fwd_parallel_workspace_bytes(const mlstm_problem_t* p,
                                                  size_t* bytes);

/*
 * One decode step for every (batch, head) (section 3, "Associative Matrix Cell
 * State", one token; section 5's constant-memory inference: the same bytes
 * are read and written at every step).
 *   q, k: [B,H,d_qk]; v, o_pre, h: [B,H,d_v]; i_pre, f_pre: [B,H].
 *   C_in, n_in, m_in: required current state.  C_out, n_out, m_out: required
 *   new state; each may equal its input pointer exactly (in-place update) but
 *   must not partially overlap it.  o_pre may be NULL (o = 1).
 */
mlstm_status_t mlstm_step(const mlstm_problem_t* p, const void* q,
                          const void* k, const void* v, const float* i_pre,
                          const float* f_pre, const void* o_pre,
                          const float* C_in, const float* n_in,
                          const float* m_in, float* C_out, float* n_out,
                          float* m_out, void* h, void* stream);

/*
 * Chunkwise backward pass: the gradient of the forward pass of
 * mlstm_fwd_chunkwise (same problem and inputs) for the scalar
 *   L = sum_t dh_t . h_t + e^{-m_T} (<dC1, C_T> + <dn1, n_T>),
 * where h is the forward output, C_T = C~_T e^{m_T} and n_T = n~_T e^{m_T} the
 * true final memory and m_T the final running maximum (held constant): dC1,
 * dn1 are gradients of the final memory in the scale of the stored final
 * state.  The pages print no gradient; this is the derivative of the
 * forward pass of section 3, "Associative Matrix Cell State" and "The
 * Parallel Dual Form", with the gates of section 2.
 *   q..m0: as for mlstm_fwd_chunkwise (C0, n0, m0 all NULL or all set).
 *   h: the forward output of the same call, [B,H,T,d_v], qkv_dtype.
 *   dh: [B,H,T,d_v], qkv_dtype.  dC1 [B,H,d_qk,d_v], dn1 [B,H,d_qk]: both
 *   NULL (zero) or both set.
 *   Outputs, all float32: dq, dk [B,H,T,d_qk]; dv [B,H,T,d_v]; di, df
 *   [B,H,T] (gradients of the preactivations i~, f~); d_o [B,H,T,d_v]
 *   (required exactly when o_pre is given); dC0 [B,H,d_qk,d_v], dn0
 *   [B,H,d_qk], dm0 [B,H] (may each be NULL): the initial-state gradients in
 *   its stored scale, dC0 = e^{m0} dL/dC_0, dn0 = e^{m0} dL/dn_0, and dm0 the
 *   derivative through the factor e^{m0} (zero without an initial state).
 *   Outputs must not overlap inputs or each other.
 *   workspace: device scratch of at least
 *   mlstm_bwd_chunkwise_workspace_bytes, 16-byte aligned, not overlapping
 *   any argument.  At chunk 16/32 it holds the state at every chunk boundary
 *   and per-column-block partial sums of dq and dk: about
 *   B*H*(T/chunk+1)*d_qk*d_v*4 + 2*(d_v/w)*B*H*T*d_qk*4 bytes with w = 32
 *   or 16.  At chunk 64 it holds the state before each chunk and the memory
 *   gradient at each chunk's end as bf16, the final state in float32, and
 *   r = sigmoid(o~) dh / den as bf16: about 2*B*H*(T/64)*d_qk*d_v*2 +
 *   B*H*d_qk*d_v*4 + B*H*T*d_v*2 bytes, plus per-token and per-chunk arrays
 *   of O(B*H*T) floats.
 *   q, k, v, h, dh, dq and dk must be 16-byte aligned; at chunk 64 also
 *   o_pre, C0, dC1, dv, d_o and dC0; every other pointer 4-byte aligned.
 * Supported: chunk 16 or 32 with d_qk <= 256 (float32 arithmetic
 * throughout), or chunk 64 with bf16 q/k/v, d_v a multiple of 64 and d_qk
 * 64, 128 or 256 (matrix products on bf16 matrix cores with float32
 * accumulation, operands such as the memory gradient rounded to bf16);
 * otherwise MLSTM_ERR_UNSUPPORTED.  The result does not depend on chunk
 * beyond rounding.  Any T >= 0 (T = 0: see "Empty inputs"); when T is not a
 * multiple of chunk, the pass runs on copies of the per-token arrays padded
 * to the next multiple Tp, at the front of the workspace (14 arrays of
 * B*H*Tp tokens each); a padding token keeps the memory unchanged and
 * contributes nothing to any gradient.
 */
mlstm_status_t mlstm_bwd_chunkwise(const mlstm_problem_t* p, int64_t chunk,
                                   const void* q, const void* k, const void* v,
                                   const float* i_pre, const float* f_pre,
                                   const void* o_pre, const float* C0,
                                   const float* n0, const float* m0,
                                   const void* h, const void* dh,
                                   const float* dC1, const float* dn1,
                                   float* dq, float* dk, float* dv, float* di,
                                   float* df, float* d_o, float* dC0,
                                   float* dn0, float* dm0, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace needed by mlstm_bwd_chunkwise for this problem (bytes). */
mlstm_status_t mlstm_bwd_chunkwise_workspace_bytes(const mlstm_problem_t* p,
                                                   int64_t chunk, size_t* bytes);

/* ---- Block operations around the cell -------------------------------------
 * The mLSTM block of the xLSTM post (llms.blog), section 4 "xLSTM Block
 * Architecture and Residual Stacking", "mLSTM Block Structure": a causal
 * depthwise convolution on the paths that feed the cell (item 3), and the
 * per-head normalization of the cell output with the output gate (item 5).
 * Both are bound by HBM bandwidth; all pointers are device pointers owned by
 * the caller, calls are asynchronous on `stream` (NULL: the null stream) and
 * every argument check runs on the host before anything is enqueued.
 */

/* Per-head group normalization with output gate:
 *   y[b,hd,t,:] = sigmoid(o_pre) * (gamma[hd] * (h - mean) / sqrt(var + eps)
 *                 + beta[hd])
 * with mean and biased variance over the d_v features of one (b, hd, t).
 *   h:     [B,H,T,d_v] in h_dtype (the cell output computed with o_pre NULL,
 *          i.e. without its own gate).
 *   o_pre: [B,H,T,d_v] in o_dtype, or NULL (no gate).
 *   gamma, beta: [H,d_v] float32, or NULL (1 and 0).
 *   eps:   added to the variance, >= 0 and finite.
 *   y:     [B,H,T,d_v] in h_dtype.  y may be h itself (in place); otherwise
 *          it must not overlap any input.
 * Supported: d_v a multiple of 4, at most 1024; B*H*T at most 2^32; h,
 * o_pre, y, gamma and beta 16-byte aligned.  Arithmetic is float32. */
mlstm_status_t mlstm_groupnorm_ogate(int64_t B, int64_t H, int64_t T, int64_t d_v,
                                     mlstm_dtype_t h_dtype, mlstm_dtype_t o_dtype,
                                     const void* h, const void* o_pre,
                                     const float* gamma, const float* beta, float eps,
                                     void* y, void* stream);

/* Causal depthwise convolution over the token axis:
 *   y[b,t,c] = bias[c] + sum_{s<K} w[c,s] x[b, t-K+1+s, c]
 * (w[c,K-1] multiplies the current token).  Inputs before t = 0 come from
 * state_in.
 *   x, y:      [B,T,C] in dtype (channels last), 16-byte aligned.
 *   w:         [C,K] float32;  bias: [C] float32 or NULL (0).
 *   state_in:  [B,K-1,C] float32, the K-1 inputs before x[:,0] oldest first,
 *              or NULL (zeros).
 *   state_out: [B,K-1,C] float32 or NULL: the last K-1 inputs of
 *              (state_in, x), to continue with the next segment.
 * No output may overlap an input or the other output.  Supported: 1 <= K <= 8,
 * C a multiple of 8 (bf16) or 4 (float32).  Arithmetic is float32. */
mlstm_status_t mlstm_causal_conv1d(int64_t B, int64_t T, int64_t C, int64_t K,
                                   mlstm_dtype_t dtype, const void* x, const float* w,
                                   const float* bias, const float* state_in, void* y,
                                   float* state_out, void* stream);

/* ---- sLSTM forward cell ------------------------------------------------------
 * The scalar-memory cell of the xLSTM post (llms.blog), section 2 "sLSTM:
 * Scalar Memory with Exponential Gating and Normalization".  Per step t,
 * head hd, unit u:
 *   pre_g = wx[b,hd,t,g,u] + sum_v R[hd,g,u,v] h_{t-1}[b,hd,v]   (g = i, f, z, o)
 *   m_t = max(log f + m_{t-1}, i~),  c_t = e^{log f + m_{t-1} - m_t} c_{t-1}
 *         + e^{i~ - m_t} z,  n_t = e^{log f + m_{t-1} - m_t} n_{t-1} + e^{i~ - m_t},
 *   h_t = sigmoid(o~) c_t / n_t
 * with log f = f~ (MLSTM_FGATE_EXP) or log sigmoid(f~) (MLSTM_FGATE_SIGMOID);
 * z is used as is (no squashing).  The state (c, n, m, h) is the stabilized
 * one; h is the gated output that feeds the next step.
 */
typedef struct {
  int64_t B, NH, T, DH;   /* batch, heads, steps, units per head */
  mlstm_dtype_t x_dtype;  /* dtype of wx and h */
  mlstm_fgate_t fgate;
} mlstm_slstm_problem_t;

/* sLSTM forward over T steps.
 *   wx: [B,NH,T,4,DH] in x_dtype, the input projections W x_t + b of the
 *       gates in the order (i, f, z, o).
 *   R:  [NH,4,DH,DH] float32, the recurrent matrices of each head
 *       (pre = R h, row index u, column index v).
 *   c0, n0, m0, h0: [B,NH,DH] float32 each, all set or all NULL (zero state).
 *   h:  [B,NH,T,DH] in x_dtype.
 *   c1, n1, m1, h1: [B,NH,DH] float32 each, all set or all NULL (not
 *       written); they may not overlap the inputs (run two buffers to chain).
 * Supported: DH = 16, 32, 64 or 128.  R must be 16-byte aligned, every
 * other pointer aligned to its element size.  One workgroup per (b, head)
 * runs the steps in order; arithmetic is float32 and the recurrent h stays
 * float32 (a bf16 h output is a rounded copy). */
mlstm_status_t mlstm_slstm_fwd(const mlstm_slstm_problem_t* p, const void* wx, const float* R,
                               const float* c0, const float* n0, const float* m0,
                               const float* h0, void* h, float* c1, float* n1, float* m1,
                               float* h1, void* stream);

/* Static description of a status code. */
const char* mlstm_status_string(mlstm_status_t s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* mlstm_last_error_detail(void);

/* Library version string. */
const char* mlstm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_H */
