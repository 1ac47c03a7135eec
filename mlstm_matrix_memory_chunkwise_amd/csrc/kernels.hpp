// Launch descriptors and launcher entry points of the mLSTM kernels.
// Only the C-ABI layer (api.hip) calls these; argument checking happens there.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mlstm {

// How the output gate o~ is given: absent (o = 1), float32 or bfloat16.
enum OGate : int { O_NONE = 0, O_F32 = 1, O_BF16 = 2 };

// Whole-sequence forward (chunkwise or parallel).  All pointers are device
// pointers; optional ones are nullptr.  Dtype codes: 0 = f32, 1 = bf16.
struct SeqArgs {
  int64_t B, H, T, dqk, dv;
  // Tokens t0 .. T-1 of each head are processed; heads lie Ts tokens apart in
  // q, k, v, i_pre, f_pre, o_pre and h (Ts >= T).  A whole sequence has t0 = 0
  // and Ts = T; the MFMA chunk kernels handle t0 = 0 only.
  int64_t Ts, t0;
  int qkv_bf16;     // q, k, v, h are bfloat16 (else float32)
  int o_mode;       // OGate: none / f32 / bf16
  int fgate_exp;    // forget gate: 1 = exponential, 0 = sigmoid
  const void* q;
  const void* k;
  const void* v;
  const float* i_pre;
  const float* f_pre;
  const void* o_pre;
  const float* C0;  // all three null = zero state
  const float* n0;
  const float* m0;
  void* h;
  float* C1;        // all three null = not written
  float* n1;
  float* m1;
};

struct StepArgs {
  int64_t B, H, dqk, dv;
  int qkv_bf16;
  int o_mode;
  int fgate_exp;
  const void* q;
  const void* k;
  const void* v;
  const float* i_pre;
  const float* f_pre;
  const void* o_pre;
  const float* C_in;
  const float* n_in;
  const float* m_in;
  float* C_out;
  float* n_out;
  float* m_out;
  void* h;
};

// Decode step: two launches (memory stream, then normalizer/max update).
hipError_t launch_step(const StepArgs& a, hipStream_t stream);

// Chunkwise forward.
// Returns true when the bf16 MFMA kernel covers (dqk, dv, chunk).
bool chunk_mfma_supported(const SeqArgs& a, int64_t chunk);
size_t chunk_mfma_workspace(const SeqArgs& a, int64_t chunk);
hipError_t launch_chunk_mfma(const SeqArgs& a, int64_t chunk, void* ws, hipStream_t stream);
// Chunk-64 variant with 8 waves per workgroup (two per SIMD); launch_chunk_mfma
// routes to it when it covers the shape.
bool chunk_mfma8_supported(const SeqArgs& a, int64_t chunk);
hipError_t launch_chunk_mfma8(const SeqArgs& a, hipStream_t stream);
// Chunk-64, d_qk-256 variant with state and intra-chunk wave groups pipelined
// by one chunk; launch_chunk_mfma routes to it first.
bool chunk_ws_supported(const SeqArgs& a, int64_t chunk);
hipError_t launch_chunk_ws(const SeqArgs& a, hipStream_t stream);
// Chunk-128, d_qk-256 variant with state and score wave groups pipelined by
// one chunk (P kept in registers); launch_chunk_mfma routes to it first.
bool chunk_ws128_supported(const SeqArgs& a, int64_t chunk);
hipError_t launch_chunk_ws128(const SeqArgs& a, hipStream_t stream);
// State-only pass: the final (C~, n~, m) after T tokens (T a multiple of 64)
// from (C0, n0, m0), no outputs; bf16 k/v, d_qk 64/128/256, d_v % 64 == 0.
// C1, n1, m1 are required.
bool chunk_state_supported(const SeqArgs& a);
hipError_t launch_chunk_state(const SeqArgs& a, hipStream_t stream);
// The states at the ends of Q equal segments of tokens 0 .. T-1 from weighted
// products over the tokens (state_gemm.hip): d_qk 256, d_v a multiple of 128,
// bf16.  State k goes to C_out + k B H d_qk d_v, n_out + k B H d_qk,
// m_out + k B H; needs state_gemm_workspace(a, Q) bytes of scratch.
bool state_gemm_supported(const SeqArgs& a, int Q);
size_t state_gemm_workspace(const SeqArgs& a, int Q);
hipError_t launch_state_gemm(const SeqArgs& a, int Q, float* C_out, float* n_out, float* m_out,
                             void* workspace, hipStream_t stream);
// Generic VALU chunkwise kernel (float32 path; bf16 shapes outside MFMA cover).
// Tokens t0 .. T-1 in chunks of `chunk`; the last chunk may be shorter.
hipError_t launch_chunk_valu(const SeqArgs& a, int64_t chunk, hipStream_t stream);

// Chunkwise backward pass.  Gradients are float32; d_o is written only when
// o_pre is given; dC0, dn0, dm0 may be null; dC1/dn1 null = zero.
struct BwdArgs {
  int64_t B, H, T, dqk, dv;
  int qkv_bf16, o_mode, fgate_exp;
  int L;            // chunk (16 or 32)
  const void* q;
  const void* k;
  const void* v;
  const float* i_pre;
  const float* f_pre;
  const void* o_pre;
  const float* C0;
  const float* n0;
  const float* m0;
  const void* h;    // forward output (qkv dtype)
  const void* dh;   // gradient of h (qkv dtype)
  const float* dC1;
  const float* dn1;
  float* d_q;
  float* d_k;
  float* d_v;
  float* d_i;
  float* d_f;
  float* d_o;
  float* dC0;
  float* dn0;
  float* dm0;
  // workspace pieces (set by launch_bwd)
  float* ws_C;      // float32 boundary states [bh][c][x][b] (chunk 16/32)
  uint16_t* ws_Cb;  // chunk 64: bf16 boundary states as swizzled [d_qk][64] tiles, [bh][cb][c]
  float* ws_CT;     // chunk 64: float32 final state [bh][x][b]
  float* ws_n;
  float* ws_m;
  float* ws_beta;
  float* ws_dq;     // chunk 16/32: per-column-block partials of dq, dk
  float* ws_dk;
  float* ws_s;
  float* ws_dm0;
  // chunk 64 only
  uint16_t* ws_dCb; // bf16 dC at each chunk's end, tiles as ws_Cb
  uint16_t* ws_R;   // bf16 r = sigmoid(o~) dh / den, [bh T][d_v]
  float* ws_dnq;    // normalizer gradient per token
  float* ws_dn;     // dn at each chunk's end, [bh][c][d_qk]
  float* ws_qd;     // q . dq and k . dk per d_qk slice, [slice][bh T]
  float* ws_kd;
  float* ws_csum;   // their sums over each chunk, [slice][bh][c][q, k]
  float* ws_kend;   // <dC1, C~_T> (+ <dn1, n~_T> in block 0) per column block, [cb][bh]
};
bool bwd_supported(const BwdArgs& a);
int bwd_tile_columns(const BwdArgs& a);
size_t bwd_workspace(const BwdArgs& a, size_t offsets[16]);
hipError_t launch_bwd(BwdArgs a, void* ws, hipStream_t stream);
// Backward of a sequence of T = 0 tokens: state gradients only.
hipError_t launch_bwd_empty(const BwdArgs& a, hipStream_t stream);
// words [off, off + count) of each of `rows` rows (row pitch `pitch` 32-bit
// words) set to `value`; pads sequences for the backward pass
hipError_t launch_fill_words(uint32_t* base, int64_t rows, int64_t pitch, int64_t off, int64_t count,
                             uint32_t value, hipStream_t stream);
// State and reverse passes on MFMA: bf16 q/k/v, chunk 64, d_v % 64 == 0, d_qk in {64, 128, 256}.
bool bwd_mfma_supported(const BwdArgs& a);
hipError_t launch_bwd_states_mfma(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_rev_mfma(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_qk_mfma(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_gates_mfma(const BwdArgs& a, hipStream_t stream);
int bwd_qk_slices(const BwdArgs& a);

// Block operations around the cell (block_ops.hip).
struct GnArgs {
  int64_t rows;     // B * H * T
  int64_t H, T;
  int dv;
  int h_bf16;       // h and y are bfloat16 (else float32)
  int o_bf16;       // o_pre is bfloat16 (else float32)
  float eps;
  const void* h;
  const void* o_pre;    // null: no output gate
  const float* gamma;   // [H, d_v] or null (1)
  const float* beta;    // [H, d_v] or null (0)
  void* y;
};
hipError_t launch_groupnorm_ogate(const GnArgs& a, hipStream_t stream);

struct ConvArgs {
  int64_t B, T, C;
  int K;
  int x_bf16;             // x and y are bfloat16 (else float32)
  const void* x;          // [B, T, C]
  const float* w;         // [C, K]
  const float* bias;      // [C] or null
  const float* state_in;  // [B, K-1, C] or null (zeros)
  void* y;                // [B, T, C]
  float* state_out;       // [B, K-1, C] or null
};
hipError_t launch_causal_conv(const ConvArgs& a, hipStream_t stream);

// sLSTM forward cell (slstm.hip).
struct SlstmArgs {
  int64_t B, NH, T;
  int DH;                 // 16, 32, 64 or 128
  int x_bf16;             // wx and h are bfloat16 (else float32)
  int fgate_exp;          // forget gate: 1 = exponential, 0 = sigmoid
  const void* wx;         // [B, NH, T, 4, DH] input projections of (i, f, z, o)
  const float* R;         // [NH, 4, DH, DH] recurrent matrices
  const float* c0;        // [B, NH, DH] each; all null = zero state
  const float* n0;
  const float* m0;
  const float* h0;
  void* h;                // [B, NH, T, DH]
  float* c1;              // all null = not written
  float* n1;
  float* m1;
  float* h1;
};
hipError_t launch_slstm(const SlstmArgs& a, hipStream_t stream);

// Parallel (quadratic) form.
size_t parallel_workspace(const SeqArgs& a);
hipError_t launch_parallel(const SeqArgs& a, void* ws, hipStream_t stream);

}  // namespace mlstm
