/*
 * libgdn -- Gated DeltaNet layer core on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes; tensor pointers
 * are DEVICE memory owned by the caller.  Calls are asynchronous on the given
 * HIP stream (`stream` is a hipStream_t; NULL = the default stream).  The
 * library never allocates device memory, never synchronises the device and
 * keeps no global state; scratch memory is passed in (`ws`, `ws_bytes`) and
 * sized by the matching *_workspace() query.
 *
 * Errors: arguments are validated on the host before anything is launched.
 * An invalid call returns a non-zero gdn_status and launches nothing, so
 * outputs are left untouched.  A failed launch returns GDN_ERR_LAUNCH.
 * Every output is fully overwritten (nothing accumulates into caller
 * buffers).  Results are deterministic: no floating-point atomics are used.
 *
 * The layer core computed here is the one the three pages wire in:
 *   conv  -> gated delta rule -> gated norm
 * (prime-rl PR "Qwen3.8 Flash Next ... layers/", "What I ran": the reference
 * conv, gated-delta-rule and gated-norm calls), with the gate parameter
 * A_log holding log(A) (Megatron-LM PR "Support gated delta net for
 * Qwen3-Next (1/4)", review comment on A_log).
 *
 * Layout conventions
 *   T         total packed tokens of all sequences (varlen "THD" packing)
 *   cu_seqlens device int32 [n_seq + 1], cu[0] = 0, non-decreasing,
 *             cu[n_seq] = T; sequence n owns tokens [cu[n], cu[n+1]).
 *   x, y      [T][ld] rows of C_ch = 2*hk*dk + hv*dv channels laid out
 *             q | k | v, each block head-major (head h at h*dk).
 *   q, k      [T][ldq] with head kh at column kh*dk (views into y).
 *   v, o      [T][ldv] / [T][hv*dv] with head h at column h*dv.
 *   g, beta   fp32 [T][hv].
 *   S0, S_final, dS0, dS_final  fp32 [n_seq][hv][dv][dk] (row-major).
 *   Value head h reads key head h / (hv / hk) (grouped values).
 */
#ifndef LIBGDN_H
#define LIBGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum */
  GDN_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head dim) */
  GDN_ERR_ALIGNMENT = 3,   /* pointer or row stride not 16-byte aligned */
  GDN_ERR_WORKSPACE = 4,   /* ws too small or null */
  GDN_ERR_LAUNCH = 5       /* HIP reported an error at launch */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_FP32 = 1, GDN_FP16 = 2 } gdn_dtype; /* token tensors; params/state are fp32 */
typedef enum { GDN_ACT_SILU = 0, GDN_ACT_SIGMOID = 1 } gdn_act;

typedef struct {
  int32_t n_seq;        /* number of packed sequences (>= 1) */
  int64_t total_tokens; /* T (>= 0) */
  int32_t hk, hv;       /* key heads, value heads; hv % hk == 0 */
  int32_t dk, dv;       /* head dims; supported: dk == dv in {32, 128} */
  int32_t conv_k;       /* short-conv taps; supported: 4 */
  int32_t chunk;        /* chunk length of the WY/UT form; supported: 64 */
  gdn_dtype dtype;      /* storage type of token tensors */
  int32_t seg_chunks;   /* segment-parallel state scan: 0 = the library decides (it splits
                           sequences into segments when sequences x value heads are too few
                           to fill the GPU), > 0 = segments of this many chunks, < 0 = never
                           split.  Results are the same up to rounding; the chunk workspace
                           size depends on it. */
} gdn_shape;

const char* gdn_status_string(gdn_status s);

/* ---------------------------------------------------------------------------
 * Depthwise causal short convolution, SiLU, and L2 normalisation of q and k.
 * Conv kernel length 4 (Megatron page, "--linear-conv-kernel-dim: 4"); the
 * conv restarts at every sequence of cu_seqlens (prime-rl page, "Summary":
 * causal_conv1d takes cu_seqlens; initial_state=None) -- zero left padding,
 * no conv state in or out.  Per channel c and token t of a sequence starting
 * at t0:  u = sum_j w[c][j] x[t-3+j][c] (terms with t-3+j < t0 dropped),
 * a = u * sigmoid(u);  if l2norm_qk, every q and k head (dk channels) is then
 * divided by sqrt(sum a^2 + l2_eps).
 *   x [T][ldx], y [T][ldy] in shape->dtype; w fp32 [C_ch][4].
 *   ldx, ldy >= C_ch and multiples of 8.
 * ------------------------------------------------------------------------- */
gdn_status gdn_conv_fwd(const gdn_shape* shape, const void* x, int64_t ldx, const float* w,
                        const int32_t* cu_seqlens, int l2norm_qk, float l2_eps, void* y,
                        int64_t ldy, void* stream);

/* Backward of gdn_conv_fwd.  dy [T][lddy] -> dx [T][lddx] (shape->dtype),
 * dw fp32 [C_ch][4] (overwritten; reduced in a fixed order). */
gdn_status gdn_conv_bwd(const gdn_shape* shape, const void* x, int64_t ldx, const float* w,
                        const int32_t* cu_seqlens, int l2norm_qk, float l2_eps, const void* dy,
                        int64_t lddy, void* dx, int64_t lddx, float* dw, void* ws,
                        size_t ws_bytes, void* stream);
size_t gdn_conv_bwd_workspace(const gdn_shape* shape);

/* The convolution with a carried conv state, so that a sequence can be fed in
 * pieces over several calls (prime-rl page, "Summary": causal_conv1d with
 * initial_state and output_final_state).  The state of sequence n is the
 * three input rows just before its first token, oldest first, in the
 * storage type: conv_state [n_seq][3][C_ch] (dense rows of C_ch channels,
 * 16-byte aligned).  conv_state_in (NULL: zeros, as gdn_conv_fwd) stands for
 * x at positions cu[n] - 3 .. cu[n] - 1; conv_state_out (NULL: not written)
 * receives the input rows at positions cu[n+1] - 3 .. cu[n+1] - 1, taken from
 * conv_state_in where a sequence is shorter than three tokens (an empty one
 * passes its state through).  Feeding conv_state_out of one call as
 * conv_state_in of the next continues every sequence exactly.  Other
 * arguments as gdn_conv_fwd. */
gdn_status gdn_conv_fwd_state(const gdn_shape* shape, const void* x, int64_t ldx, const float* w,
                              const int32_t* cu_seqlens, int l2norm_qk, float l2_eps,
                              const void* conv_state_in, void* y, int64_t ldy,
                              void* conv_state_out, void* stream);

/* Backward of gdn_conv_fwd_state: dy and d_conv_state_out (the gradient of
 * conv_state_out; NULL: zero) -> dx, dw and d_conv_state_in (the gradient of
 * conv_state_in, [n_seq][3][C_ch] in the storage type; NULL: not written).
 * conv_state_in must be the forward's.  Workspace as gdn_conv_bwd. */
gdn_status gdn_conv_bwd_state(const gdn_shape* shape, const void* x, int64_t ldx, const float* w,
                              const int32_t* cu_seqlens, int l2norm_qk, float l2_eps,
                              const void* conv_state_in, const void* dy, int64_t lddy,
                              const void* d_conv_state_out, void* dx, int64_t lddx, float* dw,
                              void* d_conv_state_in, void* ws, size_t ws_bytes, void* stream);

/* gdn_conv_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as gdn_conv_bwd, without the workspace: its
 * scratch (the per-block dw partial sums) is a device array of the library,
 * GDN_CONV_BWD_NOALLOC_MAX_BYTES on every GPU the library runs on, held
 * until the process ends.  This entry point calls no hipMalloc or hipFree.
 * Shapes that need more scratch than that (gdn_conv_bwd_workspace(shape) >
 * GDN_CONV_BWD_NOALLOC_MAX_BYTES, e.g. more than 131072 tokens at 10240
 * channels) return GDN_ERR_WORKSPACE before anything is launched.  The
 * array of the current device is used (the stream must belong to it); all
 * calls on one GPU share it, so calls that overlap in time on one GPU
 * (several streams or host threads) race and must be serialised by the
 * caller.  Unlike the rest of the library this entry point keeps state: the
 * device address of each GPU's array, looked up on its first call there. */
#define GDN_CONV_BWD_NOALLOC_MAX_BYTES (32u << 20)
gdn_status gdn_conv_bwd_noalloc(const gdn_shape* shape, const void* x, int64_t ldx,
                                const float* w, const int32_t* cu_seqlens, int l2norm_qk,
                                float l2_eps, const void* dy, int64_t lddy, void* dx,
                                int64_t lddx, float* dw, void* stream);

/* ---------------------------------------------------------------------------
 * Gate (Megatron page, review comment: A_log stores log A and the forward
 * uses exp(A_log)):  g = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h]),
 * beta = sigmoid(b[t][h]).  softplus is evaluated without a threshold.
 *   a, b [T][hv] in shape->dtype; A_log, dt_bias fp32 [hv]; g, beta fp32 [T][hv].
 * ------------------------------------------------------------------------- */
gdn_status gdn_gate_fwd(const gdn_shape* shape, const void* a, const void* b, const float* A_log,
                        const float* dt_bias, float* g, float* beta, void* stream);

/* Backward of gdn_gate_fwd: da, db [T][hv] (shape->dtype); dA_log, ddt_bias
 * fp32 [hv] (sums over tokens, fixed order). */
gdn_status gdn_gate_bwd(const gdn_shape* shape, const void* a, const void* b, const float* A_log,
                        const float* dt_bias, const float* dg, const float* dbeta, void* da,
                        void* db, float* dA_log, float* ddt_bias, void* ws, size_t ws_bytes,
                        void* stream);
size_t gdn_gate_bwd_workspace(const gdn_shape* shape);

/* ---------------------------------------------------------------------------
 * Gated delta rule, chunked (WY/UT form), forward.  Per sequence and value
 * head, with S (dv x dk) starting at S0 (or zero when S0 == NULL):
 *   S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t = S_t (scale * q_t)
 * (the gated delta rule that the pages call as one kernel, prime-rl page
 * "What I ran"; initial_state / output_final_state as in its "Summary").
 * The result equals the token-by-token recurrence up to rounding; chunks of
 * 64 tokens never straddle a sequence boundary.  g must be <= 0 (as the gate
 * produces); then every exponential evaluated is <= 1.
 * Range: with 16-bit data (bf16, fp16) the MFMA operands of the passes over
 * the state are fp16 in the forward (v, the running state S, the writes
 * R = V - diag(Gam) K S^T and Delta) and in the storage type in the
 * backward (fp16 data: also the state gradient), so these must stay below
 * 65504 in magnitude: keys L2-normalised (|k| <= 1, as gdn_conv_fwd's
 * l2norm_qk gives; unnormalised keys make the recurrence grow without
 * bound), and entries of v and S0 up to ~1e3 (checked against the oracle with
 * |v| up to 4e3 and S0 ~ N(0, 1e3)).  Beyond that the results overflow to
 * inf; fp32 data has no such limit.
 * q, k, v in shape->dtype (row strides ldq, ldk, ldv, multiples of 8);
 * o [T][hv*dv] in shape->dtype; S_final may be NULL.
 * ------------------------------------------------------------------------- */
gdn_status gdn_chunk_fwd(const gdn_shape* shape, const void* q, const void* k, const void* v,
                         int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                         const float* beta, float scale, const float* S0, float* S_final,
                         const int32_t* cu_seqlens, void* o, void* ws, size_t ws_bytes,
                         void* stream);
size_t gdn_chunk_fwd_workspace(const gdn_shape* shape);

/* Backward of gdn_chunk_fwd given dout [T][hv*dv] and dS_final (NULL = 0).
 * dq [T][lddq], dk [T][lddk] (summed over each key head's group of value
 * heads), dv [T][lddv] in shape->dtype; dg, dbeta fp32 [T][hv]; dS0 fp32
 * (may be NULL).  States are recomputed, not read from the forward. */
gdn_status gdn_chunk_bwd(const gdn_shape* shape, const void* q, const void* k, const void* v,
                         int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                         const float* beta, float scale, const float* S0,
                         const int32_t* cu_seqlens, const void* dout, const float* dS_final,
                         void* dq, void* dk, void* dv, int64_t lddq, int64_t lddk, int64_t lddv,
                         float* dg, float* dbeta, float* dS0, void* ws, size_t ws_bytes,
                         void* stream);
size_t gdn_chunk_bwd_workspace(const gdn_shape* shape);

/* ---------------------------------------------------------------------------
 * The chunk calls above, split into their phases (same arguments, same
 * workspace).  Each phase reads what the previous phases left in `ws`, so
 * they must run in this order on one stream with the same shape, inputs and
 * workspace; gdn_chunk_fwd / gdn_chunk_bwd are exactly these sequences.
 * Besides letting a caller time or schedule the phases separately, each
 * phase after gdn_chunk_prepare is one or two kernel launches.
 *   forward : gdn_chunk_prepare -> gdn_chunk_fwd_states
 *   backward: gdn_chunk_prepare_bwd -> gdn_chunk_bwd_states -> gdn_chunk_bwd_reverse
 *             -> gdn_chunk_bwd_grads
 * gdn_chunk_prepare: chunk table from cu_seqlens; per (chunk, value head)
 *   the in-chunk gate sums and the WY/UT factors M = (I + A)^-1 diag(beta)
 *   and P (masked decayed scale * Q K^T), A = strictly-lower(beta D K K^T).
 * gdn_chunk_prepare_bwd: the same factors, plus the transposed operands the
 *   reverse and gradient phases read (backward workspace size); it leaves out
 *   the Q rows only gdn_chunk_fwd_states reads, so it is followed by
 *   gdn_chunk_fwd_states_save or gdn_chunk_bwd_states, not gdn_chunk_fwd_states.
 * gdn_chunk_fwd_states: sequential pass over chunks; writes o, S_final.
 * gdn_chunk_fwd_states_save: the same result after gdn_chunk_prepare_bwd,
 *   also leaving in the (backward-size) workspace what gdn_chunk_bwd_states
 *   would recompute.  Two kernel launches: a sequential pass that stores
 *   the chunk-start states (and S_final; for bf16 data also R and Delta),
 *   then a chunk-parallel pass that forms o (fp32 data: R, Delta and o)
 *   from them.  A training step can then run its
 *   backward as gdn_chunk_bwd_reverse -> gdn_chunk_bwd_grads on that
 *   workspace (same inputs, workspace untouched in between), skipping the
 *   preparation and the state pass.
 * gdn_chunk_bwd_states: the same without o: chunk-start states, R and
 *   Delta (one launch for bf16 data, two for fp32).
 * gdn_chunk_bwd_reverse: reverse pass over chunks; writes dv, dS0 and the
 *   chunk-end state gradients.  When the shape splits sequences into segments
 *   (seg_chunks), it also reads the segments' state transitions that
 *   gdn_chunk_fwd_states_save or gdn_chunk_bwd_states left in the workspace.
 * gdn_chunk_bwd_grads: chunk-parallel gradients; writes dq, dk, dg, dbeta
 *   (reads dv written by the reverse phase, and beta as the backward
 *   preparation left it in the workspace: `beta` must be the array that
 *   preparation read, and is validated but not read again).
 * ------------------------------------------------------------------------- */
gdn_status gdn_chunk_prepare(const gdn_shape* shape, const void* q, const void* k, int64_t ldq,
                             int64_t ldk, const float* g, const float* beta, float scale,
                             const int32_t* cu_seqlens, void* ws, size_t ws_bytes, void* stream);
gdn_status gdn_chunk_prepare_bwd(const gdn_shape* shape, const void* q, const void* k,
                                 int64_t ldq, int64_t ldk, const float* g, const float* beta,
                                 float scale, const int32_t* cu_seqlens, void* ws, size_t ws_bytes,
                                 void* stream);
gdn_status gdn_chunk_fwd_states(const gdn_shape* shape, const void* q, const void* k,
                                const void* v, int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const float* S0, float* S_final, const int32_t* cu_seqlens,
                                void* o, void* ws, size_t ws_bytes, void* stream);
gdn_status gdn_chunk_fwd_states_save(const gdn_shape* shape, const void* q, const void* k,
                                     const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                                     float scale, const float* S0, float* S_final,
                                     const int32_t* cu_seqlens, void* o, void* ws,
                                     size_t ws_bytes, void* stream);
gdn_status gdn_chunk_bwd_states(const gdn_shape* shape, const void* q, const void* k,
                                const void* v, int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const float* S0, const int32_t* cu_seqlens, void* ws,
                                size_t ws_bytes, void* stream);
gdn_status gdn_chunk_bwd_reverse(const gdn_shape* shape, const void* q, const void* k, int64_t ldq,
                                 int64_t ldk, float scale, const int32_t* cu_seqlens,
                                 const void* dout, const float* dS_final, void* dv, int64_t lddv,
                                 float* dS0, void* ws, size_t ws_bytes, void* stream);
gdn_status gdn_chunk_bwd_grads(const gdn_shape* shape, const void* q, const void* k, int64_t ldq,
                               int64_t ldk, const float* beta, float scale,
                               const int32_t* cu_seqlens, const void* dout, const void* dv,
                               int64_t lddv, void* dq, void* dk, int64_t lddq, int64_t lddk,
                               float* dg, float* dbeta, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Gated zero-centred RMSNorm over rows of length dv (Megatron page,
 * "--apply-layernorm-1p": zero-centred RMSNorm; prime-rl page, "Summary":
 * ZeroCenteredRMSNorm and the "silu"/"sigmoid" gate activation kwarg):
 *   y = o / sqrt(mean(o^2) + eps) * (1 + w) * act(z)
 * o, z, y [rows][dv] in dtype; w fp32 [dv] shared by all rows.
 * ------------------------------------------------------------------------- */
gdn_status gdn_gated_norm_fwd(int64_t rows, int32_t dv, gdn_dtype dtype, const void* o,
                              const void* z, const float* w, float eps, gdn_act act, void* y,
                              void* stream);

/* Backward: dout, dz [rows][dv] in dtype; dw fp32 [dv] (fixed-order sum). */
gdn_status gdn_gated_norm_bwd(int64_t rows, int32_t dv, gdn_dtype dtype, const void* o,
                              const void* z, const float* w, float eps, gdn_act act,
                              const void* dy, void* dout, void* dz, float* dw, void* ws,
                              size_t ws_bytes, void* stream);
size_t gdn_gated_norm_bwd_workspace(int64_t rows, int32_t dv);

/* ---------------------------------------------------------------------------
 * Check of cu_seqlens (prime-rl page, "Summary": the conv and the rule take
 * cu_seqlens).  Every entry point that takes cu_seqlens assumes, without
 * checking it on the device, cu[0] = 0, cu[n_seq] = total_tokens and cu
 * non-decreasing; a table that breaks this is undefined behaviour there.
 * This call runs one small kernel that reads cu_seqlens[0 .. n_seq] (device
 * int32) and writes to *violations (device int32, caller-owned) a bit mask:
 * 1 = cu[0] != 0, 2 = cu[n_seq] != total_tokens, 4 = a decrease somewhere;
 * 0 for a valid table.  Like every call it is asynchronous: read
 * *violations once the stream has run it.  It reads nothing else and needs
 * no workspace.  Errors: GDN_ERR_INVALID_ARG for a bad shape or a null
 * pointer, GDN_ERR_ALIGNMENT for a violations pointer not 4-byte aligned.
 * ------------------------------------------------------------------------- */
gdn_status gdn_check_cu_seqlens(const gdn_shape* shape, const int32_t* cu_seqlens,
                                int32_t* violations, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBGDN_H */
