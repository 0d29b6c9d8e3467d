/*
 * gla.h -- C ABI of the causal gated-linear-attention (GLA) forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (per batch b and head h), following the pages:
 *   "Attention is recurrent", sections "Linear attention" and "Gated linear
 *   attention": once the softmax is removed, the history folds into a fixed-size
 *   state that is updated once per token, and a gate alpha_n makes it forget;
 *   "Gated Linear Attention", section "GLA / Recurrent Form": the gate
 *   G_t = alpha_t 1^T acts as Diag(alpha_t) on the state, and the Mamba2 form
 *   G_t = gamma_t 1 1^T uses one scalar gamma_t (also section "Motivation");
 *   "Transformers are RNNs" notes, feature-map paragraph: phi applied to q and k.
 *
 *     S_t = Diag(alpha_t) S_{t-1} + phi(k_t) v_t^T          S_t is d_k x d_v, fp32
 *     o_t = S_t^T phi(q_t)                                  (reads the updated state)
 *
 * with alpha_t = exp(g_t) (key-dimension gate), alpha_t = exp(g_t) * 1 (scalar
 * gate) or alpha_t = 1 (no gate), and S_{-1} = s0 (zero when s0 is NULL).
 * No normaliser and no 1/sqrt(d) scaling are applied; callers pre-scale q and k.
 *
 * gla_prefill_chunked computes all outputs of a known prompt with the chunkwise
 * block-parallel form ("Gated Linear Attention", Summary: chunks of C tokens
 * interpolate between the parallel and the recurrent form, cost
 * O(L C d + L d^2)); gla_decode_step performs one token of the recurrence on a
 * state held in device memory ("Attention is recurrent", Linear attention: o_n
 * is a function of S_{n-1}, q_n, k_n, v_n only).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *    16-byte aligned (scalar-mode gates: 4-byte aligned).  The caller owns every
 *    buffer; prefill and decode never allocate device memory and keep no state
 *    between calls.
 *  - Layouts: q, k: [B][H][L][d_k]; v, o: [B][H][L][d_v] (decode: L absent);
 *    key-dim gates g: [B][H][L][d_k]; scalar gates g: [B][H][L]; states s0,
 *    s_final, state: [B][H][d_k][d_v], always fp32; gates always fp32 natural-log
 *    values g = log(alpha), finite and <= 0 (outside that domain results are
 *    undefined; the library does not scan device data to check it).  Every finite
 *    log-gate <= 0 is exact up to rounding, however strong: the chunkwise
 *    form scales keys by exp(-(sum of the chunk's log-gates up to that token)), and a
 *    chunk whose log-gates sum below -100 / log2(e) (about -69.3) in some key
 *    dimension (a scalar gate counts in every key dimension) is computed token by
 *    token instead, inside the same launch.  Such
 *    chunks cost several times a regular chunk; the result does not depend on which
 *    form a chunk took beyond rounding.
 *  - q, k, v and o share one dtype (GLA_F32 or GLA_BF16); bf16 results are rounded
 *    to nearest even.  Arithmetic: fp32 accumulation and fp32 state; with bf16
 *    inputs the matrix-core operands are bf16.
 *  - Supported sizes: d_k, d_v in {16, 32, 64, 128}; chunk in {16, 32, 64}, and
 *    for the GLA prefills (gla_prefill_chunked, _noalloc and _norm) also 128 when
 *    d_k <= 64 (toward the parallel end of the chunkwise form; at d_k = 128 a chunk
 *    of 128 rows leaves room for only one operand buffer in a compute unit's 160 KiB
 *    of LDS and its fragments do not fit in registers, so it is rejected);
 *    B, H >= 1; L >= 0 (L need not be a multiple of chunk; L == 0 only copies the
 *    initial state to s_final); per head (L + chunk) * max(d_k, d_v) * 4 < 2^31
 *    bytes (L up to about 4.19 million tokens at d = 128), else GLA_ERR_SHAPE.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument validation is host-only and runs before any HIP call: on
 *    any error nothing is launched and nothing is written.  Faults during
 *    execution surface at the caller's next synchronisation of the stream.
 *  - Every entry point returns GLA_OK (0) or a negative gla_status.
 *    gla_last_error_detail() gives a message for the last failure on the calling
 *    thread.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GLA_OK = 0,
    GLA_ERR_NULL = -1,        /* a required pointer is NULL                          */
    GLA_ERR_SHAPE = -2,       /* a size is negative or zero where it must be positive */
    GLA_ERR_UNSUPPORTED = -3, /* d_k, d_v, chunk, dtype, gate mode or feature map     */
    GLA_ERR_ALIGN = -4,       /* a pointer is not aligned as documented below         */
    GLA_ERR_ALIAS = -5,       /* an output overlaps an input it must not overlap      */
    GLA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed           */
    GLA_ERR_OOM = -7,         /* gla_state_alloc could not allocate                   */
    GLA_ERR_WORKSPACE = -8    /* workspace missing or smaller than required           */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

typedef enum {
    GLA_GATE_NONE = 0,    /* alpha = 1 (plain linear attention); g must be NULL      */
    GLA_GATE_KEYDIM = 1,  /* alpha_t = exp(g_t), one log-gate per key dimension      */
    GLA_GATE_SCALAR = 2   /* alpha_t = exp(g_t) * 1, one log-gate per token and head */
} gla_gate_mode;

typedef enum {
    GLA_PHI_IDENTITY = 0, /* phi(x) = x                                              */
    GLA_PHI_ELU1 = 1      /* phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise    */
} gla_feature_map;

typedef void *gla_stream_t; /* a hipStream_t */

/*
 * gla_state_alloc -- allocate a zero-filled fp32 state [B][H][d_k][d_v] on the
 * current device for gla_decode_step (the fixed-size state that replaces the
 * KV cache: "Attention is recurrent", Linear attention).  The zero fill is
 * enqueued on `stream`.  *state receives the device pointer; release it with
 * gla_state_free.  Errors: GLA_ERR_NULL (state == NULL), GLA_ERR_SHAPE,
 * GLA_ERR_UNSUPPORTED (d_k / d_v), GLA_ERR_OOM, GLA_ERR_HIP.  On error *state is
 * left unchanged.
 */
int gla_state_alloc(int B, int H, int d_k, int d_v, float **state, gla_stream_t stream);

/*
 * gla_state_free -- synchronise `stream` and free a state from gla_state_alloc.
 * NULL is accepted and ignored.  Errors: GLA_ERR_HIP.
 */
int gla_state_free(float *state, gla_stream_t stream);

/*
 * gla_prefill_workspace_bytes -- size in bytes of the device workspace that
 * gla_prefill_chunked needs for these sizes (0 when none).  Returns 0 also for
 * invalid sizes (gla_prefill_chunked reports those).
 */
size_t gla_prefill_workspace_bytes(int B, int H, int L, int d_k, int d_v, int chunk,
                                   gla_dtype dtype);

/*
 * gla_prefill_chunked -- outputs of every token of a known prompt and the final
 * state, by the chunkwise block-parallel form ("Gated Linear Attention", Summary
 * and Methodology; "Attention is recurrent", Prefill: the prefix states form a
 * (weighted) scan).  Inside each chunk of `chunk` tokens the masked products run
 * on the matrix cores; chunks are chained through the fp32 state.  The result
 * equals the token recurrence above for any chunk size up to rounding.
 *
 *   q, k      in   [B][H][L][d_k], dtype (may be NULL when L == 0, as may v, o)
 *   v         in   [B][H][L][d_v], dtype
 *   g         in   fp32 log-gates, [B][H][L][d_k] (KEYDIM) / [B][H][L] (SCALAR);
 *                  must be NULL for GLA_GATE_NONE; may be NULL when L == 0
 *   s0        in   fp32 [B][H][d_k][d_v] initial state, or NULL for zero
 *   o         out  [B][H][L][d_v], dtype
 *   s_final   out  fp32 [B][H][d_k][d_v] state after the last token, or NULL;
 *                  may equal s0 (update in place) but must not partially overlap it
 *                  (in place with a workspace, s0 is first copied into it)
 *   workspace      device scratch of at least gla_prefill_workspace_bytes(...)
 *                  bytes (NULL allowed when that is 0); contents are clobbered
 *
 * o must not overlap q, k, v, g, s0, s_final or the workspace; s_final must not
 * overlap q, k, v, g or the workspace; the workspace must not overlap any argument.
 * Errors: GLA_ERR_NULL, GLA_ERR_SHAPE,
 * GLA_ERR_UNSUPPORTED, GLA_ERR_ALIGN, GLA_ERR_ALIAS, GLA_ERR_WORKSPACE, GLA_ERR_HIP.
 */
int gla_prefill_chunked(const void *q, const void *k, const void *v, const float *g,
                        gla_gate_mode gate, const float *s0, void *o, float *s_final,
                        int B, int H, int L, int d_k, int d_v, int chunk, gla_dtype dtype,
                        gla_feature_map phi, void *workspace, size_t workspace_bytes,
                        gla_stream_t stream);

/*
 * gla_prefill_chunked_noalloc -- gla_prefill_chunked for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation).  It allocates nothing and takes no workspace: when the sizes need one
 * (few long sequences, split into segments), it uses a scratch array that the library
 * holds in the device memory of each GPU it runs on, 32 MiB, kept until the process
 * ends; that covers the workspace of every size the library's launch plan segments.
 * Arguments, results and errors as gla_prefill_chunked without the workspace; a
 * workspace need (gla_prefill_workspace_bytes) above 32 MiB returns GLA_ERR_WORKSPACE.  Every call on one GPU shares that GPU's array: calls that may
 * overlap in time on one GPU (other streams, other threads) race, so callers order
 * them on one stream or otherwise serialise them.  The first call on a device looks up
 * the array's address there (a HIP call, after validation).
 */
int gla_prefill_chunked_noalloc(const void *q, const void *k, const void *v, const float *g,
                                gla_gate_mode gate, const float *s0, void *o, float *s_final, int B, int H,
                                int L, int d_k, int d_v, int chunk, gla_dtype dtype, gla_feature_map phi,
                                gla_stream_t stream);

/*
 * gla_decode_step -- one token of the recurrence on a resident state: for every
 * (b, h), state <- Diag(alpha) state + phi(k) v^T in place, then
 * o = state^T phi(q) ("Attention is recurrent", Linear attention and Gated linear
 * attention; "Gated Linear Attention", Recurrent Form and its dataflow chart).
 *
 *   q, k      in      [B][H][d_k], dtype
 *   v         in      [B][H][d_v], dtype
 *   g         in      fp32 [B][H][d_k] (KEYDIM) / [B][H] (SCALAR) / NULL (NONE)
 *   state     in/out  fp32 [B][H][d_k][d_v]
 *   o         out     [B][H][d_v], dtype
 *
 * o must not overlap state, q, k, v or g; state must not overlap q, k, v or g.
 * Errors: GLA_ERR_NULL, GLA_ERR_SHAPE, GLA_ERR_UNSUPPORTED, GLA_ERR_ALIGN,
 * GLA_ERR_ALIAS, GLA_ERR_HIP.
 */
int gla_decode_step(const void *q, const void *k, const void *v, const float *g,
                    gla_gate_mode gate, float *state, void *o, int B, int H, int d_k, int d_v,
                    gla_dtype dtype, gla_feature_map phi, gla_stream_t stream);

/*
 * gla_prefill_chunked_norm -- the normalised form of gla_prefill_chunked ("Transformers
 * are RNNs" notes: the kernel-weighted sum of values divided by the sum of the same
 * weights, numerator and denominator both through the feature map).  Beside S the
 * recurrence carries the normaliser state z, the state of a value that is 1 in every
 * token, with the same gate:
 *
 *     z_t = alpha_t (*) z_{t-1} + phi(k_t)        z is d_k, fp32; z_{-1} = z0 (or 0)
 *     o_t = (S_t^T phi(q_t)) / (phi(q_t) . z_t)
 *
 * Arguments as gla_prefill_chunked, plus
 *   z0        in   fp32 [B][H][d_k] initial normaliser state, or NULL for zero
 *   z_final   out  fp32 [B][H][d_k] normaliser state after the last token, or NULL;
 *                  must not overlap z0 (GLA_ERR_ALIAS): every workgroup of a head
 *                  reads all of z0, so it cannot be rewritten in place
 * No workspace is used.  The denominator must not vanish: no epsilon is added.  With
 * phi = elu+1 (positive features) and z0 = 0 it is positive for every token; with
 * the identity map it can be zero or negative, and such outputs are undefined.  o
 * must not overlap any other argument; s_final and z_final must not overlap any
 * input.  Errors as gla_prefill_chunked (no GLA_ERR_WORKSPACE).
 */
int gla_prefill_chunked_norm(const void *q, const void *k, const void *v, const float *g,
                             gla_gate_mode gate, const float *s0, const float *z0, void *o,
                             float *s_final, float *z_final, int B, int H, int L, int d_k,
                             int d_v, int chunk, gla_dtype dtype, gla_feature_map phi,
                             gla_stream_t stream);

/*
 * gla_decode_step_norm -- one token of the normalised recurrence on resident states:
 * state <- Diag(alpha) state + phi(k) v^T and z <- alpha (*) z + phi(k) in place, then
 * o = state^T phi(q) / (phi(q) . z).  Arguments as gla_decode_step, plus
 *   z         in/out  fp32 [B][H][d_k] normaliser state (required)
 * z must not overlap q, k, v, g, state or o.  Errors as gla_decode_step.
 */
int gla_decode_step_norm(const void *q, const void *k, const void *v, const float *g,
                         gla_gate_mode gate, float *state, float *z, void *o, int B, int H, int d_k,
                         int d_v, gla_dtype dtype, gla_feature_map phi, gla_stream_t stream);

/*
 * The delta rule ("Attention is recurrent", sections "Delta attention" and the
 * "Prefill" section after it).  Before each write the state is asked what it already
 * predicts for the key, and only the prediction error is written, scaled by the write
 * strength beta_t:
 *
 *     u_t = beta_t (v_t - S_{t-1}^T k_t)                u_t is d_v
 *     S_t = S_{t-1} + k_t u_t^T,     o_t = S_t^T q_t     (reads the updated state)
 *
 * with S_{-1} = s0 (zero when NULL).  No gate, no feature map and no key
 * normalisation are applied: callers scale keys (unit-norm keys and beta in [0, 1]
 * keep every step I - beta k k^T a contraction) and queries themselves.
 *
 * gla_delta_workspace_bytes -- bytes of device workspace gla_prefill_delta needs: 0
 * for chunks of 16 or 32 tokens (one fused kernel), and for chunks of 64
 * B*H*ceil(L/chunk)*chunk*(d_k + d_v) elements of the input dtype.  0 for L == 0 or
 * invalid sizes (gla_prefill_delta reports those).
 */
size_t gla_delta_workspace_bytes(int B, int H, int L, int d_k, int d_v, int chunk,
                                 gla_dtype dtype);

/*
 * gla_prefill_delta -- all outputs of a prompt under the delta rule.  Within a chunk
 * of `chunk` tokens the writes solve one unit lower-triangular system (the page's
 * prefill argument applied to a chunk that starts from a nonzero state).  Chunks of
 * 16 or 32 tokens: one kernel solves chunk n+1's system while it carries the state
 * through chunk n (no workspace).  Chunks of 64: the chunks' state-free parts are
 * computed for all chunks in parallel into the workspace, then a pass over each
 * head's chunks in order carries the state.
 *   q, k      in   [B][H][L][d_k], dtype
 *   v         in   [B][H][L][d_v], dtype
 *   beta      in   fp32 [B][H][L] write strengths (4-byte aligned)
 *   s0        in   fp32 [B][H][d_k][d_v] initial state, or NULL for zero
 *   o         out  [B][H][L][d_v], dtype
 *   s_final   out  fp32 [B][H][d_k][d_v] state after the last token, or NULL; may
 *                  equal s0 (in-place update) but must not partially overlap it
 *   chunk     16, 32 or 64
 *   workspace device scratch of at least gla_delta_workspace_bytes(...) bytes,
 *             16-byte aligned (NULL allowed when that is 0); contents are clobbered
 * Sizes and dtypes as for gla_prefill_chunked.  o must not overlap any other
 * argument; s_final and the workspace must not overlap any input.  Errors:
 * GLA_ERR_NULL, GLA_ERR_SHAPE, GLA_ERR_UNSUPPORTED, GLA_ERR_ALIGN, GLA_ERR_ALIAS,
 * GLA_ERR_WORKSPACE, GLA_ERR_HIP.
 */
int gla_prefill_delta(const void *q, const void *k, const void *v, const float *beta,
                      const float *s0, void *o, float *s_final, int B, int H, int L, int d_k,
                      int d_v, int chunk, gla_dtype dtype, void *workspace,
                      size_t workspace_bytes, gla_stream_t stream);

/*
 * gla_decode_step_delta -- one token of the delta rule on a resident state, in place:
 * u = beta (v - state^T k), state <- state + k u^T, o = state^T q.
 *   q, k      in      [B][H][d_k], dtype
 *   v         in      [B][H][d_v], dtype
 *   beta      in      fp32 [B][H] (4-byte aligned)
 *   state     in/out  fp32 [B][H][d_k][d_v]
 *   o         out     [B][H][d_v], dtype
 * state and o must not overlap the inputs or each other.  Errors as gla_decode_step.
 */
int gla_decode_step_delta(const void *q, const void *k, const void *v, const float *beta,
                          float *state, void *o, int B, int H, int d_k, int d_v, gla_dtype dtype,
                          gla_stream_t stream);

/*
 * gla_gate_project -- the input-side gate producer ("Gated Linear Attention", section
 * "GLA / Recurrent Form" and its flow chart: alpha_t = sigmoid(W_up W_down x_t), a
 * low-rank map from the token input to one gate per key dimension of every head).
 * Writes the natural-log gates that gla_prefill_chunked takes with GLA_GATE_KEYDIM:
 *
 *     g[b][h][t][i] = log(sigmoid(z[b][t][h*d_k + i])) / tau,
 *     z[b][t] = W_up (W_down x[b][t])
 *
 * tau = 1 is the page's form; tau > 1 gives alpha = sigmoid(z)^(1/tau).
 *   x         in   [B][L][d_model], dtype
 *   w_down    in   [rank][d_model], dtype
 *   w_up      in   [H*d_k][rank], dtype
 *   g         out  fp32 [B][H][L][d_k]; must not overlap x, w_down or w_up
 *   d_model   a multiple of 32, at most 65536;  rank 16 or 32;  d_k 16, 32, 64 or 128
 *   tau       positive and finite
 * Arithmetic: fp32 accumulation; with bf16 inputs both products take bf16
 * matrix-core operands (the rank-r code is rounded to bf16), with fp32 inputs fp32
 * ones; log and exp are the hardware base-2 instructions.  All
 * pointers 16-byte aligned.  L == 0 does nothing.  Errors: GLA_ERR_NULL,
 * GLA_ERR_SHAPE, GLA_ERR_UNSUPPORTED, GLA_ERR_ALIGN, GLA_ERR_ALIAS, GLA_ERR_HIP.
 */
int gla_gate_project(const void *x, const void *w_down, const void *w_up, float *g, int B, int L,
                     int d_model, int rank, int H, int d_k, float tau, gla_dtype dtype,
                     gla_stream_t stream);

/*
 * gla_prefill_outer -- the outer-product gate ("Gated Linear Attention", section
 * "GLA / Recurrent Form": the low-rank parameterisation G_t = alpha_t beta_t^T of the
 * general gate G_t (.) S_{t-1}), which decays the state along both dimensions:
 *
 *     S_t[i][j] = alpha_t[i] beta_t[j] S_{t-1}[i][j] + phi(k_t)[i] v_t[j]
 *     o_t = S_t^T phi(q_t)
 *
 * with alpha_t = exp(g_t) and beta_t = exp(gv_t).  Arguments as gla_prefill_chunked
 * with a key-dimension gate (chunk 16, 32 or 64 only), plus
 *   gv        in   fp32 [B][H][L][d_v] value-dimension log-gates (finite, <= 0)
 * No workspace.  Every gate strength is exact up to rounding: a chunk whose lowest
 * key-dimension and lowest value-dimension log-gate sums add up to less than
 * -100 / log2(e) is computed token by token instead (as for the key-dimension gate).
 * o must not overlap any other argument; s_final must not overlap any input (it may
 * equal s0).  Errors as gla_prefill_chunked (no GLA_ERR_WORKSPACE).
 */
int gla_prefill_outer(const void *q, const void *k, const void *v, const float *g, const float *gv,
                      const float *s0, void *o, float *s_final, int B, int H, int L, int d_k, int d_v,
                      int chunk, gla_dtype dtype, gla_feature_map phi, gla_stream_t stream);

/*
 * gla_decode_step_outer -- one token of the outer-product-gated recurrence on a
 * resident state, in place: state[i][j] <- alpha_i beta_j state[i][j] + phi(k)_i v_j,
 * then o = state^T phi(q).  Arguments as gla_decode_step with a key-dimension gate,
 * plus gv fp32 [B][H][d_v].  Errors as gla_decode_step.
 */
int gla_decode_step_outer(const void *q, const void *k, const void *v, const float *g, const float *gv,
                          float *state, void *o, int B, int H, int d_k, int d_v, gla_dtype dtype,
                          gla_feature_map phi, gla_stream_t stream);

/* gla_strerror -- static text for a gla_status value (never NULL). */
const char *gla_strerror(int status);

/* gla_last_error_detail -- message for the last non-OK status returned on the
 * calling thread ("" if none).  Valid until the next call on that thread. */
const char *gla_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
