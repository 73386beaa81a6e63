/*
 * gdr.h — C ABI of the MI355X (gfx950) Gated Delta Rule library, libgdr.so.
 *
 * The Gated Delta Rule, per token t and per value head, on a state
 * S in R^{Dk x Dv} (rows: key dimension, columns: value dimension):
 *
 *   S     <- S * exp(g_t)           (decode: row i also scaled by exp(gk_t[i]))
 *   kv    <- S^T k_t                memory read
 *   S     <- S + k_t (beta_t (v_t - kv))^T
 *   o_t   <- scale * S^T q_t
 *
 * (lite_boost.ops.recurrent_gated_delta_rule, MindSpore Lite API page:
 * algorithm section; lite_boost.ops.chunk_gated_delta_rule: formula section;
 * the Gated DeltaNet blog post, torch_recurrent_gated_delta_rule: the decay is
 * applied before the memory read and the write is the outer product k delta^T.)
 *
 * Conventions shared by both calls
 *  - Every tensor pointer is a DEVICE pointer to a dense, row-major
 *    (C-contiguous) buffer in the layout given below; the caller owns every
 *    buffer. The library allocates nothing, keeps no state between calls and
 *    never synchronises the stream; calls are thread-safe.
 *  - The work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *    stream). Device integers are never read by the host.
 *  - Element type `dtype` applies to q, k, v, beta, the states and out:
 *    GDR_BF16 (bfloat16), GDR_F16 (IEEE half) or GDR_F32; 16-bit values are
 *    stored rounded to nearest even, and all arithmetic runs in float32
 *    (the states too) with 16-bit matrix-core operands in the I/O format.
 *    The prefill operator page accepts bf16 and fp16 inputs and returns the
 *    input's type (lite_boost.ops.chunk_gated_delta_rule, wrapper and note);
 *    float32 serves small heads. g and gk are always float32. Integers are
 *    int32.
 *  - Value head h uses key/query head h / (Nv / Nk): the repeat-interleave
 *    grouping of the blog post's layer code. Nv must be a multiple of Nk.
 *  - Fused gates (optional, both calls). Instead of beta and g, a caller may
 *    pass the layer's raw gate inputs, and the kernels form the gates as the
 *    Gated DeltaNet blog post's layer code and inferencelayer deltanet.rs
 *    (module header; its DN_STEP / DN_CHUNK kernels) do:
 *      beta = sigmoid(beta_logits),  g = -exp(A_log[h]) * softplus(gate_a + dt_bias[h])
 *    beta_logits and gate_a are (B, Nv, S) in dtype; A_log and dt_bias are
 *    (Nv) float32 per value head. The four come together, in place of beta
 *    and g (which must then be NULL). The gates are formed in float32 and
 *    never stored; positions t >= L_b are never read.
 *  - In-kernel q/k normalisation (optional, both calls): with use_qk_l2norm
 *    nonzero, q and k are replaced by x / sqrt(sum(x^2) + 1e-6) over the head
 *    dimension before use (the blog post's use_qk_l2norm_in_kernel; deltanet.rs
 *    l2norm, with eps inside the square root). Otherwise callers pass
 *    normalised vectors.
 *  - Gated RMSNorm output epilogue (optional, both calls): with norm_z and
 *    norm_w given, every output row o = out[b, h, t, :] with t < L_b is
 *    replaced by
 *      o_j * w_j * silu(z_j) / sqrt(mean_j(o_j^2) + norm_eps),
 *      silu(x) = x / (1 + exp(-x)),
 *    formed in float32 from the unrounded o (inferencelayer deltanet.rs:
 *    module header, the per-head gated RMSNorm of its step and chunk code and
 *    of DN_STEP / DN_CHUNK). norm_z is (B, Nv, S, Dv) in dtype, norm_w (Dv)
 *    float32 shared by all heads, norm_eps >= 0. A row whose o is all zeros
 *    stays zero (also with norm_eps = 0); rows t >= L_b stay exact zeros and
 *    z there is never read. The two pointers come together or not at all.
 *  - Return codes are produced on the host before anything is enqueued
 *    (except GDR_ERR_LAUNCH, from the launch itself). No value of g or gk is
 *    checked (the operator pages leave their sign unchecked on purpose).
 *  - Inputs and outputs must not overlap, except where stated.
 *  - q, k, v, the states, out, gk, norm_z and norm_w must be 16-byte aligned,
 *    and beta, g, beta_logits, gate_a, A_log and dt_bias 4-byte aligned
 *    (GDR_ERR_UNSUPPORTED otherwise); torch allocations always are.
 */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>

/* Symbols of the shared library; everything else in it is hidden. */
#if defined(__GNUC__)
#define GDR_API __attribute__((visibility("default")))
#else
#define GDR_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_NULL = 1,        /* a required pointer is NULL                      */
    GDR_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes (ValueError) */
    GDR_ERR_DTYPE = 3,       /* unknown dtype code                              */
    GDR_ERR_UNSUPPORTED = 4, /* head sizes / chunk size with no compiled kernel */
    GDR_ERR_LAUNCH = 5,      /* the kernel launch failed (RuntimeError)         */
    GDR_ERR_SCRATCH_LIMIT = 6 /* gdr_chunk_noalloc: the call needs more scratch
                                than the library's fixed array holds (ValueError) */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1, GDR_F16 = 2 } gdr_dtype;

/*
 * Recurrent decode over an indexed state pool.
 * (lite_boost.ops.recurrent_gated_delta_rule: signature, parameters, returns,
 * errors and notes — decode only, S <= 8, grouped heads.)
 *
 * Sizes: B >= 0 sequences, 1 <= S <= 8 token positions per sequence,
 *        Nk, Nv heads, head sizes Dk, Dv, num_slots >= 1 pool slots.
 * Tensors (device, row-major):
 *   q, k      (B, Nk, S, Dk)   dtype; L2-normalised by the caller unless
 *                              use_qk_l2norm is set
 *   v         (B, Nv, S, Dv)   dtype
 *   beta      (B, Nv, S)       dtype, write strength in [0, 1] (NULL with
 *                              fused gates)
 *   g         (B, Nv, S)       float32 log decay; NULL means alpha = 1 (and
 *                              with fused gates)
 *   gk        (B, Nv, S, Dk)   float32 per-key log decay, or NULL
 *   state_pool (num_slots, Nv, Dk, Dv) dtype — read and UPDATED IN PLACE
 *   actual_seq_lengths (B)     int32; L_b = clamp(value, 0, S)
 *   num_accepted_tokens (B)    int32, or NULL meaning equal to L_b
 *   ssm_state_indices (num_state_indices) int32, one slot per token
 *                              position; num_state_indices must equal B*S
 *   out       (B, Nv, S, Dv)   dtype
 *   scale_value                multiplies every output (1/sqrt(Dk) is usual)
 * Semantics per sequence b (n_b = num_accepted_tokens[b] or L_b):
 *   the entering state is read from slot ssm_state_indices[b*S + n_b - 1];
 *   tokens t = 0..L_b-1 are applied in order, carrying the state in float32;
 *   after token t the state is stored (rounded to dtype) into slot
 *   ssm_state_indices[b*S + t] (a store that token t+1 would overwrite in
 *   the same slot may be skipped); out[b, :, t] = 0 for t >= L_b.
 *   If L_b == 0, n_b is outside [1, S] or the read slot is outside
 *   [0, num_slots), the sequence writes zeros to out and touches no slot;
 *   a write slot outside [0, num_slots) skips that store only.
 *   Two sequences of one call must not share a slot (the result is undefined).
 *   A call is not idempotent: it advances the pool.
 * Supported: Dk, Dv in {16, 32, 64, 128}; all three dtypes.
 * Errors: GDR_ERR_NULL if a is NULL or q, k, v, state_pool, out,
 *   actual_seq_lengths or ssm_state_indices is NULL, beta is NULL without
 *   fused gates, or one of the four fused-gate pointers is given without the
 *   others, or one of norm_z and norm_w without the other (when B > 0);
 *   GDR_ERR_SHAPE if B < 0, S outside [1, 8], Nk, Nv, Dk, Dv or num_slots < 1,
 *   Nv % Nk != 0, num_state_indices != B*S, beta or g is given together with
 *   fused gates, or norm_eps < 0 (or NaN) with the epilogue; GDR_ERR_DTYPE;
 *   GDR_ERR_UNSUPPORTED; GDR_ERR_LAUNCH. B == 0 is a no-op.
 */
typedef struct {
    int32_t dtype;
    int32_t B, Nk, Nv, S, Dk, Dv;
    int32_t num_slots;
    int64_t num_state_indices;
    const void *q, *k, *v, *beta;
    const float *g, *gk;
    void *state_pool;
    const int32_t *actual_seq_lengths;
    const int32_t *ssm_state_indices;
    const int32_t *num_accepted_tokens;
    float scale_value;
    void *out;
    /* fused gates (see the conventions above), or NULL */
    const void *beta_logits;
    const void *gate_a;
    const float *A_log, *dt_bias;
    int32_t use_qk_l2norm;   /* 0: q and k used as given */
    /* gated RMSNorm epilogue (see the conventions above), or NULL */
    const void *norm_z;
    const float *norm_w;
    float norm_eps;
} gdr_decode_args;

GDR_API gdr_status gdr_decode(const gdr_decode_args *a, void *stream);

/*
 * Chunked prefill over padded, variable-length BNSD inputs.
 * (lite_boost.ops.chunk_gated_delta_rule: signature, parameters, formula,
 * returns; the blog post's torch_chunk_gated_delta_rule: right-padding to a
 * multiple of the chunk, in-chunk cumulative decay, the triangular solve, and
 * the pass over chunks that carries the state.)
 *
 * Sizes: B >= 0, S >= 0 (padded length), Nk, Nv, Dk, Dv, chunk_size.
 * Tensors (device, row-major):
 *   q, k      (B, Nk, S, Dk)   dtype
 *   v         (B, Nv, S, Dv)   dtype
 *   beta      (B, Nv, S)       dtype (NULL with fused gates)
 *   g         (B, Nv, S)       float32 log decay, or NULL meaning alpha = 1
 *                              (NULL with fused gates)
 *   initial_state (B, Nv, Dk, Dv) dtype, or NULL meaning zeros
 *   actual_seq_lengths (B)     int32 or NULL (all S); L_b = clamp(value, 0, S)
 *   out       (B, Nv, S, Dv)   dtype; rows t >= L_b are written as exact zeros
 *   final_state (B, Nv, Dk, Dv) dtype: the state after token L_b - 1 (the
 *                              initial state when L_b == 0). final_state MAY
 *                              alias initial_state (same pointer).
 *   scale_value                multiplies every output
 *   workspace, workspace_bytes device scratch owned by the caller, at least
 *                              gdr_chunk_workspace_size(a) bytes, 16-byte
 *                              aligned (may be NULL when that size is 0). Its
 *                              contents on entry do not matter and on return
 *                              are unspecified; calls that share a workspace
 *                              must be ordered on one stream.
 * Inputs at positions t >= L_b are never read.
 * The result equals the token-by-token recurrence up to rounding; the state
 * is carried in float32 between chunks.
 * Supported: bf16 or fp16 with Dk = Dv = 128 and chunk_size 16, 32 or 64
 *   (matrix-core path, which computes in chunks of 64 whatever the chunk
 *   size: a chunk size is a blocking of the same recurrence and changes only
 *   rounding; it first forms (I + A)^-1 of every chunk of 64 in the
 *   workspace: B * Nv * ceil(S / 64) * 6144 bytes); f32 with Dk = Dv in {16, 32} and
 *   chunk_size in {16, 32, 64}, or Dk = Dv = 64 and chunk_size in {16, 32}
 *   (no workspace).
 * Errors: GDR_ERR_NULL if a, q, k, v, out or final_state is NULL, beta is
 *   NULL without fused gates, one of the four fused-gate pointers is given
 *   without the others, one of norm_z and norm_w without the other, or
 *   workspace is NULL while a workspace is needed (when B > 0);
 *   GDR_ERR_SHAPE if B < 0, S < 0, Nk, Nv, Dk, Dv < 1, Nv % Nk != 0,
 *   chunk_size < 1, workspace_bytes is below the needed size, beta or g is
 *   given together with fused gates, or norm_eps < 0 (or NaN) with the
 *   epilogue;
 *   GDR_ERR_DTYPE; GDR_ERR_UNSUPPORTED (also for a misaligned pointer or
 *   S * D * 4 beyond 2^31 - 1); GDR_ERR_LAUNCH. B == 0 is a no-op.
 */
typedef struct {
    int32_t dtype;
    int32_t B, Nk, Nv, S, Dk, Dv;
    int32_t chunk_size;
    const void *q, *k, *v, *beta;
    const float *g;
    const void *initial_state;
    const int32_t *actual_seq_lengths;
    float scale_value;
    void *out;
    void *final_state;
    void *workspace;
    int64_t workspace_bytes;
    /* fused gates (see the conventions above), or NULL */
    const void *beta_logits;
    const void *gate_a;
    const float *A_log, *dt_bias;
    int32_t use_qk_l2norm;   /* 0: q and k used as given */
    /* gated RMSNorm epilogue (see the conventions above), or NULL */
    const void *norm_z;
    const float *norm_w;
    float norm_eps;
} gdr_chunk_args;

GDR_API gdr_status gdr_chunk(const gdr_chunk_args *a, void *stream);

/*
 * Depthwise causal conv1d + SiLU ahead of the recurrence, with the split into
 * q, k and v (the Gated DeltaNet blog post's layer code: causal_conv1d_fn /
 * causal_conv1d_update with the SiLU activation, then torch.split; inferencelayer
 * deltanet.rs: the conv ring of its step and chunk code and DN_CONV).
 *
 * The input x holds, per token, the C = 2*Nk*Dk + Nv*Dv channels of the fused
 * projection in the order (q heads | k heads | v heads). For every channel c:
 *   y_t[c] = silu(bias[c] + sum_{j=0}^{K-1} weight[c, j] * x_{t-K+1+j}[c]),
 *   silu(u) = u / (1 + exp(-u)),
 * taps oldest first, inputs before the first token taken from the carried
 * state: the last K - 1 inputs of the channel, oldest first. y is written
 * straight into q (B, Nk, S, Dk), k (B, Nk, S, Dk) and v (B, Nv, S, Dv):
 * channel c < Nk*Dk is q[b, c / Dk, t, c % Dk], the next Nk*Dk are k likewise,
 * the rest v. Rows t >= L_b of q, k and v are written as exact zeros, and
 * x there is never read. The sums run in float32, the SiLU's division as a
 * hardware reciprocal (within 1 ulp of float32); outputs are rounded once.
 *
 * Sizes: B >= 0, S >= 1 (decode: S <= 8), Nk, Nv, Dk, Dv >= 1 with Nv % Nk == 0,
 *   Dk and Dv even, 1 <= K <= 8. Tensors (device, row-major, dtype as for the
 *   recurrence; weight and bias float32):
 *   x (B, S, C); weight (C, K); bias (C) or NULL (zero).
 * Errors: GDR_ERR_NULL for a missing required pointer (when B > 0);
 *   GDR_ERR_SHAPE for sizes outside the ranges above or num_state_indices !=
 *   B*S; GDR_ERR_DTYPE; GDR_ERR_UNSUPPORTED for a misaligned pointer (x, the
 *   states and q, k, v 16-byte aligned; weight and bias 4-byte) or sizes beyond
 *   the kernels' 32-bit offsets; GDR_ERR_LAUNCH. B == 0 is a no-op.
 */

/* Prefill: initial_state (B, C, K-1) or NULL (zeros); final_state (B, C, K-1)
 * or NULL (not written) receives the last K-1 inputs after token L_b - 1
 * (taking the initial state's where L_b < K - 1) and MAY alias initial_state;
 * actual_seq_lengths (B) int32 or NULL (all S). */
typedef struct {
    int32_t dtype;
    int32_t B, S, Nk, Nv, Dk, Dv, K;
    const void *x;
    const float *weight, *bias;
    const void *initial_state;
    void *final_state;
    const int32_t *actual_seq_lengths;
    void *q, *k, *v;
} gdr_conv_prefill_args;

GDR_API gdr_status gdr_conv_prefill(const gdr_conv_prefill_args *a, void *stream);

/* Decode over an indexed pool of conv states, with the slot rule of
 * gdr_decode: state_pool (num_slots, C, K-1) is read from slot
 * ssm_state_indices[b*S + n_b - 1] (n_b = num_accepted_tokens[b], or L_b when
 * NULL) and the state after valid token t is stored into slot
 * ssm_state_indices[b*S + t]; a sequence with L_b == 0, n_b outside [1, S] or
 * a read slot outside [0, num_slots) writes zeros and touches no slot, and a
 * write slot outside that range skips that store only. A caller passes the
 * same lengths, counts and indices as to gdr_decode. */
typedef struct {
    int32_t dtype;
    int32_t B, S, Nk, Nv, Dk, Dv, K;
    int32_t num_slots;
    int64_t num_state_indices;
    const void *x;
    const float *weight, *bias;
    void *state_pool;
    const int32_t *actual_seq_lengths;
    const int32_t *ssm_state_indices;
    const int32_t *num_accepted_tokens;
    void *q, *k, *v;
} gdr_conv_decode_args;

GDR_API gdr_status gdr_conv_decode(const gdr_conv_decode_args *a, void *stream);

/*
 * gdr_chunk for callers that cannot allocate device memory: code under HIP
 * graph (stream) capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, semantics and results as gdr_chunk, except that
 * workspace and workspace_bytes are ignored: the scratch that gdr_chunk takes
 * from the caller comes from a fixed device array inside the library,
 * GDR_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends. The call itself
 * allocates nothing. Its first call on a device (the device current on the
 * calling thread, which must own `stream`) resolves the array's address once.
 * Every call on one GPU uses that GPU's single array, which keeps whatever the
 * last call left in it (nothing in it needs to start at zero): calls that can
 * run at the same time on one GPU — on different streams, or from host
 * threads without ordering between them — race on it and must not overlap;
 * calls ordered on one stream are safe.
 * Limit: gdr_chunk_workspace_size(a) <= GDR_NOALLOC_SCRATCH_BYTES; for the
 * 16-bit 128/128 path that is B * Nv * ceil(S / 64) <= 8192 chunks (the chunked
 * prefill of B = 4, Nv = 32, S = 4096 exactly). f32 calls need no scratch.
 * Errors: those of gdr_chunk (without its workspace checks), then
 *   GDR_ERR_SCRATCH_LIMIT beyond the limit (nothing is enqueued), and
 *   GDR_ERR_LAUNCH if the array's address cannot be resolved.
 */
#define GDR_NOALLOC_SCRATCH_BYTES (48LL << 20)
GDR_API gdr_status gdr_chunk_noalloc(const gdr_chunk_args *a, void *stream);

/* Bytes of workspace gdr_chunk needs for these arguments (0 if none; reads
 * dtype, B, Nv, S, Dk, Dv and chunk_size only); -1 if a is NULL. */
GDR_API int64_t gdr_chunk_workspace_size(const gdr_chunk_args *a);

/* Static, NUL-terminated description of a status code. */
GDR_API const char *gdr_status_string(gdr_status s);

/* ABI version of this header (incremented on any layout change). */
GDR_API int32_t gdr_abi_version(void);

#define GDR_ABI_VERSION 8

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
