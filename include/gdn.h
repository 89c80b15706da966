/*
 * gdn.h -- C ABI of libgdn, the gfx950 (MI355X) implementation of the gated
 * delta rule used by the Gated DeltaNet linear-attention layers of Qwen3.5.
 *
 * The rule (Qwen3.5-9B architecture page, section Gated DeltaNet; the NPU
 * page runs the same step token by token, section "How it works"):
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   a_t = exp(g_t)
 *     o_t = scale * S_t^T q_t
 * for each value head, with the state S (dk x dv) carried from token to
 * token.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is a pointer to DEVICE memory owned by
 *           the caller; the library never allocates, frees or keeps a
 *           pointer after the call returns.  Scratch space is passed in
 *           through `workspace`.  Tensors are dense and contiguous in the
 *           layouts given below (last index fastest).  Pointers to q, k, v,
 *           o and state tensors must be 16-byte aligned; g and beta 4-byte.
 * Heads.    HQK query/key heads serve HV value heads, HV a multiple of
 *           HQK; value head h reads query/key head floor(h * HQK / HV)
 *           (contiguous grouped-query blocks).
 * Dtypes.   q, k, v and o share one io dtype (fp32 or bf16).  g, beta and
 *           every state are fp32.  Arithmetic is fp32 (bf16 operands of the
 *           matrix cores accumulate in fp32); the state is never rounded
 *           below fp32.
 * Gate.     g is the log of the forget gate (a_t = exp(g_t)), one value per
 *           token and value head.  PRECONDITION, not checked on the device:
 *           g <= 0 and beta finite (the chunked form relies on every decay
 *           exponent being <= 0).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *           stream).  Every call only enqueues work on that stream and
 *           returns; it never synchronises and never reads device memory
 *           on the host.  Results are ready when the stream reaches them.
 * Errors.   Calls return GDN_OK or an error code; nothing throws or aborts
 *           across this boundary.  Argument errors are detected on the host
 *           BEFORE any device work is enqueued, so a failing call leaves
 *           every buffer untouched.  gdn_last_error() gives a message for
 *           the calling thread's last failure.
 * Sizes.    Supported head dimensions: dk == dv in {32, 64, 128}; chunk
 *           length in {16, 64} (chunk 16 only with dk <= 64, except fp32 io at
 *           dk = 128, whose prefill runs the token-by-token recurrence at either
 *           chunk length).  Anything else returns GDN_ERR_UNSUPPORTED.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, bad cu_seqlens (host copy) */
    GDN_ERR_UNSUPPORTED = 2,  /* a valid request this build has no kernel for */
    GDN_ERR_WORKSPACE = 3,    /* workspace missing or too small for the batch */
    GDN_ERR_HIP = 4           /* the HIP runtime refused a launch; see gdn_last_error() */
} gdn_status;

typedef enum gdn_dtype {
    GDN_DTYPE_F32 = 0,
    GDN_DTYPE_BF16 = 1
} gdn_dtype;

typedef struct gdn_shape {
    int32_t num_qk_heads; /* HQK >= 1 */
    int32_t num_v_heads;  /* HV >= 1, HV % HQK == 0 */
    int32_t dk;           /* key/query head dimension */
    int32_t dv;           /* value head dimension */
    int32_t chunk;        /* prefill chunk length C (16 or 64) */
    int32_t io_dtype;     /* gdn_dtype of q, k, v, o */
    float scale;          /* output multiplier, usually 1/sqrt(dk) */
} gdn_shape;

/*
 * Bytes of device scratch that gdn_prefill_chunked needs for a packed batch
 * of `total_tokens` tokens in `num_seqs` sequences.  Returns 0 for an
 * unsupported or invalid shape.
 */
size_t gdn_prefill_workspace_bytes(const gdn_shape *shape, int64_t total_tokens, int32_t num_seqs);

/*
 * Bytes of device scratch that gdn_prefill_chunked actually uses for the batch
 * whose host offsets are `cu_seqlens_host` ([num_seqs + 1], as for
 * gdn_prefill_chunked), when it is given those offsets: at most
 * gdn_prefill_workspace_bytes().  Long sequences are run in segments of local
 * chunks (a segment's chunk matrices stay in the last-level cache between the
 * prep and the scan), and a segment needs slots for its own chunks only: for
 * one 32768-token sequence at 32 value heads of d = 128, about 105 MB instead
 * of 420 MB.  Returns 0 for an unsupported shape or invalid offsets (negative
 * lengths, cu_seqlens_host[0] != 0).  Pure host computation.
 */
size_t gdn_prefill_workspace_bytes_for(const gdn_shape *shape, const int32_t *cu_seqlens_host, int32_t num_seqs);

/*
 * Chunked prefill over a packed batch of variable-length sequences.
 *
 * Defined by the chunkwise-parallel form on the NPU page (section "How it
 * works"): the tokens of a sequence are taken C at a time; within a chunk the
 * decay is the running sum G of g, the corrections of the chunk's writes are
 * the solution of one unit lower-triangular system (keys against earlier keys
 * of the chunk, decayed and scaled by beta), and the state entering the chunk
 * contributes to every output and to the state leaving it through decayed
 * products with the chunk's queries and keys.  Chunks are carried one after
 * the other; the triangular system is solved by forward substitution per chunk,
 * and decay exponents are masked in log space before exp (Candle pull-request
 * page, section Chunked GatedDeltaNet Scan).  The result equals the
 * token-by-token recurrence up to rounding.
 *
 *   q, k           [total_tokens, HQK, dk]  io dtype
 *   v              [total_tokens, HV, dv]   io dtype
 *   g, beta        [total_tokens, HV]       fp32
 *   cu_seqlens     [num_seqs + 1] int32, device: sequence n owns tokens
 *                  cu_seqlens[n] .. cu_seqlens[n+1]-1; cu_seqlens[0] = 0,
 *                  non-decreasing, cu_seqlens[num_seqs] = total_tokens.
 *                  Zero-length sequences are allowed (their state passes
 *                  through).
 *   cu_seqlens_host  optional host copy of the same offsets; when given it
 *                  is validated and the call fails with GDN_ERR_INVALID_ARG
 *                  on a violation.  Without it, invalid device offsets give
 *                  unspecified results but never out-of-bounds accesses.
 *                  When it shows every sequence at most 8 tokens long (and
 *                  dk = dv), the call runs the token-by-token recurrence
 *                  instead (the decode step's form, one launch, the workspace
 *                  untouched): same results up to rounding.  fp32 io at
 *                  dk = 128 always runs that recurrence (there is no chunked
 *                  kernel for it; its time grows with the longest sequence).
 *                  With it the library also plans the chunked launches from
 *                  the lengths (segments or windows of local chunks, a split
 *                  of the longest sequences into the row-split scan); the
 *                  results do not depend on the plan beyond rounding.
 *   initial_state  [num_seqs, HV, dk, dv] fp32, or NULL for zeros
 *   final_state    [num_seqs, HV, dk, dv] fp32 out; MAY alias initial_state
 *                  (in-place prefix reuse), must not overlap anything else
 *   o              [total_tokens, HV, dv] io dtype out; must not overlap
 *                  any input
 *   workspace      device scratch, 256-byte aligned; contents on entry are
 *                  ignored.  gdn_prefill_workspace_bytes() bytes always
 *                  suffice.  With cu_seqlens_host, less is accepted: the
 *                  batch is then run in segments of local chunks sized to
 *                  the workspace (gdn_prefill_workspace_bytes_for() gives the
 *                  size of the plan taken with the whole-batch workspace), and
 *                  the call fails with GDN_ERR_WORKSPACE, touching nothing,
 *                  when the workspace cannot hold one chunk of every sequence.
 *                  Without cu_seqlens_host a smaller workspace fails with
 *                  GDN_ERR_WORKSPACE.  The results do not depend on the plan.
 */
gdn_status gdn_prefill_chunked(const gdn_shape *shape,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                               const int32_t *cu_seqlens_host,
                               const float *initial_state, float *final_state,
                               void *o, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing: its chunk workspace
 * is the library's own device scratch of 64 MiB (67,108,864 bytes), one copy
 * per device, allocated when the library's code is loaded on that device and
 * held until the process ends.  Every other argument, the output and the
 * result are those of gdn_prefill_chunked.
 *
 * Limit.  A batch whose chunk workspace (gdn_prefill_workspace_bytes) fits the
 * scratch runs as with gdn_prefill_chunked.  A larger one needs
 * cu_seqlens_host: it is then run in segments of local chunks sized to the
 * scratch, which fails with GDN_ERR_WORKSPACE (and touches nothing) when even
 * one chunk per sequence does not fit (at the Qwen3.5-9B shapes, 32 value
 * heads of d = 128: 819,200 bytes per chunk slot, i.e. about 80 sequences).
 * Without cu_seqlens_host a larger batch fails with GDN_ERR_WORKSPACE.
 *
 * Sharing.  All calls on one device use the same scratch and leave their
 * contents in it (nothing has to be cleared: the calls overwrite what they
 * read).  Calls that overlap in time on one device -- on two streams, or from
 * two threads without ordering -- RACE on the scratch and give wrong results;
 * the caller must order them (for example, one stream per device).
 */
gdn_status gdn_prefill_chunked_noalloc(const gdn_shape *shape,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta,
                                       const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                       const int32_t *cu_seqlens_host,
                                       const float *initial_state, float *final_state,
                                       void *o, void *stream);

/*
 * One decode step: one new token for each of `num_seqs` independent
 * sequences, state updated IN PLACE.  Defined by the one-token matrix form
 * on the NPU page (section "How it works"): with d = exp(g) and
 * delta = beta (v - d S^T k),  o = scale (d S^T q + (q.k) delta),
 * S' = d S + k delta^T.  The state is read once and written once.
 *
 *   q, k    [num_seqs, HQK, dk]  io dtype
 *   v       [num_seqs, HV, dv]   io dtype
 *   g, beta [num_seqs, HV]       fp32
 *   state   [num_seqs, HV, dk, dv] fp32, read and overwritten
 *   o       [num_seqs, HV, dv]   io dtype out (must not overlap the state)
 */
gdn_status gdn_decode_step(const gdn_shape *shape,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, void *o, int32_t num_seqs, void *stream);

/*
 * State snapshot / restore: copies whole per-sequence states (all HV heads,
 * dk x dv fp32 each) between two state buffers, so that a verify pass can
 * be rolled back and re-fed (NPU page, "New in v2": the recurrent state
 * cannot be rewound, so it is saved before a draft is checked).
 *
 * For i in [0, num_rows): dst[dst_rows ? dst_rows[i] : i] =
 *                         src[src_rows ? src_rows[i] : i].
 *   src, dst          [capacity, HV, dk, dv] fp32 device buffers; they must
 *                     not overlap.
 *   src_rows, dst_rows  optional device int32 index arrays of num_rows
 *                     entries (gather / scatter).  Entries outside
 *                     [0, src_capacity) resp. [0, dst_capacity) are skipped.
 *                     Restore is the same call with the buffers swapped.
 *   With both index arrays NULL, num_rows must not exceed either capacity.
 */
gdn_status gdn_state_snapshot(const gdn_shape *shape,
                              const float *src, const int32_t *src_rows, int32_t src_capacity,
                              float *dst, const int32_t *dst_rows, int32_t dst_capacity,
                              int32_t num_rows, void *stream);

/*
 * The depthwise causal conv1d ahead of the recurrence, with its conv state,
 * fused with the L2 normalisation of the q and k heads.  The pages put the
 * conv in the layer ahead of the recurrence and keep one conv state per layer
 * between calls (NPU page "Qwen3.5-9B -- every component on the Intel NPU",
 * section "How it works": 24 conv states and 24 recurrent states; section
 * "New in v2": prefix reuse keeps the recurrent/conv/KV state); it is a
 * cross-correlation over the window ending at the current token, as PyTorch's
 * left-padded Conv1d (Candle pull-request page, section "Bug elimination
 * log", bug 2).  For channel c of token t of a sequence starting at token a:
 *     y[t, c] = sum_{i<K} weight[c, i] * x[t - K + 1 + i, c]
 * where x[a - m] (m = 1 .. K-1) is state_in[n, c, K-1-m] (zero with no state).
 * Then y = silu(y) = y / (1 + exp(-y)) if `silu`; the channels are
 * [q heads | k heads | v heads], and if `l2norm` each q and k head is divided
 * by sqrt(sum of its squares + eps).
 *
 *   x          [total_tokens, C] io dtype, C = 2 HQK dk + HV dv
 *   weight     [C, K] fp32, K = width in 1..8
 *   cu_seqlens DEVICE int32 [num_seqs + 1] token offsets (as for the prefill)
 *   state_in   [num_seqs, C, K-1] fp32 (oldest input first) or NULL (zeros)
 *   state_out  [num_seqs, C, K-1] fp32 or NULL (not written); receives the last
 *              K-1 inputs of each sequence (older state entries for a sequence
 *              shorter than K-1).  May be state_in itself (updated in place).
 *   q, k       [total_tokens, HQK, dk] io dtype out; v [total_tokens, HV, dv]
 * dk and dv in {32, 64, 128}.  x, weight, q, k and v 16-byte aligned.
 * Outputs must not overlap any input or each other; state_out must not
 * overlap x or weight (nor state_in partially).  With width 1 there is no
 * state: state_in and state_out are neither read nor written.
 * cu_seqlens must start at 0, be non-decreasing and end at total_tokens; this
 * is not checked on the device (other offsets give unspecified values, never
 * an access outside the buffers).
 * All buffers are caller-owned device memory; the call only enqueues work on
 * `stream` (a hipStream_t).  Argument errors are returned before any launch:
 * GDN_ERR_UNSUPPORTED for dk, dv or width outside the lists above,
 * GDN_ERR_INVALID_ARG for null, misaligned or overlapping buffers, negative
 * counts, tokens without sequences or a bad eps.  num_seqs == 0 (with
 * total_tokens == 0) is a no-op; an empty sequence keeps its state.
 */
gdn_status gdn_conv1d_qkv(const gdn_shape *shape, const void *x, const float *weight, int32_t width,
                          const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          const float *state_in, float *state_out, int32_t silu, int32_t l2norm, float eps,
                          void *q, void *k, void *v, void *stream);

/*
 * Chunked prefill whose output rows go through the gated RMSNorm of the
 * layer before they are stored (NPU page "Qwen3.5-9B -- every component on
 * the Intel NPU", section "How it works": the DeltaNet output feeds a gated
 * RMSNorm; eps 1e-6 for Qwen3.5, Candle pull-request page, section "Bug
 * elimination log", bug 7).  Every argument as for gdn_prefill_chunked, with
 * o replaced by
 *   y            [total_tokens, HV, dv] io dtype out:
 *                y = o / sqrt(mean(o^2) + eps) * norm_weight * silu(z) per
 *                (token, value head) row, silu(z) = z / (1 + exp(-z))
 * and
 *   z            [total_tokens, HV, dv] io dtype (the gate), 16-byte aligned
 *   norm_weight  [dv] fp32, shared by the heads, 16-byte aligned
 *   eps          finite, >= 0
 * y must not overlap z, norm_weight or any other input.  The norm runs on the
 * same stream right after the scans, in place on y (one pass over y and z).
 */
gdn_status gdn_prefill_chunked_gated_rmsnorm(const gdn_shape *shape,
                                             const void *q, const void *k, const void *v,
                                             const float *g, const float *beta,
                                             const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                             const int32_t *cu_seqlens_host,
                                             const float *initial_state, float *final_state,
                                             const void *z, const float *norm_weight, float eps, void *y,
                                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Conv state snapshot / restore: copies whole per-sequence conv states
 * (C x (width - 1) fp32 each, C = 2 HQK dk + HV dv channels) between two
 * buffers, so that a verify pass through the conv can be rolled back with
 * the recurrent state (NPU page "Qwen3.5-9B -- every component on the Intel
 * NPU", section "New in v2": the draft is verified after a snapshot, and prefix
 * reuse keeps the recurrent/conv/KV state).
 *
 * For i in [0, num_rows): dst[dst_rows ? dst_rows[i] : i] =
 *                         src[src_rows ? src_rows[i] : i].
 *   src, dst          [capacity, C, width - 1] fp32 device buffers, 16-byte
 *                     aligned; they must not overlap.
 *   src_rows, dst_rows  optional device int32 index arrays of num_rows
 *                     entries (gather / scatter); entries outside
 *                     [0, src_capacity) resp. [0, dst_capacity) are skipped.
 *                     Restore is the same call with the buffers swapped.
 *   With both index arrays NULL, num_rows must not exceed either capacity.
 * channels in 1..2^24, width in 1..8 (width 1: no state, a no-op);
 * C * (width - 1) must be a multiple of 4.  Caller-owned device memory; the
 * call only enqueues work on `stream`; argument errors are returned before any
 * launch.
 */
gdn_status gdn_conv_state_snapshot(int64_t channels, int32_t width,
                                   const float *src, const int32_t *src_rows, int32_t src_capacity,
                                   float *dst, const int32_t *dst_rows, int32_t dst_capacity,
                                   int32_t num_rows, void *stream);

/*
 * Gated RMSNorm of the DeltaNet output, the step right after the recurrence
 * (NPU page "Qwen3.5-9B -- every component on the Intel NPU", section "How it
 * works": the output feeds a gated RMSNorm that is scale-invariant in it; the
 * SSM norm epsilon is 1e-6 for Qwen3.5, Candle pull-request page, section "Bug
 * elimination log", bug 7).  For every token t and value head h, over the dv
 * elements of the row:
 *     y = o / sqrt(mean(o^2) + eps) * weight * silu(z),   silu(z) = z / (1 + exp(-z))
 *
 *   o, z    [tokens, HV, dv]  io dtype (z: the gate, shaped like o)
 *   weight  [dv]              fp32, shared by the heads
 *   y       [tokens, HV, dv]  io dtype out; may be o or z itself (in place),
 *                             must not overlap either partially, nor weight
 *   eps     finite, >= 0
 * Uses HV, dv and io_dtype of `shape` (dk, HQK and scale are not read beyond
 * the shape checks).  dv in {32, 64, 128}; o, z, y and weight 16-byte
 * aligned.  tokens == 0 is a no-op.
 * All buffers are caller-owned device memory; the call only enqueues work on
 * `stream` (a hipStream_t).  Argument errors are returned before any launch:
 * GDN_ERR_UNSUPPORTED for dv outside the list, GDN_ERR_INVALID_ARG for null,
 * misaligned or partially overlapping buffers, negative tokens or a bad eps.
 */
gdn_status gdn_gated_rmsnorm(const gdn_shape *shape, const void *o, const void *z, const float *weight,
                             void *y, int64_t tokens, float eps, void *stream);

/*
 * Kernel timing for benchmarks (not needed for normal use).
 * gdn_profile_enable(1) clears the record and starts timing every kernel the
 * library launches, on any thread: each launch carries a start and a stop HIP
 * event (hipExtLaunchKernelGGL) that record the kernel's own start and
 * completion on its stream; gdn_profile_enable(0) stops recording new
 * launches.
 * gdn_profile_collect() waits for the recorded events of one kernel and
 * returns how many launches were recorded and their summed duration in ms.
 * Kernel identifiers: 0 chunk table and scan order, 1 prep (Gram products and solve),
 * 2 chunk scan (state pass and outputs, any of its kernels), 3 decode, 4 snapshot,
 * 5 gated RMSNorm, 6 conv1d, 7 conv state update; and which chunk-scan kernel ran
 * (each of these launches also counts under 2): 8 the row-split scan (few
 * (sequence, head) pairs, bf16, chunk 64), 9 the whole-head scan (many pairs,
 * bf16, chunk 64, dk = 128, in a batch split by length), 10 the general scan (fp32 io
 * or chunk 16), 11 the whole-head scan of the T form (many pairs, bf16, chunk 64,
 * dk = 128); 12 the token-recurrent prefill of short sequences (every sequence at most
 * 8 tokens, known from cu_seqlens_host).
 * The events are created on first use and kept until the process ends;
 * no device memory is allocated.
 */
gdn_status gdn_profile_enable(int32_t enable);
gdn_status gdn_profile_collect(int32_t kernel, int32_t *launches, double *total_ms);

/* Static description of a status code. */
const char *gdn_status_string(gdn_status status);

/* Message of the calling thread's most recent failed call ("" if none). */
const char *gdn_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
