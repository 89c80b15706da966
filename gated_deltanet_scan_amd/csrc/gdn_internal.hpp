// gdn_internal.hpp -- launch descriptors shared by the C ABI layer
// (gdn_api.cpp) and the kernel translation units.  Host-side only.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Byte offset in the workspace of the per-slot (first token, length) pairs, after the chunk
// table (num_seqs + 1 entries) and the scan order (num_seqs entries).
inline size_t prefill_slot_info_offset(int32_t num_seqs)
{
    return ((2 * (size_t)num_seqs + 1) * sizeof(int32_t) + 7) / 8 * 8;
}

struct PrefillArgs {
    int32_t hqk, hv, dk, dv, chunk, io_dtype;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    int32_t num_seqs;
    int64_t total_tokens;
    const float *initial_state;
    float *final_state;
    void *o;
    void *workspace;
    int32_t max_chunks;    // chunk slots the workspace holds (upper bound on the chunks of the batch)
    size_t table_bytes;    // bytes of the chunk table, sequence order and slot entries at the start of the workspace
    int32_t seg_len;       // > 0: segment mode, local chunks per sequence per segment (0: global mode)
    int32_t max_seq_chunks;  // segment mode: chunks of the longest sequence
    bool ordered;            // host offsets show chunk counts that never increase along the batch
                             // (the scans' longest-first order is then the batch order)
    int32_t long_ranks;      // > 0: the first long_ranks ranks (longest sequences) are scanned by
                             // the row-split kernel, the rest by the whole-head kernel
    int32_t max_len;         // tokens of the longest sequence (host offsets), -1 if unknown
    int32_t win_len;         // > 0 (global mode, long_ranks > 0): the batch is run in windows of
                             // win_len local chunks of every sequence, one chunk table per window
    const int64_t *win_slots;  // host array: chunk slots of window j (ceil(max_seq_chunks / win_len))
    int32_t rest_chunks;     // chunks of the longest sequence past the first long_ranks ranks, -1 if unknown
    // optional gated RMSNorm of the output rows (o then holds y): gate, weight and eps
    const void *norm_z;
    const float *norm_weight;
    float norm_eps;
    void *stream;
};

struct DecodeArgs {
    int32_t hqk, hv, dk, dv, io_dtype;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    void *o;
    int32_t num_seqs;
    void *stream;
};

struct ConvArgs {
    int32_t dk, io_dtype, width;
    int32_t channels, nq;          // channels = 2 nq + HV dv, nq = HQK dk
    const void *x;
    const float *weight;
    const int32_t *cu_seqlens;
    int32_t num_seqs;
    int64_t tokens;
    const float *state_in;
    float *state_out;
    int32_t silu, l2norm;
    float eps;
    void *q, *k, *v;
    void *stream;
};

struct NormArgs {
    int32_t hv, dv, io_dtype;
    const void *o, *z;
    const float *weight;
    void *y;
    int64_t tokens;
    float eps;
    void *stream;
};

struct SnapshotArgs {
    const float *src;
    const int32_t *src_rows;
    int32_t src_capacity;
    float *dst;
    const int32_t *dst_rows;
    int32_t dst_capacity;
    int32_t num_rows;
    int64_t row_floats;  // HV * dk * dv
    void *stream;
};

// Whether the prefill's chunk matrices take the absorbed form (W = K^T diag(lambda) T and
// M = A T in place of T and A): bf16 io at chunk 64.  The kernels' AbsorbedForm agrees.
inline bool prefill_absorbed(int32_t io_dtype, int32_t chunk) { return io_dtype == 1 && chunk == 64; }

// Workspace layout of the prefill: [chunk table, sequence order | T (or W) matrices |
// A (or M) matrices | decay records].
struct PrefillWorkspace {
    int32_t max_chunks;
    size_t table_bytes;
    size_t total_bytes;
};

// Bytes of the library's own device scratch behind gdn_prefill_chunked_noalloc (one copy per
// device, held until the process ends).
constexpr size_t kPrefillScratchBytes = size_t(64) << 20;
// Device address of that scratch on the device of `stream` (the null stream: the current
// device), looked up once per device.
hipError_t prefill_scratch(hipStream_t stream, void **ptr, size_t *bytes);

bool prefill_supported(int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype);
bool decode_supported(int32_t dk, int32_t dv, int32_t io_dtype);
PrefillWorkspace prefill_workspace(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, int64_t total_tokens,
                                   int32_t num_seqs);
// Workspace bytes per chunk slot (the chunk matrices and the decay record of every value head).
size_t prefill_slot_bytes(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype);
// Number of longest sequences to scan apart from the rest (0: one scan kernel for the batch);
// chunks_desc: the chunk counts of the batch, longest first.
int32_t prefill_long_ranks(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, const int64_t *chunks_desc,
                           int32_t num_seqs);
// Segment length (local chunks per sequence) for a batch whose longest sequence has
// max_seq_chunks chunks; 0 selects the single-launch global mode.
int32_t prefill_segment_len(int32_t hqk, int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype,
                            int32_t num_seqs, int32_t max_seq_chunks, int32_t slot_capacity);
// Window length (local chunks of every sequence per window) of a global-mode batch whose first
// long_ranks ranks take the row-split scan; 0: one window.
int32_t prefill_window_len(int32_t hqk, int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, int32_t long_ranks,
                           int32_t max_seq_chunks);

hipError_t launch_prefill(const PrefillArgs &p);
hipError_t launch_decode(const DecodeArgs &p);
// Batches whose sequences are all at most this many tokens long (known from host offsets) take
// the token-recurrent prefill: one launch, no chunk matrices.  Measured against prep + chunk
// scan at dk = dv = 128, 32 value heads, 1-32 sequences: 2-2.5x faster at 4 tokens, even at
// 16, slower at 32 (its token steps are a chain of dependent vector products and reductions,
// about 1 us each).
constexpr int32_t kShortPrefillTokens = 8;
bool short_prefill_supported(int32_t dk, int32_t dv);
hipError_t launch_short_prefill(const PrefillArgs &p);
hipError_t launch_snapshot(const SnapshotArgs &p);
hipError_t launch_norm(const NormArgs &p);
hipError_t launch_conv(const ConvArgs &p);

}  // namespace gdn
