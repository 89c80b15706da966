// gdn_api.cpp -- the extern "C" entry points of libgdn: argument validation
// on the host, workspace sizing and dispatch to the kernel launchers.  Every
// check runs before anything is enqueued, so an invalid call touches no
// device memory (and needs no device at all).
#include "../../include/gdn.h"
#include "gdn_internal.hpp"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <vector>

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

gdn_status ok()
{
    g_last_error[0] = '\0';
    return GDN_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t io_size(int32_t io_dtype) { return io_dtype == GDN_DTYPE_BF16 ? 2 : 4; }

// [p, p + bytes) and [r, r + rbytes) share a byte.
bool overlaps(const void *p, size_t bytes, const void *r, size_t rbytes)
{
    if (!p || !r || bytes == 0 || rbytes == 0)
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(r);
    return a < b + rbytes && b < a + bytes;
}

gdn_status check_shape(const gdn_shape *s)
{
    if (!s)
        return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
    if (s->num_qk_heads < 1 || s->num_v_heads < 1)
        return fail(GDN_ERR_INVALID_ARG, "head counts must be >= 1 (HQK=%d, HV=%d)", s->num_qk_heads,
                    s->num_v_heads);
    if (s->num_v_heads % s->num_qk_heads != 0)
        return fail(GDN_ERR_INVALID_ARG, "HV=%d is not a multiple of HQK=%d", s->num_v_heads, s->num_qk_heads);
    if (s->dk < 1 || s->dv < 1)
        return fail(GDN_ERR_INVALID_ARG, "head dimensions must be >= 1 (dk=%d, dv=%d)", s->dk, s->dv);
    if (s->io_dtype != GDN_DTYPE_F32 && s->io_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_INVALID_ARG, "io_dtype %d is neither GDN_DTYPE_F32 nor GDN_DTYPE_BF16", s->io_dtype);
    if (!std::isfinite(s->scale))
        return fail(GDN_ERR_INVALID_ARG, "scale is not finite");
    return GDN_OK;
}

}  // namespace

namespace gdn {

bool prefill_supported(int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype)
{
    if (dk != dv)
        return false;
    if (io_dtype == GDN_DTYPE_F32 && dk == 128)   // the token-recurrent kernel (no chunked one)
        return chunk == 16 || chunk == 64;
    if (chunk == 64)
        return dk == 32 || dk == 64 || dk == 128;
    if (chunk == 16)
        return dk == 32 || dk == 64;
    return false;
}

bool decode_supported(int32_t dk, int32_t dv, int32_t io_dtype)
{
    (void)io_dtype;
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

size_t prefill_slot_bytes(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype)
{
    // T and A (C x C io elements each), or W (dk x C) and M (C x C) in the absorbed form,
    // and the decay record exp(G), exp(G_last - G), beta, beta exp(G) (4 C floats)
    const size_t first = prefill_absorbed(io_dtype, chunk) ? (size_t)dk : (size_t)chunk;
    return (size_t)hv * ((first + (size_t)chunk) * (size_t)chunk * io_size(io_dtype) + 4 * (size_t)chunk * sizeof(float));
}

PrefillWorkspace prefill_workspace(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, int64_t total_tokens,
                                   int32_t num_seqs)
{
    PrefillWorkspace w{0, 0, 0};
    if (chunk <= 0 || total_tokens < 0 || num_seqs < 0 || hv <= 0)
        return w;
    const int64_t max_chunks = (total_tokens + chunk - 1) / chunk + num_seqs;
    if (max_chunks > INT32_MAX)
        return w;
    w.max_chunks = (int32_t)max_chunks;
    // chunk table (num_seqs + 1 entries), the scan order of the sequences (num_seqs), then
    // (8-byte aligned) the first token and length of every chunk slot
    w.table_bytes = (prefill_slot_info_offset(num_seqs) + (size_t)max_chunks * 2 * sizeof(int32_t) + 255) / 256 * 256;
    w.total_bytes = w.table_bytes + (size_t)max_chunks * prefill_slot_bytes(hv, dk, chunk, io_dtype);
    return w;
}

// Segments keep the chunk matrices plus the q and k rows of one segment (about
// kSegmentBytes) resident in the 256 MB last-level cache between the prep and the scan
// kernels.  A segment that would hold fewer than kMinSegmentChunks chunks per sequence
// (many sequences: every segment then re-reads and re-writes all their states, and runs
// its pairs in rounds of a few chunks) is not worth it: such batches take the single
// launch over the chunk table, whose scan runs every (sequence, head) chain to its end,
// longest first.
constexpr size_t kSegmentBytes = 176u << 20;
constexpr int64_t kMinSegmentChunks = 32;

int32_t prefill_segment_len(int32_t hqk, int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype,
                            int32_t num_seqs, int32_t max_seq_chunks, int32_t slot_capacity)
{
    if (num_seqs <= 0 || max_seq_chunks <= 0)
        return 0;
    const size_t es = io_size(io_dtype);
    const size_t first = prefill_absorbed(io_dtype, chunk) ? (size_t)dk : (size_t)chunk;
    const size_t per_slot = (size_t)hv * (first + chunk) * chunk * es + (size_t)chunk * 2 * hqk * dk * es;
    const int64_t m = (int64_t)(kSegmentBytes / per_slot) / num_seqs;
    if (m < kMinSegmentChunks && m < max_seq_chunks)
        return 0;
    // as few segments as the budget allows (one if the batch fits), of balanced length
    const int64_t nseg = m >= max_seq_chunks ? 1 : (max_seq_chunks + m - 1) / m;
    const int64_t len = (max_seq_chunks + nseg - 1) / nseg;
    // a segment takes num_seqs * len slots; the workspace holds ceil(T / C) + N
    if (len > slot_capacity / num_seqs)
        return 0;
    return (int32_t)len;
}

// Windows: a batch whose longest sequences take the row-split scan keeps, as segments do, the
// chunk matrices of one window resident in the last-level cache between the prep and the scans.
// Unlike segments, a window's chunk table gives slots only to the chunks that fall in it, so the
// short sequences (done in the first window) cost no slots in the later ones, and the whole-batch
// workspace holds every window.  The budget is the long ranks' slots: the first window also
// holds the short sequences' chunks.
int32_t prefill_window_len(int32_t hqk, int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, int32_t long_ranks,
                           int32_t max_seq_chunks)
{
    if (long_ranks <= 0 || max_seq_chunks <= 0)
        return 0;
    const size_t es = io_size(io_dtype);
    const size_t first = prefill_absorbed(io_dtype, chunk) ? (size_t)dk : (size_t)chunk;
    const size_t per_slot = (size_t)hv * (first + chunk) * chunk * es + (size_t)chunk * 2 * hqk * dk * es;
    const int64_t m = (int64_t)(kSegmentBytes / per_slot) / long_ranks;
    if (m >= max_seq_chunks || m < kMinSegmentChunks)
        return 0;
    const int64_t nwin = (max_seq_chunks + m - 1) / m;
    return (int32_t)((max_seq_chunks + nwin - 1) / nwin);
}

// A batch whose longest sequences would bound a whole-head scan (each of its workgroups runs
// one (sequence, head) chain, about 3 us per chunk step when its CU is to itself, about 4 us
// when the chip is busy) runs them in the row-split scan instead (about 1.2 us per step, eight
// workgroups per pair, so at most 256 / (8 HV) sequences in one round of the chip), then the
// rest in the whole-head scan.  The split is taken when its modelled time is under 80% of the
// single kernel's.
int32_t prefill_long_ranks(int32_t hv, int32_t dk, int32_t chunk, int32_t io_dtype, const int64_t *chunks_desc,
                           int32_t num_seqs)
{
    if (!prefill_absorbed(io_dtype, chunk) || dk != 128 || num_seqs < 2 || (int64_t)num_seqs * hv <= 64)
        return 0;
    constexpr double kRowStep = 1.2, kWholeChain = 3.0, kWholeBusy = 4.0, kCUs = 256.0;
    const int32_t kmax = std::min<int32_t>(num_seqs - 1, std::max<int32_t>(1, 256 / (8 * hv)));
    std::vector<double> tail(num_seqs + 1, 0.0);   // chunks of ranks >= r
    for (int32_t r = num_seqs - 1; r >= 0; --r)
        tail[r] = tail[r + 1] + (double)chunks_desc[r];
    auto whole = [&](int32_t r) {   // whole-head scan of ranks >= r
        return std::max(chunks_desc[r] * kWholeChain, tail[r] * hv * kWholeBusy / kCUs);
    };
    const double single = whole(0);
    int32_t best = 0;
    double best_t = 0.8 * single;
    for (int32_t k = 1; k <= kmax; ++k) {
        const double t = chunks_desc[0] * kRowStep + whole(k);
        if (t < best_t) {
            best_t = t;
            best = k;
        }
    }
    return best;
}

}  // namespace gdn

extern "C" {

size_t gdn_prefill_workspace_bytes(const gdn_shape *shape, int64_t total_tokens, int32_t num_seqs)
{
    if (check_shape(shape) != GDN_OK)
        return 0;
    if (!gdn::prefill_supported(shape->dk, shape->dv, shape->chunk, shape->io_dtype))
        return 0;
    return gdn::prefill_workspace(shape->num_v_heads, shape->dk, shape->chunk, shape->io_dtype, total_tokens,
                                  num_seqs)
        .total_bytes;
}

size_t gdn_prefill_workspace_bytes_for(const gdn_shape *shape, const int32_t *cu_seqlens_host, int32_t num_seqs)
{
    if (!cu_seqlens_host || num_seqs < 0 || check_shape(shape) != GDN_OK)
        return 0;
    const gdn_shape &s = *shape;
    if (!gdn::prefill_supported(s.dk, s.dv, s.chunk, s.io_dtype) || cu_seqlens_host[0] != 0)
        return 0;
    int64_t longest = 0;
    for (int32_t n = 0; n < num_seqs; ++n) {
        const int64_t len = (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n];
        if (len < 0)
            return 0;
        longest = std::max(longest, len);
    }
    const int64_t total = cu_seqlens_host[num_seqs];
    const gdn::PrefillWorkspace ws = gdn::prefill_workspace(s.num_v_heads, s.dk, s.chunk, s.io_dtype, total, num_seqs);
    if (ws.total_bytes == 0 || num_seqs == 0)
        return ws.total_bytes;
    // the plan gdn_prefill_chunked takes for these lengths with the whole-batch workspace:
    // segments use num_seqs * seg_len chunk slots, the single launch all of them
    const int32_t seg_len = gdn::prefill_segment_len(s.num_qk_heads, s.num_v_heads, s.dk, s.chunk, s.io_dtype,
                                                     num_seqs, (int32_t)((longest + s.chunk - 1) / s.chunk),
                                                     ws.max_chunks);
    if (seg_len <= 0)
        return ws.total_bytes;
    return ws.table_bytes +
           (size_t)num_seqs * seg_len * gdn::prefill_slot_bytes(s.num_v_heads, s.dk, s.chunk, s.io_dtype);
}

// The gated RMSNorm applied to the prefill's output rows (gdn_prefill_chunked_gated_rmsnorm).
struct NormIn {
    const void *z;
    const float *weight;
    float eps;
};

// own_scratch: the workspace is the library's own device scratch (gdn_prefill_chunked_noalloc),
// not an argument.
static gdn_status prefill_impl(const gdn_shape *shape, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                               const int32_t *cu_seqlens_host, const float *initial_state, float *final_state, void *o,
                               void *workspace, size_t workspace_bytes, void *stream, const NormIn *norm,
                               bool own_scratch = false)
{
    gdn_status st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape &s = *shape;
    if (!gdn::prefill_supported(s.dk, s.dv, s.chunk, s.io_dtype))
        return fail(GDN_ERR_UNSUPPORTED,
                    "no prefill kernel for dk=%d dv=%d chunk=%d io_dtype=%d (dk == dv in {32,64,128}, "
                    "chunk 64, or chunk 16 with dk <= 64 (fp32 io: also dk = 128))",
                    s.dk, s.dv, s.chunk, s.io_dtype);
    if (num_seqs < 0 || total_tokens < 0)
        return fail(GDN_ERR_INVALID_ARG, "negative num_seqs (%d) or total_tokens (%lld)", num_seqs,
                    (long long)total_tokens);
    if (num_seqs == 0) {
        if (total_tokens != 0)
            return fail(GDN_ERR_INVALID_ARG, "total_tokens=%lld with no sequences", (long long)total_tokens);
        return ok();
    }
    if ((int64_t)num_seqs * s.num_v_heads > INT32_MAX / 16)
        return fail(GDN_ERR_INVALID_ARG, "num_seqs * HV too large");
    if (!cu_seqlens || !final_state)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens and final_state are required");
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta and o are required when total_tokens > 0");
    if (norm) {
        if (total_tokens > 0 && (!norm->z || !norm->weight))
            return fail(GDN_ERR_INVALID_ARG, "z and the norm weight are required when total_tokens > 0");
        if (!aligned(norm->z, 16) || !aligned(norm->weight, 16))
            return fail(GDN_ERR_INVALID_ARG, "z and the norm weight must be 16-byte aligned");
        if (!std::isfinite(norm->eps) || norm->eps < 0.f)
            return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(final_state, 16) ||
        !aligned(initial_state, 16))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, o and state pointers must be 16-byte aligned");
    if (!aligned(g, 4) || !aligned(beta, 4) || !aligned(cu_seqlens, 4))
        return fail(GDN_ERR_INVALID_ARG, "g, beta and cu_seqlens must be 4-byte aligned");
    if (cu_seqlens_host) {
        if (cu_seqlens_host[0] != 0)
            return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu_seqlens_host[0]);
        for (int32_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
                return fail(GDN_ERR_INVALID_ARG, "cu_seqlens decreases at index %d", n + 1);
        if (cu_seqlens_host[num_seqs] != total_tokens)
            return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[%d] = %d but total_tokens = %lld", num_seqs,
                        cu_seqlens_host[num_seqs], (long long)total_tokens);
    }
    const gdn::PrefillWorkspace ws =
        gdn::prefill_workspace(s.num_v_heads, s.dk, s.chunk, s.io_dtype, total_tokens, num_seqs);
    if (ws.total_bytes == 0)
        return fail(GDN_ERR_INVALID_ARG, "batch too large for the chunk table");
    int32_t slot_capacity = ws.max_chunks;   // chunk slots the workspace holds
    bool must_segment = false;               // the workspace holds less than the whole batch
    const size_t avail = own_scratch ? gdn::kPrefillScratchBytes : (workspace ? workspace_bytes : 0);
    if (!own_scratch && !workspace)
        return fail(GDN_ERR_WORKSPACE, "workspace needs %zu bytes, got none", ws.total_bytes);
    if (ws.total_bytes > avail) {
        // Less than the whole batch: segments of the host-known sequence lengths sized to it.
        const char *what = own_scratch ? "the scratch of gdn_prefill_chunked_noalloc" : "the workspace";
        if (!cu_seqlens_host)
            return fail(GDN_ERR_WORKSPACE,
                        "the batch needs %zu bytes of chunk workspace and %s holds %zu; pass cu_seqlens_host "
                        "(the batch is then cut into segments that fit)",
                        ws.total_bytes, what, avail);
        const size_t slot_bytes = gdn::prefill_slot_bytes(s.num_v_heads, s.dk, s.chunk, s.io_dtype);
        const int64_t cap = ws.table_bytes < avail ? (int64_t)((avail - ws.table_bytes) / slot_bytes) : 0;
        if (cap < num_seqs)
            return fail(GDN_ERR_WORKSPACE,
                        "%d sequences need at least %zu bytes of chunk workspace (one chunk each); %s holds %zu",
                        num_seqs, ws.table_bytes + (size_t)num_seqs * slot_bytes, what, avail);
        slot_capacity = (int32_t)cap;
        must_segment = true;
    }
    if (own_scratch) {
        const hipError_t e = gdn::prefill_scratch(static_cast<hipStream_t>(stream), &workspace, &workspace_bytes);
        if (e != hipSuccess)
            return fail(GDN_ERR_HIP, "scratch of gdn_prefill_chunked_noalloc: %s", hipGetErrorString(e));
    }
    if (!aligned(workspace, 256))
        return fail(GDN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    const size_t es = io_size(s.io_dtype);
    const size_t qk_bytes = (size_t)total_tokens * s.num_qk_heads * s.dk * es;
    const size_t v_bytes = (size_t)total_tokens * s.num_v_heads * s.dv * es;
    const size_t gb_bytes = (size_t)total_tokens * s.num_v_heads * sizeof(float);
    const size_t state_bytes = (size_t)num_seqs * s.num_v_heads * s.dk * s.dv * sizeof(float);
    const void *inputs[] = {q, k, v, g, beta, initial_state, workspace, norm ? norm->z : nullptr,
                            norm ? norm->weight : nullptr};
    const size_t in_bytes[] = {qk_bytes, qk_bytes, v_bytes, gb_bytes, gb_bytes, state_bytes,
                               std::min(ws.total_bytes, workspace_bytes), v_bytes, (size_t)s.dv * sizeof(float)};
    for (int i = 0; i < 9; ++i) {
        if (overlaps(o, v_bytes, inputs[i], in_bytes[i]))
            return fail(GDN_ERR_INVALID_ARG, "o overlaps an input or the workspace");
        if (i != 5 && overlaps(final_state, state_bytes, inputs[i], in_bytes[i]))
            return fail(GDN_ERR_INVALID_ARG, "final_state overlaps an input or the workspace");
    }
    if (overlaps(o, v_bytes, final_state, state_bytes))
        return fail(GDN_ERR_INVALID_ARG, "o overlaps final_state");
    if (initial_state && initial_state != final_state && overlaps(final_state, state_bytes, initial_state, state_bytes))
        return fail(GDN_ERR_INVALID_ARG, "final_state partially overlaps initial_state (only exact aliasing is allowed)");

    gdn::PrefillArgs p{};
    p.hqk = s.num_qk_heads;
    p.hv = s.num_v_heads;
    p.dk = s.dk;
    p.dv = s.dv;
    p.chunk = s.chunk;
    p.io_dtype = s.io_dtype;
    p.scale = s.scale;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.cu_seqlens = cu_seqlens;
    p.num_seqs = num_seqs;
    p.total_tokens = total_tokens;
    p.initial_state = initial_state;
    p.final_state = final_state;
    p.o = o;
    p.workspace = workspace;
    p.max_chunks = slot_capacity;
    p.table_bytes = ws.table_bytes;
    p.seg_len = 0;
    p.max_seq_chunks = 0;
    p.max_len = -1;
    p.win_len = 0;
    p.win_slots = nullptr;
    p.rest_chunks = -1;
    std::vector<int64_t> win_slots;   // chunk slots of each window (host offsets, windows only)
    if (cu_seqlens_host) {
        int64_t longest = 0, prev_chunks = INT64_MAX;
        p.ordered = true;
        for (int32_t n = 0; n < num_seqs; ++n) {
            const int64_t len = cu_seqlens_host[n + 1] - cu_seqlens_host[n];
            const int64_t chunks = (len + s.chunk - 1) / s.chunk;
            longest = std::max<int64_t>(longest, len);
            p.ordered = p.ordered && chunks <= prev_chunks;
            prev_chunks = chunks;
        }
        p.max_seq_chunks = (int32_t)((longest + s.chunk - 1) / s.chunk);
        p.max_len = (int32_t)longest;
        {
            std::vector<int64_t> chunks(num_seqs);
            for (int32_t n = 0; n < num_seqs; ++n)
                chunks[n] = (cu_seqlens_host[n + 1] - cu_seqlens_host[n] + s.chunk - 1) / s.chunk;
            std::sort(chunks.begin(), chunks.end(), std::greater<int64_t>());
            p.long_ranks = gdn::prefill_long_ranks(s.num_v_heads, s.dk, s.chunk, s.io_dtype, chunks.data(), num_seqs);
            if (p.long_ranks > 0)
                p.rest_chunks = (int32_t)chunks[p.long_ranks];
        }
        p.seg_len = gdn::prefill_segment_len(s.num_qk_heads, s.num_v_heads, s.dk, s.chunk, s.io_dtype, num_seqs,
                                             p.max_seq_chunks, slot_capacity);
        if (must_segment && p.seg_len == 0 && p.max_seq_chunks > 0) {
            // the workspace holds less than the batch: segments as long as it allows, balanced
            const int64_t m = slot_capacity / num_seqs;   // >= 1 (checked above)
            const int64_t nseg = (p.max_seq_chunks + m - 1) / m;
            p.seg_len = (int32_t)((p.max_seq_chunks + nseg - 1) / nseg);
        }
        if (p.seg_len == 0 && p.long_ranks > 0) {
            p.win_len = gdn::prefill_window_len(s.num_qk_heads, s.num_v_heads, s.dk, s.chunk, s.io_dtype,
                                                p.long_ranks, p.max_seq_chunks);
            if (p.win_len > 0) {
                // window j holds local chunks [j L, (j + 1) L) of every sequence
                const int64_t L = p.win_len;
                win_slots.assign((p.max_seq_chunks + L - 1) / L, 0);
                for (int32_t n = 0; n < num_seqs; ++n) {
                    const int64_t c = ((int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n] + s.chunk - 1) / s.chunk;
                    for (size_t j = 0; (int64_t)j * L < c; ++j)
                        win_slots[j] += std::min<int64_t>(L, c - (int64_t)j * L);
                }
                p.win_slots = win_slots.data();
            }
        }
        if (p.max_seq_chunks == 0) {   // every sequence empty: one launch passes the states through
            p.seg_len = 1;
            p.max_seq_chunks = 1;
        }
    }
    if (norm) {
        p.norm_z = norm->z;
        p.norm_weight = norm->weight;
        p.norm_eps = norm->eps;
    }
    p.stream = stream;
    const hipError_t err = gdn::launch_prefill(p);
    if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(err));
    return ok();
}

gdn_status gdn_prefill_chunked(const gdn_shape *shape, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const int32_t *cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, const int32_t *cu_seqlens_host, const float *initial_state,
                               float *final_state, void *o, void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_impl(shape, q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, cu_seqlens_host, initial_state,
                        final_state, o, workspace, workspace_bytes, stream, nullptr);
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_shape *shape, const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, const int32_t *cu_seqlens, int32_t num_seqs,
                                       int64_t total_tokens, const int32_t *cu_seqlens_host, const float *initial_state,
                                       float *final_state, void *o, void *stream)
{
    return prefill_impl(shape, q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, cu_seqlens_host, initial_state,
                        final_state, o, nullptr, 0, stream, nullptr, true);
}

gdn_status gdn_prefill_chunked_gated_rmsnorm(const gdn_shape *shape, const void *q, const void *k, const void *v,
                                             const float *g, const float *beta, const int32_t *cu_seqlens,
                                             int32_t num_seqs, int64_t total_tokens, const int32_t *cu_seqlens_host,
                                             const float *initial_state, float *final_state, const void *z,
                                             const float *norm_weight, float eps, void *y, void *workspace,
                                             size_t workspace_bytes, void *stream)
{
    const NormIn norm{z, norm_weight, eps};
    return prefill_impl(shape, q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, cu_seqlens_host, initial_state,
                        final_state, y, workspace, workspace_bytes, stream, &norm);
}

gdn_status gdn_decode_step(const gdn_shape *shape, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, int32_t num_seqs, void *stream)
{
    gdn_status st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape &s = *shape;
    if (!gdn::decode_supported(s.dk, s.dv, s.io_dtype))
        return fail(GDN_ERR_UNSUPPORTED, "no decode kernel for dk=%d dv=%d (dk == dv in {32,64,128})", s.dk, s.dv);
    if (num_seqs < 0)
        return fail(GDN_ERR_INVALID_ARG, "negative num_seqs");
    if (num_seqs == 0)
        return ok();
    if ((int64_t)num_seqs * s.num_v_heads > (int64_t(1) << 24))
        return fail(GDN_ERR_INVALID_ARG, "num_seqs * HV too large (at most 2^24 states per call)");
    if (!q || !k || !v || !g || !beta || !state || !o)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta, state and o are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state, 16))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, o and state must be 16-byte aligned");
    if (!aligned(g, 4) || !aligned(beta, 4))
        return fail(GDN_ERR_INVALID_ARG, "g and beta must be 4-byte aligned");
    const size_t es = io_size(s.io_dtype);
    const size_t state_bytes = (size_t)num_seqs * s.num_v_heads * s.dk * s.dv * sizeof(float);
    const size_t o_bytes = (size_t)num_seqs * s.num_v_heads * s.dv * es;
    const size_t qk_bytes = (size_t)num_seqs * s.num_qk_heads * s.dk * es;
    const size_t gb_bytes = (size_t)num_seqs * s.num_v_heads * sizeof(float);
    const void *others[] = {q, k, v, g, beta};
    const size_t ob[] = {qk_bytes, qk_bytes, o_bytes, gb_bytes, gb_bytes};
    for (int i = 0; i < 5; ++i)
        if (overlaps(state, state_bytes, others[i], ob[i]) || overlaps(o, o_bytes, others[i], ob[i]))
            return fail(GDN_ERR_INVALID_ARG, "state or o overlaps an input");
    if (overlaps(o, o_bytes, state, state_bytes))
        return fail(GDN_ERR_INVALID_ARG, "o overlaps the state");

    gdn::DecodeArgs p{};
    p.hqk = s.num_qk_heads;
    p.hv = s.num_v_heads;
    p.dk = s.dk;
    p.dv = s.dv;
    p.io_dtype = s.io_dtype;
    p.scale = s.scale;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.state = state;
    p.o = o;
    p.num_seqs = num_seqs;
    p.stream = stream;
    const hipError_t err = gdn::launch_decode(p);
    if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "decode launch failed: %s", hipGetErrorString(err));
    return ok();
}

gdn_status gdn_conv1d_qkv(const gdn_shape *shape, const void *x, const float *weight, int32_t width,
                          const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, const float *state_in,
                          float *state_out, int32_t silu, int32_t l2norm, float eps, void *q, void *k, void *v,
                          void *stream)
{
    gdn_status st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape &s = *shape;
    if ((s.dk != 32 && s.dk != 64 && s.dk != 128) || (s.dv != 32 && s.dv != 64 && s.dv != 128))
        return fail(GDN_ERR_UNSUPPORTED, "no conv kernel for dk=%d dv=%d (each in {32,64,128})", s.dk, s.dv);
    if (width < 1 || width > 8)
        return fail(GDN_ERR_UNSUPPORTED, "conv width %d not in 1..8", width);
    if (num_seqs < 0 || total_tokens < 0)
        return fail(GDN_ERR_INVALID_ARG, "negative num_seqs or total_tokens");
    if (num_seqs == 0) {
        if (total_tokens != 0)
            return fail(GDN_ERR_INVALID_ARG, "tokens without sequences");
        return ok();
    }
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const int64_t channels = 2 * (int64_t)s.num_qk_heads * s.dk + (int64_t)s.num_v_heads * s.dv;
    if (channels > (int64_t(1) << 24) || total_tokens > (int64_t(1) << 31))
        return fail(GDN_ERR_INVALID_ARG, "too many channels or tokens");
    const int64_t waves_per_token = (channels + 64 * (16 / (int64_t)io_size(s.io_dtype)) - 1) /
                                    (64 * (16 / (int64_t)io_size(s.io_dtype)));
    if (total_tokens * waves_per_token > (int64_t(1) << 33))
        return fail(GDN_ERR_INVALID_ARG, "total_tokens * C too large for one launch");
    if (!cu_seqlens || !weight || (total_tokens > 0 && (!x || !q || !k || !v)))
        return fail(GDN_ERR_INVALID_ARG, "x, weight, cu_seqlens, q, k and v are required");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(weight, 16))
        return fail(GDN_ERR_INVALID_ARG, "x, weight, q, k and v must be 16-byte aligned");
    if (!aligned(cu_seqlens, 4) || !aligned(state_in, 4) || !aligned(state_out, 4))
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens and the states must be 4-byte aligned");
    const size_t es = io_size(s.io_dtype);
    const size_t x_bytes = (size_t)total_tokens * channels * es;
    const size_t qk_bytes = (size_t)total_tokens * s.num_qk_heads * s.dk * es;
    const size_t v_bytes = (size_t)total_tokens * s.num_v_heads * s.dv * es;
    const size_t st_bytes = (size_t)num_seqs * channels * (width - 1) * sizeof(float);
    const void *outs[] = {q, k, v};
    const size_t ob[] = {qk_bytes, qk_bytes, v_bytes};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], ob[i], x, x_bytes) || overlaps(outs[i], ob[i], weight, (size_t)channels * width * 4) ||
            overlaps(outs[i], ob[i], state_in, st_bytes) || overlaps(outs[i], ob[i], state_out, st_bytes))
            return fail(GDN_ERR_INVALID_ARG, "q, k or v overlaps an input or a state");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], ob[i], outs[j], ob[j]))
                return fail(GDN_ERR_INVALID_ARG, "q, k and v overlap each other");
    }
    if (state_out && state_out != state_in && overlaps(state_out, st_bytes, state_in, st_bytes))
        return fail(GDN_ERR_INVALID_ARG, "state_out partially overlaps state_in");
    if (overlaps(state_out, st_bytes, x, x_bytes) || overlaps(state_out, st_bytes, weight, (size_t)channels * width * 4))
        return fail(GDN_ERR_INVALID_ARG, "state_out overlaps x or the weight");

    gdn::ConvArgs p{};
    p.dk = s.dk;
    p.io_dtype = s.io_dtype;
    p.width = width;
    p.channels = (int32_t)channels;
    p.nq = s.num_qk_heads * s.dk;
    p.x = x;
    p.weight = weight;
    p.cu_seqlens = cu_seqlens;
    p.num_seqs = num_seqs;
    p.tokens = total_tokens;
    p.state_in = state_in;
    p.state_out = width > 1 ? state_out : nullptr;
    p.silu = silu ? 1 : 0;
    p.l2norm = l2norm ? 1 : 0;
    p.eps = eps;
    p.q = q;
    p.k = k;
    p.v = v;
    p.stream = stream;
    const hipError_t err = gdn::launch_conv(p);
    if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "conv launch failed: %s", hipGetErrorString(err));
    return ok();
}

gdn_status gdn_gated_rmsnorm(const gdn_shape *shape, const void *o, const void *z, const float *weight, void *y,
                             int64_t tokens, float eps, void *stream)
{
    gdn_status st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape &s = *shape;
    if (s.dv != 32 && s.dv != 64 && s.dv != 128)
        return fail(GDN_ERR_UNSUPPORTED, "no gated RMSNorm kernel for dv=%d (dv in {32,64,128})", s.dv);
    if (tokens < 0)
        return fail(GDN_ERR_INVALID_ARG, "negative token count");
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (tokens == 0)
        return ok();
    if (tokens > (int64_t(1) << 32) / s.num_v_heads)
        return fail(GDN_ERR_INVALID_ARG, "tokens * HV too large (at most 2^32 rows per call)");
    if (!o || !z || !weight || !y)
        return fail(GDN_ERR_INVALID_ARG, "o, z, weight and y are required");
    if (!aligned(o, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(weight, 16))
        return fail(GDN_ERR_INVALID_ARG, "o, z, y and weight must be 16-byte aligned");
    const size_t bytes = (size_t)tokens * s.num_v_heads * s.dv * io_size(s.io_dtype);
    // y may be o or z exactly (in place), but no buffer may overlap another partially
    if ((y != o && overlaps(y, bytes, o, bytes)) || (y != z && overlaps(y, bytes, z, bytes)))
        return fail(GDN_ERR_INVALID_ARG, "y partially overlaps o or z");
    if (overlaps(y, bytes, weight, (size_t)s.dv * sizeof(float)))
        return fail(GDN_ERR_INVALID_ARG, "y overlaps the weight");

    gdn::NormArgs p{};
    p.hv = s.num_v_heads;
    p.dv = s.dv;
    p.io_dtype = s.io_dtype;
    p.o = o;
    p.z = z;
    p.weight = weight;
    p.y = y;
    p.tokens = tokens;
    p.eps = eps;
    p.stream = stream;
    const hipError_t err = gdn::launch_norm(p);
    if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "gated RMSNorm launch failed: %s", hipGetErrorString(err));
    return ok();
}

// Gather/scatter of whole rows of row_floats fp32 values (the checks and the launch shared by
// the recurrent-state and the conv-state snapshots).
static gdn_status snapshot_rows(int64_t row_floats, const float *src, const int32_t *src_rows, int32_t src_capacity,
                                float *dst, const int32_t *dst_rows, int32_t dst_capacity, int32_t num_rows,
                                void *stream)
{
    if (num_rows < 0 || src_capacity < 0 || dst_capacity < 0)
        return fail(GDN_ERR_INVALID_ARG, "negative row count or capacity");
    if (num_rows == 0 || row_floats == 0)
        return ok();
    if (!src || !dst)
        return fail(GDN_ERR_INVALID_ARG, "src and dst are required");
    if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(src_rows, 4) || !aligned(dst_rows, 4))
        return fail(GDN_ERR_INVALID_ARG, "src/dst must be 16-byte aligned, row indices 4-byte aligned");
    if (row_floats % 4 != 0)
        return fail(GDN_ERR_UNSUPPORTED, "a row of %lld floats is not a whole number of 16-byte vectors",
                    (long long)row_floats);
    if (!src_rows && num_rows > src_capacity)
        return fail(GDN_ERR_INVALID_ARG, "num_rows=%d exceeds src_capacity=%d", num_rows, src_capacity);
    if (!dst_rows && num_rows > dst_capacity)
        return fail(GDN_ERR_INVALID_ARG, "num_rows=%d exceeds dst_capacity=%d", num_rows, dst_capacity);
    if (overlaps(src, (size_t)src_capacity * row_floats * 4, dst, (size_t)dst_capacity * row_floats * 4))
        return fail(GDN_ERR_INVALID_ARG, "src and dst overlap");

    gdn::SnapshotArgs p{};
    p.src = src;
    p.src_rows = src_rows;
    p.src_capacity = src_capacity;
    p.dst = dst;
    p.dst_rows = dst_rows;
    p.dst_capacity = dst_capacity;
    p.num_rows = num_rows;
    p.row_floats = row_floats;
    p.stream = stream;
    const hipError_t err = gdn::launch_snapshot(p);
    if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "snapshot launch failed: %s", hipGetErrorString(err));
    return ok();
}

gdn_status gdn_state_snapshot(const gdn_shape *shape, const float *src, const int32_t *src_rows,
                              int32_t src_capacity, float *dst, const int32_t *dst_rows, int32_t dst_capacity,
                              int32_t num_rows, void *stream)
{
    gdn_status st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const int64_t row_floats = (int64_t)shape->num_v_heads * shape->dk * shape->dv;
    return snapshot_rows(row_floats, src, src_rows, src_capacity, dst, dst_rows, dst_capacity, num_rows, stream);
}

gdn_status gdn_conv_state_snapshot(int64_t channels, int32_t width, const float *src, const int32_t *src_rows,
                                   int32_t src_capacity, float *dst, const int32_t *dst_rows, int32_t dst_capacity,
                                   int32_t num_rows, void *stream)
{
    if (channels <= 0 || channels > (int64_t)1 << 24)
        return fail(GDN_ERR_INVALID_ARG, "channels=%lld not in 1..2^24", (long long)channels);
    if (width < 1 || width > 8)
        return fail(GDN_ERR_UNSUPPORTED, "conv width %d not in 1..8", width);
    return snapshot_rows(channels * (width - 1), src, src_rows, src_capacity, dst, dst_rows, dst_capacity, num_rows,
                         stream);
}

const char *gdn_status_string(gdn_status status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    }
    return "GDN_ERR_UNKNOWN";
}

const char *gdn_last_error(void) { return g_last_error; }

int32_t gdn_version(void) { return 100; }

}  // extern "C"
