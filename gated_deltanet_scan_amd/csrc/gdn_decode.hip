// gdn_decode.hip -- one-token decode step and state snapshot copies (gfx950).
//
// Decode follows the one-token matrix form on the NPU page ("Qwen3.5-9B --
// every component on the Intel NPU", section "How it works"): S^T k and
// S^T q come out of one pass over the state, then with d = exp(g) and
// delta = beta (v - d S^T k):
//     o  = scale (d S^T q + (q.k) delta)
//     S' = d S + k delta^T
// so the state is read once and written once (the step is a pure stream of
// the dk x dv fp32 state: 0.875 flop per byte at dk = dv = 128).
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

namespace gdn {

// Each wave owns one 32-column slice of one (sequence, value head) state, all
// dk rows: lane (rg, cg) = (lane / 8, lane % 8) holds columns 4 cg .. 4 cg + 3
// of the RPL consecutive rows rg * RPL .. rg * RPL + RPL - 1.  Every load and
// store instruction of the wave covers 8 whole 128-byte row segments.  The
// sums over dk are a register sum over the lane's rows followed by a
// butterfly over the 8 row groups (fixed order: deterministic).  Waves never
// wait for each other: no LDS and no barrier.
constexpr int kDecodeCols = 32;

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    E *__restrict__ o, int32_t hqk, int32_t hv, int64_t waves, float scale)
{
    constexpr int NS = D / kDecodeCols;   // column slices per state
    constexpr int RG = 8;                 // row groups per wave
    constexpr int RPL = D / RG;           // rows per lane
    constexpr int VN = 16 / (int)sizeof(E);
    static_assert(D % kDecodeCols == 0, "lane layout");
    typedef typename Vec16<E>::type V16;

    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    if (w >= waves)
        return;
    const int64_t pair = w / NS;            // n * hv + h
    const int slice = (int)(w - pair * NS);
    const int n = (int)(pair / hv), h = (int)(pair - (int64_t)n * hv);
    const int hq = h / (hv / hqk);
    const int rg = lane / 8, cg = lane % 8;
    const int col = slice * kDecodeCols + 4 * cg;
    float *S = state + (size_t)pair * D * D + (size_t)(rg * RPL) * D + col;

    // the state: ordinary loads, non-temporal stores (measured at decode_64: 44.7 us per launch;
    // 47.0 with non-temporal loads as well, 52.4 with neither)
    f32x4 s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        s[i] = *reinterpret_cast<const f32x4 *>(S + (size_t)i * D);

    // this lane's rows of k and q
    float kr[RPL], qr[RPL];
    const E *kp = k + ((size_t)n * hqk + hq) * D + rg * RPL;
    const E *qp = q + ((size_t)n * hqk + hq) * D + rg * RPL;
    if constexpr (RPL % VN == 0) {
#pragma unroll
        for (int c = 0; c < RPL / VN; ++c) {
            const V16 kv = *reinterpret_cast<const V16 *>(kp + c * VN);
            const V16 qv = *reinterpret_cast<const V16 *>(qp + c * VN);
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                kr[c * VN + e] = to_f32(kv[e]);
                qr[c * VN + e] = to_f32(qv[e]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            kr[i] = to_f32(kp[i]);
            qr[i] = to_f32(qp[i]);
        }
    }
    const float alpha = expf(g[pair]);
    const float bt = beta[pair];
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        vv[e] = to_f32(v[(size_t)pair * D + col + e]);

    f32x4 a4 = zero4(), b4 = zero4();
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        a4 += kr[i] * s[i];
        b4 += qr[i] * s[i];
        qk += qr[i] * kr[i];
    }
    // butterfly over the row groups (lane bits 3..5)
#pragma unroll
    for (int m = 8; m < kWave; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a4[e] += __shfl_xor(a4[e], m, kWave);
            b4[e] += __shfl_xor(b4[e], m, kWave);
        }
        qk += __shfl_xor(qk, m, kWave);
    }
    f32x4 d4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        d4[e] = bt * (vv[e] - alpha * a4[e]);
    if (rg == 0) {
        E *op = o + (size_t)pair * D + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            op[e] = (E)(scale * (alpha * b4[e] + qk * d4[e]));
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        __builtin_nontemporal_store(alpha * s[i] + kr[i] * d4, reinterpret_cast<f32x4 *>(S + (size_t)i * D));
}

template <typename E, int D>
static hipError_t launch_decode_t(const DecodeArgs &p)
{
    const int64_t waves = (int64_t)p.num_seqs * p.hv * (D / kDecodeCols);
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    if (blocks > 0) {
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        const ProfEvents ev = prof_events(PROF_DECODE);
        hipExtLaunchKernelGGL((gdn_decode_kernel<E, D>), dim3((unsigned)blocks), dim3(kThreads), 0, st, ev.start,
                              ev.stop, 0, static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                              static_cast<const E *>(p.v), p.g, p.beta, p.state, static_cast<E *>(p.o), p.hqk, p.hv,
                              waves, p.scale);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &p)
{
    const bool bf = p.io_dtype == 1;
    switch (p.dk) {
    case 32: return bf ? launch_decode_t<bf16, 32>(p) : launch_decode_t<float, 32>(p);
    case 64: return bf ? launch_decode_t<bf16, 64>(p) : launch_decode_t<float, 64>(p);
    case 128: return bf ? launch_decode_t<bf16, 128>(p) : launch_decode_t<float, 128>(p);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Prefill of a batch of short sequences (each at most kShortPrefillTokens tokens): the
// one-token step above, token by token, with the state slices held in registers for the
// whole sequence.  This is the recurrence of the NPU page's per-token loop (section "How
// it works") rather than its chunkwise form: for a sequence shorter than one chunk the
// chunkwise form's per-chunk matrices cost a second launch (the prep) and a chunk step of
// work for a handful of tokens, while here the state is read once and written once and the
// batch is one launch.
//
// One workgroup per (sequence, value head), one wave per 32-column slice as in the decode
// kernel.  The sequence's k and q rows (of its query/key head), its v rows, g and beta are
// staged in LDS kShortPrefillTokens tokens at a time (16-byte loads spread over the
// workgroup); the token loop then reads only LDS and registers.  Sequences longer than one
// block (fp32 io at dk = 128, which has no chunked kernel, takes this path at any length)
// run block after block with the state kept in registers.  Sequence bounds are clamped to
// [0, total_tokens], so inconsistent offsets cannot send an access out of bounds.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(D / kDecodeCols * kWave) void gdn_short_prefill_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, int64_t total_tokens,
    const float *state_in, float *state_out, E *__restrict__ o, int32_t hqk, int32_t hv, float scale)
{
    constexpr int NS = D / kDecodeCols;   // waves: column slices per state
    constexpr int NT = NS * kWave;
    constexpr int RG = 8;                 // row groups per wave
    constexpr int RPL = D / RG;           // rows per lane
    constexpr int L = kShortPrefillTokens;
    constexpr int VN = Vec16<E>::n;
    constexpr int VPR = D / VN;           // 16-byte vectors per row
    typedef typename Vec16<E>::type V16;
    static_assert(D % kDecodeCols == 0 && D % VN == 0, "lane layout");

    __shared__ __attribute__((aligned(16))) E ks[L][D];
    __shared__ __attribute__((aligned(16))) E qs[L][D];
    __shared__ __attribute__((aligned(16))) E vs[L][D];
    __shared__ float gs[L], bs[L];

    const int pair = blockIdx.x;   // n * hv + h
    const int n = pair / hv, h = pair - n * hv;
    const int hq = h / (hv / hqk);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t a0 = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
    const int64_t b = min<int64_t>(max<int64_t>(cu[n + 1], a0), total_tokens);

    // lane (rg, cg): columns col .. col + 3 of rows rg * RPL .. rg * RPL + RPL - 1
    const int rg = lane / 8, cg = lane % 8;
    const int col = wave * kDecodeCols + 4 * cg;
    const size_t sbase = (size_t)pair * D * D + (size_t)(rg * RPL) * D + col;
    f32x4 s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        s[i] = state_in ? *reinterpret_cast<const f32x4 *>(state_in + sbase + (size_t)i * D) : zero4();

    for (int64_t a = a0; a < b; a += L) {
    const int len = (int)min<int64_t>(b - a, L);
    if (a != a0)
        __syncthreads();   // every wave is done with the previous block's staged tokens
    for (int i = tid; i < len * VPR; i += NT) {
        const int t = i / VPR, c = (i - t * VPR) * VN;
        const size_t tok = (size_t)(a + t);
        *reinterpret_cast<V16 *>(&ks[t][c]) = *reinterpret_cast<const V16 *>(k + (tok * hqk + hq) * D + c);
        *reinterpret_cast<V16 *>(&qs[t][c]) = *reinterpret_cast<const V16 *>(q + (tok * hqk + hq) * D + c);
        *reinterpret_cast<V16 *>(&vs[t][c]) = *reinterpret_cast<const V16 *>(v + (tok * hv + h) * D + c);
    }
    for (int t = tid; t < len; t += NT) {
        gs[t] = g[(size_t)(a + t) * hv + h];
        bs[t] = beta[(size_t)(a + t) * hv + h];
    }
    __syncthreads();

    for (int t = 0; t < len; ++t) {
        float kr[RPL], qr[RPL];
        if constexpr (RPL % VN == 0) {
#pragma unroll
            for (int c = 0; c < RPL / VN; ++c) {
                const V16 kv = *reinterpret_cast<const V16 *>(&ks[t][rg * RPL + c * VN]);
                const V16 qv = *reinterpret_cast<const V16 *>(&qs[t][rg * RPL + c * VN]);
#pragma unroll
                for (int e = 0; e < VN; ++e) {
                    kr[c * VN + e] = to_f32(kv[e]);
                    qr[c * VN + e] = to_f32(qv[e]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                kr[i] = to_f32(ks[t][rg * RPL + i]);
                qr[i] = to_f32(qs[t][rg * RPL + i]);
            }
        }
        const float alpha = expf(gs[t]);
        const float bt = bs[t];
        float vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vv[e] = to_f32(vs[t][col + e]);

        f32x4 a4 = zero4(), b4 = zero4();
        float qk = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            a4 += kr[i] * s[i];
            b4 += qr[i] * s[i];
            qk += qr[i] * kr[i];
        }
#pragma unroll
        for (int m = 8; m < kWave; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a4[e] += __shfl_xor(a4[e], m, kWave);
                b4[e] += __shfl_xor(b4[e], m, kWave);
            }
            qk += __shfl_xor(qk, m, kWave);
        }
        f32x4 d4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d4[e] = bt * (vv[e] - alpha * a4[e]);
        if (rg == 0) {
            E *op = o + ((size_t)(a + t) * hv + h) * D + col;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                op[e] = (E)(scale * (alpha * b4[e] + qk * d4[e]));
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            s[i] = alpha * s[i] + kr[i] * d4;
    }
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        *reinterpret_cast<f32x4 *>(state_out + sbase + (size_t)i * D) = s[i];
}

template <typename E, int D>
static hipError_t launch_short_prefill_t(const PrefillArgs &p)
{
    const int64_t blocks = (int64_t)p.num_seqs * p.hv;
    if (blocks > 0) {
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        const ProfEvents ev = prof_events(PROF_SHORT);
        hipExtLaunchKernelGGL((gdn_short_prefill_kernel<E, D>), dim3((unsigned)blocks),
                              dim3(D / kDecodeCols * kWave), 0, st, ev.start, ev.stop, 0,
                              static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                              static_cast<const E *>(p.v), p.g, p.beta, p.cu_seqlens, p.total_tokens,
                              p.initial_state, p.final_state, static_cast<E *>(p.o), p.hqk, p.hv, p.scale);
    }
    return hipGetLastError();
}

bool short_prefill_supported(int32_t dk, int32_t dv)
{
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_short_prefill(const PrefillArgs &p)
{
    const bool bf = p.io_dtype == 1;
    switch (p.dk) {
    case 32: return bf ? launch_short_prefill_t<bf16, 32>(p) : launch_short_prefill_t<float, 32>(p);
    case 64: return bf ? launch_short_prefill_t<bf16, 64>(p) : launch_short_prefill_t<float, 64>(p);
    case 128: return bf ? launch_short_prefill_t<bf16, 128>(p) : launch_short_prefill_t<float, 128>(p);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Snapshot: dst[dst_rows[i]] = src[src_rows[i]] for whole per-sequence states.
// Grid (num_rows, parts of 2048 16-byte vectors).  Out-of-range row indices
// are skipped so that device index arrays can never send a copy out of
// bounds.
// ---------------------------------------------------------------------------
// 16-byte vectors per thread, all loaded before any is stored: 16 (256 bytes in flight per
// thread) copies the 32 MB of a 16-sequence, 32-head batch in 11.3 us; 8: 17.4 us; 32: 12.8 us.
constexpr int kSnapVecsPerThread = 16;

__global__ __launch_bounds__(kThreads) void gdn_snapshot_kernel(
    const float *__restrict__ src, const int32_t *__restrict__ src_rows, int32_t src_cap,
    float *__restrict__ dst, const int32_t *__restrict__ dst_rows, int32_t dst_cap, int64_t row_vec4)
{
    const int32_t i = blockIdx.x;
    const int32_t sr = src_rows ? src_rows[i] : i;
    const int32_t dr = dst_rows ? dst_rows[i] : i;
    if (sr < 0 || sr >= src_cap || dr < 0 || dr >= dst_cap)
        return;
    const f32x4 *s = reinterpret_cast<const f32x4 *>(src + (size_t)sr * row_vec4 * 4);
    f32x4 *d = reinterpret_cast<f32x4 *>(dst + (size_t)dr * row_vec4 * 4);
    const int64_t base = (int64_t)blockIdx.y * kThreads * kSnapVecsPerThread + threadIdx.x;
    f32x4 buf[kSnapVecsPerThread];
#pragma unroll
    for (int u = 0; u < kSnapVecsPerThread; ++u) {
        const int64_t j = base + (int64_t)u * kThreads;
        if (j < row_vec4)
            buf[u] = s[j];
    }
#pragma unroll
    for (int u = 0; u < kSnapVecsPerThread; ++u) {
        const int64_t j = base + (int64_t)u * kThreads;
        if (j < row_vec4)
            d[j] = buf[u];
    }
}

hipError_t launch_snapshot(const SnapshotArgs &p)
{
    const int64_t row_vec4 = p.row_floats / 4;
    const int64_t per_block = (int64_t)kThreads * kSnapVecsPerThread;
    const int64_t parts = (row_vec4 + per_block - 1) / per_block;
    if (p.num_rows > 0 && parts > 0) {
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        const ProfEvents ev = prof_events(PROF_SNAPSHOT);
        hipExtLaunchKernelGGL(gdn_snapshot_kernel, dim3((unsigned)p.num_rows, (unsigned)parts), dim3(kThreads), 0,
                              st, ev.start, ev.stop, 0, p.src, p.src_rows, p.src_capacity, p.dst, p.dst_rows,
                              p.dst_capacity, row_vec4);
    }
    return hipGetLastError();
}

}  // namespace gdn
