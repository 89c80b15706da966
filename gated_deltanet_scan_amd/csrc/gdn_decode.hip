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

// One workgroup per (sequence, value head).  Thread t owns 4 consecutive
// columns (one 16-byte vector per row, lanes along dv so every row is read
// and written as whole coalesced segments) of RPT rows spaced RG apart; the
// reductions over dk go through LDS in a fixed order (deterministic).
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    E *__restrict__ o, int32_t hqk, int32_t hv, float scale)
{
    constexpr int C4 = D / 4;           // 16-byte column groups per row
    constexpr int RG = kThreads / C4;   // row groups
    constexpr int RPT = D / RG;         // rows per thread
    static_assert(RG * C4 == kThreads && RPT * RG == D, "thread layout");

    __shared__ float qs[D], ks[D];
    __shared__ __attribute__((aligned(16))) float pa[RG * D];
    __shared__ __attribute__((aligned(16))) float pb[RG * D];
    __shared__ __attribute__((aligned(16))) float dl[D];
    __shared__ float qk_s;

    const int pair = blockIdx.x;  // n * hv + h
    const int n = pair / hv, h = pair - (pair / hv) * hv;
    const int hq = h / (hv / hqk);
    const int tid = threadIdx.x, cg = tid % C4, rg = tid / C4;
    float *S = state + (size_t)pair * D * D;

    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *reinterpret_cast<const f32x4 *>(S + (size_t)(rg + RG * i) * D + 4 * cg);
    if (tid < D) {
        qs[tid] = to_f32(q[((size_t)n * hqk + hq) * D + tid]);
        ks[tid] = to_f32(k[((size_t)n * hqk + hq) * D + tid]);
    }
    const float alpha = expf(g[pair]);
    const float bt = beta[pair];
    __syncthreads();

    f32x4 pa4 = zero4(), pb4 = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        pa4 += ks[r] * s[i];
        pb4 += qs[r] * s[i];
    }
    *reinterpret_cast<f32x4 *>(pa + rg * D + 4 * cg) = pa4;
    *reinterpret_cast<f32x4 *>(pb + rg * D + 4 * cg) = pb4;
    if (tid < kWave) {
        float x = 0.f;
        for (int i = tid; i < D; i += kWave)
            x += qs[i] * ks[i];
        x = wave_sum(x);
        if (tid == 0)
            qk_s = x;
    }
    __syncthreads();

    if (tid < D) {
        float A = 0.f, B = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            A += pa[r * D + tid];
            B += pb[r * D + tid];
        }
        const float d = bt * (to_f32(v[(size_t)pair * D + tid]) - alpha * A);
        dl[tid] = d;
        o[(size_t)pair * D + tid] = (E)(scale * (alpha * B + qk_s * d));
    }
    __syncthreads();

    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dl + 4 * cg);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        *reinterpret_cast<f32x4 *>(S + (size_t)r * D + 4 * cg) = alpha * s[i] + ks[r] * d4;
    }
}

template <typename E, int D>
static hipError_t launch_decode_t(const DecodeArgs &p)
{
    const int64_t blocks = (int64_t)p.num_seqs * p.hv;
    if (blocks > 0) {
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        prof_begin(PROF_DECODE, st);
        hipLaunchKernelGGL((gdn_decode_kernel<E, D>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                           static_cast<const E *>(p.v), p.g, p.beta, p.state, static_cast<E *>(p.o), p.hqk,
                           p.hv, p.scale);
        prof_end(st);
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
// Snapshot: dst[dst_rows[i]] = src[src_rows[i]] for whole per-sequence states.
// Grid (num_rows, parts of 2048 16-byte vectors).  Out-of-range row indices
// are skipped so that device index arrays can never send a copy out of
// bounds.
// ---------------------------------------------------------------------------
constexpr int kSnapVecsPerThread = 8;

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
        prof_begin(PROF_SNAPSHOT, st);
        hipLaunchKernelGGL(gdn_snapshot_kernel, dim3((unsigned)p.num_rows, (unsigned)parts), dim3(kThreads), 0,
                           st, p.src, p.src_rows, p.src_capacity, p.dst, p.dst_rows, p.dst_capacity, row_vec4);
        prof_end(st);
    }
    return hipGetLastError();
}

}  // namespace gdn
