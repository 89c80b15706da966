// gdn_norm.hip -- gated RMSNorm of the Gated DeltaNet output on gfx950.
//
// The pages put a gated RMSNorm right after the DeltaNet output and note that
// it is scale-invariant in that output (NPU page "Qwen3.5-9B -- every
// component on the Intel NPU", section "How it works", the paragraph on fp16
// precision of the DeltaNet output); the SSM norm epsilon comes from the
// config, 1e-6 for Qwen3.5 (Candle pull-request page, section "Bug
// elimination log", bug 7).  Per (token, value head) row of dv elements:
//     y = o / sqrt(mean(o^2) + eps) * w * silu(z),   silu(z) = z / (1 + exp(-z))
// with the weight w [dv] shared by the heads and the gate z shaped like o.
//
// The kernel is bound by HBM: each row of o and z is read once and y written
// once (3 dv io elements per row); the weight stays in cache.  Each lane owns
// 16 bytes of a row (8 bf16 or 4 fp32), a row is dv / 8 (or dv / 4) adjacent
// lanes, and the mean square is reduced over those lanes with xor shuffles.
// A wave runs 4 passes over consecutive row blocks with all their loads issued
// first, so that each lane keeps 8 streaming loads in flight.
// y may be o itself (in place): every lane reads its 16 bytes before writing
// them, and no other lane touches them.
#include "gdn.h"
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

namespace gdn {

constexpr int kNormPasses = 4;   // rows handled per lane (each pass: one row of dv / (16 / sizeof(E)) lanes)

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void gdn_gated_rmsnorm_kernel(const E *o, const E *z, const float *__restrict__ w,
                                                                      E *y, int64_t rows, float eps)
{
    constexpr int VN = Vec16<E>::n;
    constexpr int LPR = D / VN;        // lanes per row
    constexpr int RPW = kWave / LPR;   // rows per wave and pass
    constexpr int UR = kNormPasses;    // passes per wave, all loads issued before any use
    static_assert(D % VN == 0 && LPR <= kWave && (LPR & (LPR - 1)) == 0, "rows of a power-of-two lanes");
    typedef typename Vec16<E>::type V16;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int col = (lane % LPR) * VN;
    // o and z are streamed once: non-temporal loads and stores keep them out of the caches
    V16 ov[UR], zv[UR];
    int64_t row[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        row[u] = (wave * UR + u) * RPW + lane / LPR;
        ov[u] = (V16)(E)0.f;
        zv[u] = (V16)(E)0.f;
        if (row[u] < rows) {   // lanes past the last row read nothing but join the shuffles
            ov[u] = __builtin_nontemporal_load(reinterpret_cast<const V16 *>(o + row[u] * D + col));
            zv[u] = __builtin_nontemporal_load(reinterpret_cast<const V16 *>(z + row[u] * D + col));
        }
    }
    f32x4 wv[VN / 4];
#pragma unroll
    for (int e4 = 0; e4 < VN; e4 += 4)
        wv[e4 / 4] = *reinterpret_cast<const f32x4 *>(w + col + e4);
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        float of[VN], ss = 0.f;
#pragma unroll
        for (int e = 0; e < VN; ++e) {
            of[e] = to_f32(ov[u][e]);
            ss += of[e] * of[e];
        }
#pragma unroll
        for (int d = LPR / 2; d >= 1; d >>= 1)
            ss += __shfl_xor(ss, d, kWave);
        const float r = 1.f / sqrtf(ss * (1.f / D) + eps);
        V16 yv;
#pragma unroll
        for (int e = 0; e < VN; ++e) {
            const float zf = to_f32(zv[u][e]);
            // silu with the hardware exponential and reciprocal (relative error ~1e-6)
            const float gate = zf * __builtin_amdgcn_rcpf(1.f + __expf(-zf));
            yv[e] = (E)(of[e] * r * wv[e / 4][e % 4] * gate);
        }
        if (row[u] < rows)
            __builtin_nontemporal_store(yv, reinterpret_cast<V16 *>(y + row[u] * D + col));
    }
}

template <typename E, int D>
static hipError_t launch_norm_t(const NormArgs &p)
{
    constexpr int RPW = kWave / (D / Vec16<E>::n);
    const int64_t rows = p.tokens * p.hv;
    const int64_t waves = (rows + RPW * kNormPasses - 1) / (RPW * kNormPasses);
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    const ProfEvents ev = prof_events(PROF_NORM);
    hipExtLaunchKernelGGL((gdn_gated_rmsnorm_kernel<E, D>), dim3((unsigned)blocks), dim3(kThreads), 0,
                          static_cast<hipStream_t>(p.stream), ev.start, ev.stop, 0, static_cast<const E *>(p.o),
                          static_cast<const E *>(p.z), p.weight, static_cast<E *>(p.y), rows, p.eps);
    return hipGetLastError();
}

hipError_t launch_norm(const NormArgs &p)
{
    const bool bf = p.io_dtype == GDN_DTYPE_BF16;
    switch (p.dv) {
    case 32: return bf ? launch_norm_t<bf16, 32>(p) : launch_norm_t<float, 32>(p);
    case 64: return bf ? launch_norm_t<bf16, 64>(p) : launch_norm_t<float, 64>(p);
    default: return bf ? launch_norm_t<bf16, 128>(p) : launch_norm_t<float, 128>(p);
    }
}

}  // namespace gdn
