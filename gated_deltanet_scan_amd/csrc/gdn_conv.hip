// gdn_conv.hip -- the depthwise causal conv1d ahead of the gated delta rule,
// fused with the L2 normalisation of the q and k heads, on gfx950.
//
// The pages put a depthwise causal conv in the layer ahead of the recurrence,
// with a per-layer conv state kept between calls next to the recurrent state
// (NPU page "Qwen3.5-9B -- every component on the Intel NPU", section "How it
// works": 24 conv states and 24 recurrent states; section "New in v2": prefix
// reuse keeps the recurrent/conv/KV state), oriented like PyTorch's
// left-padded Conv1d (Candle pull-request page, section "Bug elimination log",
// bug 2).  For channel c of token t of a sequence starting at token a:
//     y[t, c] = sum_{i<K} w[c, i] x[t - K + 1 + i, c],
// where x[a - m] (m = 1 .. K-1) is entry K-1-m of the sequence's conv state.
// Channels are [q heads | k heads | v heads]; optionally silu(y); the q and k
// heads are then divided by sqrt(sum of squares + eps), and the three parts
// are written as the q, k and v operands of the recurrence.
//
// gdn_conv_kernel: each lane owns 16 bytes of channels (8 bf16 or 4 fp32), a
// wave 64 such slots over 16 consecutive tokens: the lane loads its taps and
// the block's rows with the K-1 rows before it at once, then forms the 16
// outputs from registers.  A block whose windows reach before the start of
// its sequence (or across two sequences) takes the taps before each
// sequence's first token from that sequence's state instead.  The head norms
// reduce over the dk / 8 (or dk / 4) lanes of a head with xor shuffles.
// gdn_conv_state_kernel: one thread per (sequence, channel) gathers the last
// K-1 inputs (from the old state when the sequence is shorter) into registers
// and then writes them, so the state can be updated in place; it runs after
// the conv kernel on the same stream.
#include "gdn.h"
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

namespace gdn {

// Sequence n with cu[n] <= t < cu[n + 1] (offsets clamped like the prefill's).
__device__ inline int conv_sequence(const int32_t *cu, int32_t num_seqs, int64_t t)
{
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {   // first n with cu[n + 1] > t
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid + 1] > t)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

constexpr int kConvTokens = 16;   // consecutive tokens per wave

template <typename E, int DK, int KW>
__global__ __launch_bounds__(kThreads) void gdn_conv_kernel(const E *__restrict__ x, const float *__restrict__ w,
                                                             const int32_t *__restrict__ cu, int32_t num_seqs,
                                                             int64_t tokens, int32_t channels, int32_t nq,
                                                             const float *__restrict__ state_in, int32_t silu,
                                                             int32_t l2norm, float eps, E *__restrict__ q,
                                                             E *__restrict__ k, E *__restrict__ v)
{
    constexpr int VN = Vec16<E>::n;
    constexpr int LPH = DK / VN;              // lanes per q/k head
    constexpr int NR = KW - 1 + kConvTokens;  // rows of the block with the window before it
    typedef typename Vec16<E>::type V16;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int groups = (channels + kWave * VN - 1) / (kWave * VN);   // channel groups of one wave
    const int64_t tblock = wave / groups;
    const int64_t t_begin = tblock * kConvTokens;
    if (t_begin >= tokens)
        return;   // whole wave: the token block is uniform
    const int64_t t_end = min<int64_t>(t_begin + kConvTokens, tokens);
    const int c0 = (int)(wave - tblock * groups) * kWave * VN + lane * VN;
    const bool active = c0 < channels;
    const bool in_qk = active && c0 < 2 * nq;

    // this lane's taps, and the block's rows with the K-1 rows before it, all in flight together
    // (the lane's VN x KW taps are 16 * KW contiguous bytes per 4 channels: 16-byte loads)
    float wt[VN][KW];
    static_assert(VN * KW % 4 == 0, "whole 16-byte tap vectors");
#pragma unroll
    for (int u = 0; u < VN * KW / 4; ++u) {
        const f32x4 t4 = active ? *reinterpret_cast<const f32x4 *>(w + (size_t)c0 * KW + 4 * u) : zero4();
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            wt[(4 * u + e4) / KW][(4 * u + e4) % KW] = t4[e4];
    }
    V16 xr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t tau = t_begin - (KW - 1) + r;
        xr[r] = (V16)(E)0.f;
        if (active && tau >= 0 && tau < t_end)
            xr[r] = *reinterpret_cast<const V16 *>(x + tau * channels + c0);
    }
    const int n0 = conv_sequence(cu, num_seqs, t_begin);
    const int64_t a0 = min<int64_t>(max<int64_t>(cu[n0], 0), tokens);
    const int64_t b0 = min<int64_t>(max<int64_t>(cu[n0 + 1], a0), tokens);
    // Every window of the block inside one sequence (the common case): all taps from xr.
    const bool inside = t_begin - (KW - 1) >= a0 && t_end <= b0;

    // silu, the q/k head norm and the store of token t's outputs
    auto finish = [&](int64_t t, float (&acc)[VN]) __attribute__((always_inline)) {
        if (silu) {
#pragma unroll
            for (int e = 0; e < VN; ++e)
                acc[e] = acc[e] * __builtin_amdgcn_rcpf(1.f + __expf(-acc[e]));
        }
        // L2 norm of each q or k head over its LPH lanes (every lane joins the shuffles)
        if (l2norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e)
                ss += acc[e] * acc[e];
#pragma unroll
            for (int d = LPH / 2; d >= 1; d >>= 1)
                ss += __shfl_xor(ss, d, kWave);
            if (in_qk) {
                const float r = 1.f / sqrtf(ss + eps);
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    acc[e] *= r;
            }
        }
        if (active) {
            V16 out;
#pragma unroll
            for (int e = 0; e < VN; ++e)
                out[e] = (E)acc[e];
            E *dst = c0 < nq ? q + t * nq + c0
                             : c0 < 2 * nq ? k + t * nq + (c0 - nq) : v + t * (channels - 2 * nq) + (c0 - 2 * nq);
            *reinterpret_cast<V16 *>(dst) = out;
        }
    };

    if (inside && t_end == t_begin + kConvTokens) {
        static_for<kConvTokens>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            float acc[VN];
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                acc[e] = 0.f;
#pragma unroll
                for (int j = 0; j < KW; ++j)
                    acc[e] += wt[e][j] * to_f32(xr[i + j][e]);
            }
            finish(t_begin + i, acc);
        });
        return;
    }
    // A sequence starts within reach of the block (or the batch ends inside it): the taps
    // before each sequence's first token come from that sequence's state.
    static_for<kConvTokens>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int64_t t = t_begin + i;
        if (t >= t_end)
            return;
        const int n = conv_sequence(cu, num_seqs, t);
        const int64_t a = min<int64_t>(max<int64_t>(cu[n], 0), tokens);
        float acc[VN];
#pragma unroll
        for (int e = 0; e < VN; ++e)
            acc[e] = 0.f;
        static_for<KW>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int64_t tau = t - (KW - 1) + j;
            if (tau >= a) {
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    acc[e] += wt[e][j] * to_f32(xr[i + j][e]);
            } else if (state_in && a - tau <= KW - 1 && active) {
                // entry KW-1-(a - tau) of the state (anything else reads zeros)
                const int64_t m = a - tau;
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    acc[e] += wt[e][j] * state_in[((size_t)n * channels + c0 + e) * (KW - 1) + (KW - 1 - m)];
            }
        });
        finish(t, acc);
    });
}

template <typename E, int KW>
__global__ __launch_bounds__(kThreads) void gdn_conv_state_kernel(const E *__restrict__ x,
                                                                   const int32_t *__restrict__ cu, int32_t num_seqs,
                                                                   int64_t tokens, int32_t channels,
                                                                   const float *state_in, float *state_out)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)num_seqs * channels)
        return;
    const int n = (int)(i / channels), c = (int)(i - (int64_t)n * channels);
    const int64_t a = min<int64_t>(max<int64_t>(cu[n], 0), tokens);
    const int64_t b = min<int64_t>(max<int64_t>(cu[n + 1], a), tokens);
    const int64_t L = b - a;
    float nw[KW - 1];
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) {
        const int64_t tau = L - (KW - 1) + j;   // relative to the sequence start
        if (tau >= 0)
            nw[j] = to_f32(x[(a + tau) * channels + c]);
        else
            nw[j] = state_in ? state_in[(size_t)i * (KW - 1) + (KW - 1) + tau] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < KW - 1; ++j)
        state_out[(size_t)i * (KW - 1) + j] = nw[j];
}

template <typename E, int DK, int KW>
static hipError_t launch_conv_t(const ConvArgs &p)
{
    constexpr int VN = Vec16<E>::n;
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    const int groups = (p.channels + kWave * VN - 1) / (kWave * VN);
    const int64_t waves = (p.tokens + kConvTokens - 1) / kConvTokens * groups;
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    if (blocks > 0) {
        const ProfEvents ev = prof_events(PROF_CONV);
        hipExtLaunchKernelGGL((gdn_conv_kernel<E, DK, KW>), dim3((unsigned)blocks), dim3(kThreads), 0, st, ev.start,
                              ev.stop, 0, static_cast<const E *>(p.x), p.weight, p.cu_seqlens, p.num_seqs, p.tokens,
                              p.channels, p.nq, p.state_in, p.silu, p.l2norm, p.eps, static_cast<E *>(p.q),
                              static_cast<E *>(p.k), static_cast<E *>(p.v));
    }
    if constexpr (KW > 1) {
        if (p.state_out) {
            const int64_t items = (int64_t)p.num_seqs * p.channels;
            const ProfEvents ev = prof_events(PROF_CONV);
            hipExtLaunchKernelGGL((gdn_conv_state_kernel<E, KW>), dim3((unsigned)((items + kThreads - 1) / kThreads)),
                                  dim3(kThreads), 0, st, ev.start, ev.stop, 0, static_cast<const E *>(p.x),
                                  p.cu_seqlens, p.num_seqs, p.tokens, p.channels, p.state_in, p.state_out);
        }
    }
    return hipGetLastError();
}

template <typename E, int DK>
static hipError_t launch_conv_w(const ConvArgs &p)
{
    switch (p.width) {
    case 1: return launch_conv_t<E, DK, 1>(p);
    case 2: return launch_conv_t<E, DK, 2>(p);
    case 3: return launch_conv_t<E, DK, 3>(p);
    case 4: return launch_conv_t<E, DK, 4>(p);
    case 5: return launch_conv_t<E, DK, 5>(p);
    case 6: return launch_conv_t<E, DK, 6>(p);
    case 7: return launch_conv_t<E, DK, 7>(p);
    default: return launch_conv_t<E, DK, 8>(p);
    }
}

hipError_t launch_conv(const ConvArgs &p)
{
    const bool bf = p.io_dtype == GDN_DTYPE_BF16;
    switch (p.dk) {
    case 32: return bf ? launch_conv_w<bf16, 32>(p) : launch_conv_w<float, 32>(p);
    case 64: return bf ? launch_conv_w<bf16, 64>(p) : launch_conv_w<float, 64>(p);
    default: return bf ? launch_conv_w<bf16, 128>(p) : launch_conv_w<float, 128>(p);
    }
}

}  // namespace gdn
