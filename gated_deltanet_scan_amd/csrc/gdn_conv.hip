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
// gdn_conv_kernel: each lane owns 16 bytes of channels (8 bf16 or 4 fp32) and
// a wave 64 such slots; a wave walks a range of tokens in blocks of 16.  The
// lane loads its taps once, keeps the current token's window in fp32
// registers (each row converted once, moving down one tap per token) and
// refills a block's row registers with the next block's rows as they are
// consumed, so a block of loads is in flight during compute.  The sequence of
// a token comes from one wide search for the range's first token plus one
// load of the next 63 sequence offsets (a ballot count per token).  Where a
// sequence starts within reach, the window's taps before its first token are
// that sequence's state entries.  The head norms sum over the dk / 8 (or
// dk / 4) lanes of a head with DPP row moves.
// gdn_conv_state_kernel: one thread per (sequence, channel) gathers the last
// K-1 inputs (from the old state when the sequence is shorter) into registers
// and then writes them, so the state can be updated in place; it runs after
// the conv kernel on the same stream.
#include "gdn.h"
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

namespace gdn {

// Sequence of token t: the first n in [0, N-1] with cu[n + 1] > t (N - 1 if there is none).
// t is uniform over the wave and every lane takes part: each round the lanes test the ends of
// 64 sub-spans of the candidates at once, so a batch of up to 65 sequences needs one round of
// loads.  Indexes stay in [0, N - 1] whatever the offsets hold.
__device__ inline int conv_sequence(const int32_t *cu, int32_t num_seqs, int64_t t, int lane)
{
    int lo = 0, hi = num_seqs - 1;   // the answer lies in [lo, hi]
    while (lo < hi) {
        const int step = (hi - lo + kWave - 1) / kWave;
        const int m = lo + (lane + 1) * step - 1;   // last candidate of this lane's sub-span
        const bool past = m < hi && (int64_t)cu[m + 1] <= t;
        lo += __popcll(__ballot(past)) * step;
        hi = min(hi, lo + step - 1);
    }
    return lo;
}

// Workgroups go to the 8 XCDs in turn; renumbered, each XCD takes a contiguous range of the
// work, so the K-1 rows a wave reads before its range (the previous range's last rows) were
// fetched by a wave of the same XCD and sit in its L2.
__device__ inline int64_t xcd_contiguous(int64_t b, int64_t nb)
{
    const int64_t q = nb / 8, r = nb % 8, x = b % 8, s = b / 8;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// s_waitcnt operand: vector memory count 0, the export and LDS/scalar counts left at their maxima
constexpr int kVmcnt0 = 0x0f70;

constexpr int kConvTokens = 16;     // tokens per block: the rows a wave keeps in flight
constexpr int kConvMaxBlocks = 8;   // blocks per wave at most
// Waves per round of the grid: four times what is resident at once (256 CUs x 4 SIMDs x 2, the
// conv kernel's registers allowing two per SIMD), so that finished waves are replaced from the
// queue rather than the chip draining in one step.
constexpr int64_t kConvRound = 8192;

template <typename E, int DK, int KW>
__global__ __launch_bounds__(kThreads) void gdn_conv_kernel(const E *__restrict__ x, const float *__restrict__ w,
                                                             const int32_t *__restrict__ cu, int32_t num_seqs,
                                                             int64_t tokens, int32_t channels, int32_t nq,
                                                             const float *__restrict__ state_in, int32_t silu,
                                                             int32_t l2norm, float eps, E *__restrict__ q,
                                                             E *__restrict__ k, E *__restrict__ v,
                                                             int32_t blocks_per_wave)
{
    constexpr int VN = Vec16<E>::n;
    constexpr int LPH = DK / VN;   // lanes per q/k head
    typedef typename Vec16<E>::type V16;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = xcd_contiguous(blockIdx.x, gridDim.x) * kWaves + threadIdx.x / kWave;
    const int groups = (channels + kWave * VN - 1) / (kWave * VN);   // channel groups of one wave
    const int64_t chunk = wave / groups;
    const int64_t t_w0 = chunk * blocks_per_wave * kConvTokens;
    if (t_w0 >= tokens)
        return;   // whole wave: the token range is uniform
    const int64_t t_w1 = min<int64_t>(t_w0 + (int64_t)blocks_per_wave * kConvTokens, tokens);
    const int c0 = (int)(wave - chunk * groups) * kWave * VN + lane * VN;
    const bool active = c0 < channels;
    const bool in_qk = active && c0 < 2 * nq;
    // Loads of rows and taps are unconditional (no merge of a pending load with another value,
    // so no wait before the next token): lanes past the channels read the last ones, rows past
    // the range repeat its last row; neither reaches an output.
    const int c_ld = active ? c0 : channels - VN;

    // The wave's first sequence, and lane l holding cu[n_first + l]: the sequence of any token
    // of the range is n_first plus the number of those offsets at or before it.  These loads go
    // first so that their round trips overlap the rows'.
    const int n_first = conv_sequence(cu, num_seqs, t_w0, lane);
    const int64_t offs = cu[min(n_first + lane, (int)num_seqs)];
    auto seq_of = [&](int64_t t) __attribute__((always_inline)) {
        const bool past = lane >= 1 && n_first + lane <= num_seqs - 1 && offs <= t;
        const int c = __popcll(__ballot(past));
        // (all 63 offsets passed: only with runs of empty sequences; search from scratch)
        return c < kWave - 1 ? n_first + c : conv_sequence(cu, num_seqs, t, lane);
    };

    // this lane's taps (16 * KW contiguous bytes per 4 channels: 16-byte loads)
    float wt[VN][KW];
    static_assert(VN * KW % 4 == 0, "whole 16-byte tap vectors");
#pragma unroll
    for (int u = 0; u < VN * KW / 4; ++u) {
        const f32x4 t4 = *reinterpret_cast<const f32x4 *>(w + (size_t)c_ld * KW + 4 * u);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            wt[(4 * u + e4) / KW][(4 * u + e4) % KW] = t4[e4];
    }
    // The window of the current token in fp32: xf[j] is tap j, the input K-1-j tokens back.
    // Before the first token it holds the K-1 rows before the range (zeros before token 0).
    float xf[KW][VN];
#pragma unroll
    for (int j = 0; j + 1 < KW; ++j) {
        const int64_t tau = t_w0 - (KW - 1) + j;
        V16 r = (V16)(E)0.f;
        if (tau >= 0)
            r = *reinterpret_cast<const V16 *>(x + tau * channels + c_ld);
#pragma unroll
        for (int e = 0; e < VN; ++e)
            xf[j][e] = to_f32(r[e]);
    }
    // xr[i]: the row of token i of the current block; refilled with the next block's row i as
    // soon as it has entered the window, so a block of rows stays in flight.
    V16 xr[kConvTokens];
#pragma unroll
    for (int i = 0; i < kConvTokens; ++i)
        xr[i] = *reinterpret_cast<const V16 *>(x + min<int64_t>(t_w0 + i, t_w1 - 1) * channels + c_ld);

    // Where a sequence starts within reach, the taps before its first token are its state
    // entries: taps j <- entries first + j, moving down the window like rows.
    auto inject = [&](int n, int first) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j + 1 < KW; ++j) {
            if (first + j < KW - 1) {
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    xf[j][e] = state_in && active
                                   ? state_in[((size_t)n * channels + c0 + e) * (KW - 1) + first + j]
                                   : 0.f;
            }
        }
        // (the state loads complete here, in this rare branch: after it the window holds no
        // pending load, and the tokens that follow need no wait for it)
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
    };
    const int64_t a_first = min<int64_t>(max<int64_t>(__builtin_amdgcn_readfirstlane((int)offs), 0), tokens);
    if (t_w0 - a_first < KW - 1)
        inject(n_first, (int)max<int64_t>(t_w0 - a_first, 0));   // the range starts near its first token
    int n_prev = n_first;

    // where this lane's outputs go: its channels of q, k or v, one row per token
    E *const dst = c0 < nq ? q + c0 : c0 < 2 * nq ? k + (c0 - nq) : v + (c0 - 2 * nq);
    const int64_t dst_stride = c0 < 2 * nq ? nq : channels - 2 * nq;

    // One block of tokens.  The first block runs before the loop, so that the loop is entered
    // with the same loads in flight as its back edge (the wait before each row then counts the
    // refills and stores issued since, not the initial loads).
    auto block = [&](const int64_t t_begin) __attribute__((always_inline)) {
        const int64_t t_end = min<int64_t>(t_begin + kConvTokens, t_w1);
        const bool starts = seq_of(t_end - 1) != n_prev;   // a sequence starts in the block
        E *const dst_block = dst + t_begin * dst_stride;
        static_for<kConvTokens>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int64_t t = t_begin + i;
            if (t >= t_end)
                return;
#pragma unroll
            for (int e = 0; e < VN; ++e)
                xf[KW - 1][e] = to_f32(xr[i][e]);
            // The refill goes after the conversion, into the same registers (no copy, no wait):
            // the empty asm makes the converted values exist here, so the conversion is not sunk
            // to the taps' uses (which would keep the old row alive past the refill).
#pragma unroll
            for (int e = 0; e < VN; ++e)
                asm volatile("" : "+v"(xf[KW - 1][e]));
            __builtin_amdgcn_sched_barrier(0);
            xr[i] = *reinterpret_cast<const V16 *>(x + min<int64_t>(t + kConvTokens, t_w1 - 1) * channels + c_ld);
            if (starts) {
                const int n = seq_of(t);
                if (n != n_prev)
                    inject(n, 0);   // a new sequence starts at t
                n_prev = n;
            }
            float acc[VN];
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                acc[e] = 0.f;
#pragma unroll
                for (int j = 0; j < KW; ++j)
                    acc[e] += wt[e][j] * xf[j][e];
            }
#pragma unroll
            for (int j = 0; j + 1 < KW; ++j)
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    xf[j][e] = xf[j + 1][e];

            if (silu) {
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    acc[e] = acc[e] * __builtin_amdgcn_rcpf(1.f + __expf(-acc[e]));
            }
            // L2 norm of each q or k head over its LPH lanes (every lane joins the exchange)
            if (l2norm) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    ss += acc[e] * acc[e];
                ss = group_sum<LPH>(ss);
                const float r = in_qk ? __builtin_amdgcn_rsqf(ss + eps) : 1.f;
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    acc[e] *= r;
            }
            if (active) {
                V16 out;
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    out[e] = (E)acc[e];
                __builtin_nontemporal_store(out, reinterpret_cast<V16 *>(dst_block + i * dst_stride));
            }
        });
    };
    block(t_w0);
    for (int64_t t_begin = t_w0 + kConvTokens; t_begin < t_w1; t_begin += kConvTokens)
        block(t_begin);
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
    // Blocks per wave: as few rounds of kConvRound waves as kConvMaxBlocks allows, the blocks
    // spread evenly over them (one block per wave while the work fits in one round).
    const int64_t tblocks = (p.tokens + kConvTokens - 1) / kConvTokens;
    const int64_t work = tblocks * groups;
    const int64_t rounds =
        std::max<int64_t>(1, (work + kConvRound * kConvMaxBlocks - 1) / (kConvRound * kConvMaxBlocks));
    const int bpw = (int)std::min<int64_t>(
        kConvMaxBlocks, std::max<int64_t>(1, (work + rounds * kConvRound - 1) / (rounds * kConvRound)));
    const int64_t waves = (tblocks + bpw - 1) / bpw * groups;
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    if (blocks > 0) {
        const ProfEvents ev = prof_events(PROF_CONV);
        hipExtLaunchKernelGGL((gdn_conv_kernel<E, DK, KW>), dim3((unsigned)blocks), dim3(kThreads), 0, st, ev.start,
                              ev.stop, 0, static_cast<const E *>(p.x), p.weight, p.cu_seqlens, p.num_seqs, p.tokens,
                              p.channels, p.nq, p.state_in, p.silu, p.l2norm, p.eps, static_cast<E *>(p.q),
                              static_cast<E *>(p.k), static_cast<E *>(p.v), bpw);
    }
    if constexpr (KW > 1) {
        if (p.state_out) {
            const int64_t items = (int64_t)p.num_seqs * p.channels;
            const ProfEvents ev = prof_events(PROF_CONV_STATE);
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
