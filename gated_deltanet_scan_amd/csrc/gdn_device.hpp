// gdn_device.hpp -- device-side building blocks shared by the libgdn kernels
// (gfx950 only): element types, 16x16 matrix-core tiles and small helpers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // every kernel runs 4 waves per workgroup
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------------------
// Matrix-core tiles.  All products are built from 16x16 output tiles:
//   acc[16x16] += A[16 x K] * B[K x 16]
// with A given row-major (row stride lda elements) and B given TRANSPOSED,
// i.e. as Bt[16 x K] row-major (row stride ldb), so that both operands are
// read along contiguous K.  A lane contributes row (lane % 16) of A and row
// (lane % 16) of Bt over the K-slice selected by (lane / 16); A and B use the
// same K-slice per lane, so the contraction is complete whatever order the
// hardware sums the slice in.  The result tile is held with lane l owning
// column (l % 16) and rows 4 * (l / 16) + {0, 1, 2, 3}.
// ---------------------------------------------------------------------------
template <typename E>
struct Mma;

template <>
struct Mma<bf16> {
    static constexpr int kStep = 32;  // K per instruction
    static constexpr int kPerLane = 8;
    typedef bf16x8 frag;
    __device__ static inline frag load(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    static constexpr int kStep = 4;
    static constexpr int kPerLane = 1;
    typedef float frag;
    __device__ static inline frag load(const float *p) { return *p; }
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// bf16 with K = 16 per instruction, for contractions whose length is not a
// multiple of 32 (the chunk index when C = 16).
struct MmaBf16K16 {
    static constexpr int kStep = 16;
    static constexpr int kPerLane = 4;
    typedef bf16x4 frag;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    __device__ static inline frag load(const bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                         c, 0, 0, 0);
    }
};

// Instruction used for a contraction of length K.
template <typename E, int K>
struct MmaFor {
    typedef Mma<E> type;
};
template <int K>
struct MmaFor<bf16, K> {
    typedef typename std::conditional<K % 32 == 0, Mma<bf16>, MmaBf16K16>::type type;
};

template <typename E, int K>
__device__ inline f32x4 mma_tile(f32x4 acc, const E *A, int lda, const E *Bt, int ldb, int lane)
{
    typedef typename MmaFor<E, K>::type M;
    static_assert(K % M::kStep == 0, "contraction length must be a whole number of instructions");
    const int r = lane & 15;
    const int kk = (lane >> 4) * M::kPerLane;
    const E *a = A + r * lda + kk;
    const E *b = Bt + r * ldb + kk;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += M::kStep)
        acc = M::mma(M::load(a + k0), M::load(b + k0), acc);
    return acc;
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row of the result tile held in accumulator slot i by this lane.
__device__ inline int tile_row(int lane, int i) { return ((lane >> 4) << 2) + i; }
__device__ inline int tile_col(int lane) { return lane & 15; }

// Four consecutive elements of one column of a result tile, written to a
// transposed LDS buffer (one 8- or 16-byte store).
__device__ inline void store4(bf16 *p, float a, float b, float c, float d)
{
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ inline void store4(float *p, float a, float b, float c, float d)
{
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

// 16-byte vectors of io elements.
template <typename E>
struct Vec16 {
    static constexpr int n = 16 / sizeof(E);
    typedef E type __attribute__((ext_vector_type(16 / sizeof(E))));
};

template <typename E>
__device__ inline float to_f32(E x) { return (float)x; }

// Padding (in elements) that keeps 16-byte alignment of LDS rows and spreads
// consecutive rows over different banks.
template <typename E>
struct LdsPad {
    static constexpr int value = 16 / sizeof(E);
};

// Inclusive prefix sum over the 64 lanes of a wave, on the DPP lane network (no
// LDS traffic): a Hillis-Steele scan inside each row of 16 lanes (shifts 1, 2, 4,
// 8; lanes shifted in from outside the row add 0), then the row totals carried
// forward by the row broadcasts of lanes 15 (into rows 1 and 3) and 31 (into rows
// 2 and 3).
__device__ inline float wave_inclusive_sum(float x)
{
    constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowShr + 1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowShr + 2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowShr + 4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowShr + 8, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, kRowBcast31, 0xc, 0xf, false);
    return x;
}

// Sum over each aligned group of L lanes (L a power of two up to 64), returned to every lane
// of the group.  Within a 16-lane row the exchanges are DPP moves: swap neighbours, swap
// pairs, mirror each half-row, mirror the row; beyond a row they are cross-lane reads.
template <int L>
__device__ inline float group_sum(float x)
{
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "a power of two up to the wave");
    constexpr int kSwap1 = 0xb1, kSwap2 = 0x4e, kHalfMirror = 0x141, kMirror = 0x140;
    if constexpr (L >= 2)
        x += __builtin_amdgcn_update_dpp(0.f, x, kSwap1, 0xf, 0xf, false);
    if constexpr (L >= 4)
        x += __builtin_amdgcn_update_dpp(0.f, x, kSwap2, 0xf, 0xf, false);
    if constexpr (L >= 8)
        x += __builtin_amdgcn_update_dpp(0.f, x, kHalfMirror, 0xf, 0xf, false);
    if constexpr (L >= 16)
        x += __builtin_amdgcn_update_dpp(0.f, x, kMirror, 0xf, 0xf, false);
    if constexpr (L >= 32)
        x += __shfl_xor(x, 16, kWave);
    if constexpr (L >= 64)
        x += __shfl_xor(x, 32, kWave);
    return x;
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (compile-time loop).
template <typename F, int... Is>
__device__ inline void static_for_impl(F &&f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1)
        x += __shfl_xor(x, d, kWave);
    return x;
}

}  // namespace gdn
