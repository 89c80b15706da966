// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The chunkwise-parallel form (NPU page "Qwen3.5-9B -- every component on
// the Intel NPU", section "How it works"): for one chunk of C tokens of one
// value head, with G the cumulative sum of g inside the chunk,
//   N   = diag(beta) [exp(G_t - G_j) k_t.k_j]_{j<t}
//   D   = (I + N)^-1 diag(beta) (V - diag(exp G) K S0)
//   O   = diag(exp G) Q S0 + [exp(G_t - G_j) q_t.k_j]_{j<=t} D
//   S_T = exp(G_T) S0 + K^T diag(exp(G_T - G)) D
// Everything that does not depend on the state (the Gram products, the
// decay matrix, the inverse of I + N, the decayed query-key matrix) is done
// for many chunks at once by the prep kernel; the scan kernel then walks the
// chunks of each sequence in order with the state slice held on chip (the
// state is carried from chunk to chunk in order, the work inside a chunk is
// batched products: Candle pull-request page, section Chunked GatedDeltaNet
// Scan).  Kernels:
//   gdn_chunk_table_kernel  chunk offsets of every sequence (integer scan)
//   gdn_prep_kernel         per (chunk, query/key head): K K^T and Q K^T on
//                           the matrix cores; per value head of the group:
//                           G, log-space-masked exp(G_t - G_j), N, the unit
//                           lower-triangular T = (I + N)^-1, A = decayed Q K^T
//   gdn_chunk_scan_kernel   per (sequence, value head, dv-slice): for each
//                           chunk, [Q;K] S, X = diag(beta)(V - diag(exp G) K S),
//                           D = T X, O = diag(exp G) Q S + A D, S update.
//
// Where the chunks' T and A live.  Global mode: one slot per chunk of the
// batch, slot = chunk_start[n] + c.  Segment mode (the host knows the
// sequence lengths): the launch is split into segments of M local chunk
// indices [s0, s0 + M) of every sequence, slot = n * M + (c - s0); prep and
// scan run per segment, the state is carried in final_state between
// segments, and a segment's T, A, q and k stay in the last-level cache
// between the two kernels.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// Chunk table: chunk_start[n] = sum_{m<n} ceil(L_m / C), clamped to
// max_chunks; chunk_start[num_seqs] = total number of chunks.  Offsets are
// clamped to [0, total_tokens] so that invalid input cannot send later
// kernels out of bounds.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void gdn_chunk_table_kernel(
    const int32_t *__restrict__ cu, int32_t num_seqs, int64_t total_tokens, int32_t chunk,
    int32_t max_chunks, int32_t *__restrict__ chunk_start)
{
    __shared__ int64_t wave_tot[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int64_t carry = 0;
    for (int32_t base = 0; base < num_seqs; base += kThreads) {
        const int32_t n = base + tid;
        int64_t cnt = 0;
        if (n < num_seqs) {
            const int64_t a = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
            const int64_t b = min<int64_t>(max<int64_t>(cu[n + 1], a), total_tokens);
            cnt = (b - a + chunk - 1) / chunk;
        }
        int64_t incl = cnt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            int64_t y = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += y;
        }
        if (lane == kWave - 1)
            wave_tot[wave] = incl;
        __syncthreads();
        int64_t before = carry;
        for (int w = 0; w < wave; ++w)
            before += wave_tot[w];
        if (n < num_seqs)
            chunk_start[n] = (int32_t)min<int64_t>(before + incl - cnt, max_chunks);
        int64_t block = 0;
        for (int w = 0; w < kWaves; ++w)
            block += wave_tot[w];
        carry += block;
        __syncthreads();
    }
    if (tid == 0)
        chunk_start[num_seqs] = (int32_t)min<int64_t>(carry, max_chunks);
}

// Sequence that owns chunk entry e: chunk_start[n] <= e < chunk_start[n+1].
__device__ inline int find_sequence(const int32_t *chunk_start, int32_t num_seqs, int32_t e)
{
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_start[mid] <= e)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

__device__ inline void seq_range(const int32_t *cu, int n, int64_t total_tokens, int64_t &a, int64_t &b)
{
    a = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
    b = min<int64_t>(max<int64_t>(cu[n + 1], a), total_tokens);
}

// Placement of chunk slots in the workspace (see the file header).
struct SlotMap {
    const int32_t *chunk_start;  // global mode: per-sequence first slot; NULL in segment mode
    int32_t seg_first;           // first local chunk index of this launch
    int32_t seg_len;             // local chunks per sequence in this launch
};

// Number of chunks of sequence n (consistent with the clamping of the chunk table).
__device__ inline int seq_chunks(const SlotMap &m, const int32_t *cu, int n, int64_t total_tokens, int chunk)
{
    if (m.chunk_start)
        return m.chunk_start[n + 1] - m.chunk_start[n];
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    return (int)((b - a + chunk - 1) / chunk);
}

__device__ inline size_t slot_of(const SlotMap &m, int n, int c)
{
    if (m.chunk_start)
        return (size_t)m.chunk_start[n] + c;
    return (size_t)n * m.seg_len + (c - m.seg_first);
}

// ---------------------------------------------------------------------------
// Prep kernel.  One workgroup per (chunk slot, query/key head); writes, for
// every value head h of the group,
//   tmat[slot][h] = (I + N)^-1   (C x C, row-major, unit lower triangular)
//   amat[slot][h] = [exp(G_t - G_j) q_t.k_j]_{j<=t}  (C x C, zero above)
//
// The inverse is formed in 16 x 16 blocks: the diagonal blocks D_b by
// forward substitution (one lane per column), then the blocks below the
// diagonal, one block-diagonal at a time, by
//   T_{b,b'} = -D_b * sum_{b' <= m < b} N_{b,m} T_{m,b'}
// which is the exact block-doubling identity (D + C)^-1 = D^-1 - D^-1 C D^-1
// of the NPU page applied to the block-triangular split, in fp32 on the
// matrix cores.
// ---------------------------------------------------------------------------
template <typename E, int C, int DK>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, SlotMap map, int32_t num_seqs,
    int64_t total_tokens, int32_t hqk, int32_t hv, E *__restrict__ tmat, E *__restrict__ amat,
    float *__restrict__ dec)
{
    constexpr int PAD = LdsPad<E>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDF = C + 4;      // fp32 C x C rows
    constexpr int RT = C / 16;      // 16-row blocks
    constexpr int HB = 2;           // value heads per pass
    constexpr int IN_BYTES = 2 * C * LDK * (int)sizeof(E);
    constexpr int F_BYTES = HB * C * LDF * (int)sizeof(float);
    constexpr int U1 = IN_BYTES > F_BYTES ? IN_BYTES : F_BYTES;   // Ks,Qs  then N of HB heads
    constexpr int U2 = 2 * C * LDF * (int)sizeof(float);           // KK,QK  then T of HB heads
    static_assert(U2 >= F_BYTES, "T of HB heads must fit where the Gram products were");
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;

    __shared__ __attribute__((aligned(16))) unsigned char smem_a[U1];
    __shared__ __attribute__((aligned(16))) unsigned char smem_b[U2];
    __shared__ __attribute__((aligned(16))) float Yw[kWaves][16][17];
    __shared__ float Gs[HB][C];
    __shared__ float Bs[HB][C];
    E *Ks = reinterpret_cast<E *>(smem_a);
    E *Qs = Ks + C * LDK;
    float *Nm = reinterpret_cast<float *>(smem_a);   // [HB][C][LDF], after the Gram products
    float *KK = reinterpret_cast<float *>(smem_b);
    float *QK = KK + C * LDF;
    float *Tf = reinterpret_cast<float *>(smem_b);   // [HB][C][LDF], after N and A are built

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int hq = blockIdx.y;
    int n, c;
    size_t slot;
    if (map.chunk_start) {
        const int32_t e = blockIdx.x;
        if (e >= map.chunk_start[num_seqs])
            return;
        n = find_sequence(map.chunk_start, num_seqs, e);
        c = e - map.chunk_start[n];
        slot = e;
    } else {
        n = blockIdx.x / map.seg_len;
        c = map.seg_first + (int)(blockIdx.x - n * map.seg_len);
        if (n >= num_seqs || c >= seq_chunks(map, cu, n, total_tokens, C))
            return;
        slot = blockIdx.x;
    }
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int64_t t0 = a + (int64_t)c * C;
    const int len = (int)min<int64_t>(C, b - t0);

    // Q and K rows of this query/key head (rows past the end are zero), then K K^T and
    // Q K^T, lower block triangle only (tile row >= tile column).  The T of one pass
    // overwrites the Gram products, so every pass after the first stages them again.
    auto stage_gram = [&]() {
        for (int i = tid; i < C * DK / VN; i += kThreads) {
            const int r = i / (DK / VN), c0 = (i % (DK / VN)) * VN;
            V16 kv = (V16)(E)0.f, qv = (V16)(E)0.f;
            if (r < len) {
                const size_t off = ((size_t)(t0 + r) * hqk + hq) * DK + c0;
                kv = *reinterpret_cast<const V16 *>(k + off);
                qv = *reinterpret_cast<const V16 *>(q + off);
            }
            *reinterpret_cast<V16 *>(Ks + r * LDK + c0) = kv;
            *reinterpret_cast<V16 *>(Qs + r * LDK + c0) = qv;
        }
        __syncthreads();
        constexpr int NT = RT * (RT + 1) / 2;
        for (int it = wave; it < 2 * NT; it += kWaves) {
            const int which = it / NT;
            const int t = it % NT;
            int tr = 0;
            while ((tr + 1) * (tr + 2) / 2 <= t)
                ++tr;
            const int tc = t - tr * (tr + 1) / 2;
            const E *A = (which ? Qs : Ks) + tr * 16 * LDK;
            const E *Bt = Ks + tc * 16 * LDK;
            const f32x4 acc = mma_tile<E, DK>(zero4(), A, LDK, Bt, LDK, lane);
            float *dst = which ? QK : KK;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(tr * 16 + tile_row(lane, i)) * LDF + tc * 16 + tile_col(lane)] = acc[i];
        }
        __syncthreads();
    };

    const int group = hv / hqk;
    for (int hb = 0; hb < group; hb += HB) {
        const int nh = min(HB, group - hb);
        stage_gram();
        // G = in-chunk inclusive cumulative sum of g; padding tokens carry g = 0, beta = 0.
        if (wave < nh) {
            const int h = hq * group + hb + wave;
            float gv = 0.f, bv = 0.f;
            if (lane < len) {
                gv = g[(size_t)(t0 + lane) * hv + h];
                bv = beta[(size_t)(t0 + lane) * hv + h];
            }
            const float G = wave_inclusive_sum(gv, lane);
            // lanes >= len carry g = 0, so lane C-1 holds G at the last real token
            const float Glast = __shfl(G, C - 1, kWave);
            if (lane < C) {
                Gs[wave][lane] = G;
                Bs[wave][lane] = bv;
                // decay record of the chunk for the scan: exp(G_t), exp(G_last - G_t), beta_t
                float *rec = dec + (slot * hv + h) * 3 * C;
                rec[lane] = expf(G);
                rec[C + lane] = expf(Glast - G);
                rec[2 * C + lane] = bv;
            }
        }
        __syncthreads();
        // exp(G_t - G_j) only for j <= t, where the exponent is <= 0 (log-space mask).
        // One thread per VN consecutive entries of a row: one 16-byte store of A.
        for (int idx = tid; idx < nh * C * C / VN; idx += kThreads) {
            const int hh = idx / (C * C / VN);
            const int rem = (idx - hh * (C * C / VN)) * VN;
            const int t = rem / C, j0 = rem - (rem / C) * C;
            const int h = hq * group + hb + hh;
            const float gt = Gs[hh][t], bt = Bs[hh][t];
            V16 av;
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const int j = j0 + e;
                const float ed = (j <= t) ? __expf(gt - Gs[hh][j]) : 0.f;
                Nm[(hh * C + t) * LDF + j] = (j < t) ? bt * ed * KK[t * LDF + j] : 0.f;
                av[e] = (E)(ed * QK[t * LDF + j]);
            }
            *reinterpret_cast<V16 *>(amat + (slot * hv + h) * C * C + rem) = av;
        }
        __syncthreads();   // KK, QK are dead from here: their space holds T

        // Diagonal blocks D_b: one wave per head, lane = (block b, column j).
        if (wave < nh) {
            const int bb = lane >> 4, j = lane & 15;
            if (bb < RT) {
                const float *Nb = Nm + (wave * C + bb * 16) * LDF + bb * 16;
                float *Tb = Tf + (wave * C + bb * 16) * LDF + bb * 16;
                float x[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float s = (t == j) ? 1.f : 0.f;
#pragma unroll
                    for (int u = 0; u < t; ++u)
                        s -= Nb[t * LDF + u] * x[u];
                    x[t] = s;
                }
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    Tb[t * LDF + j] = x[t];
            }
        }
        __syncthreads();

        // Blocks below the diagonal, one block-diagonal (distance d) at a time.
        for (int d = 1; d < RT; ++d) {
            const int nblk = nh * (RT - d);
            // Y = sum_m N_{b,m} T_{m,b'}   (b = b' + d), one wave per block
            for (int base = 0; base < nblk; base += kWaves) {
                const int blk = base + wave;
                if (blk < nblk) {
                    const int hh = blk / (RT - d), bp = blk % (RT - d), bq = bp + d;
                    const float *Nh = Nm + hh * C * LDF;
                    const float *Th = Tf + hh * C * LDF;
                    f32x4 acc = zero4();
                    for (int m = bp; m < bq; ++m) {
#pragma unroll
                        for (int k4 = 0; k4 < 16; k4 += 4) {
                            const float av = Nh[(bq * 16 + (lane & 15)) * LDF + m * 16 + k4 + (lane >> 4)];
                            const float bv = Th[(m * 16 + k4 + (lane >> 4)) * LDF + bp * 16 + (lane & 15)];
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Yw[wave][tile_row(lane, i)][tile_col(lane)] = acc[i];
                }
                __syncthreads();
                if (blk < nblk) {
                    const int hh = blk / (RT - d), bp = blk % (RT - d), bq = bp + d;
                    float *Th = Tf + hh * C * LDF;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int k4 = 0; k4 < 16; k4 += 4) {
                        const float av = Th[(bq * 16 + (lane & 15)) * LDF + bq * 16 + k4 + (lane >> 4)];
                        const float bv = Yw[wave][k4 + (lane >> 4)][lane & 15];
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Th[(bq * 16 + tile_row(lane, i)) * LDF + bp * 16 + tile_col(lane)] = -acc[i];
                }
                __syncthreads();
            }
        }

        // T to global, zero above the diagonal blocks.
        for (int idx = tid; idx < nh * C * C / VN; idx += kThreads) {
            const int hh = idx / (C * C / VN);
            const int rem = (idx - hh * (C * C / VN)) * VN;
            const int t = rem / C, j0 = rem - (rem / C) * C;
            const int h = hq * group + hb + hh;
            V16 tv;
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const int j = j0 + e;
                tv[e] = (E)(((j >> 4) <= (t >> 4)) ? Tf[(hh * C + t) * LDF + j] : 0.f);
            }
            *reinterpret_cast<V16 *>(tmat + (slot * hv + h) * C * C + rem) = tv;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Scan kernel.  One workgroup per (sequence, value head, dv-slice of DVS
// columns).  The dv columns of S evolve independently (each column of the
// state only ever meets the same column of v), so slices need no exchange;
// the key dimension is never split.  The fp32 state slice lives in the
// accumulators of the S-update tiles for the whole sequence; a bf16 (or
// fp32) copy transposed in LDS feeds the [Q;K] S product of the next chunk.
//
// Chunk inputs (Q, K, T, A, the V slice and the decay record) are copied
// from global memory straight into one of two LDS stage buffers by the
// direct-to-LDS loads (lane i of a load lands at base + 16 i), one chunk
// ahead of the chunk being computed, so no registers or LDS store
// instructions are spent on staging.  Staged rows are not padded: within a
// row the 16-byte chunks are permuted (Swz) so that the 16-row operand
// reads and the 4-row transpose reads hit distinct LDS banks.  Rows past the
// end of a sequence are loaded from its last row: every term they feed is
// multiplied by beta = 0, by a zero column of A or by a unit row of T.
//
// The S update contracts over the chunk index, so it needs K^T as a matrix
// operand: with bf16 it is read from the row-major K tile with the LDS
// transpose read (ds_read_b64_tr_b16: in every group of 16 lanes, input lane
// 4e + q reads 4 consecutive elements of row e, and output lane j receives
// column j of the 4 rows); with fp32 every lane reads its single element.
//
// Block index -> work: the 8 XCDs take workgroups round-robin, so the dv
// slices of one (sequence, head) are placed on one XCD (shared Q, K, T, A
// reads then hit the same L2).
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Byte layout of a staged tile with rows of RB bytes: row r holds its 16-byte
// chunk j at position j ^ perm(r).  perm is injective over 16 consecutive rows
// of one 256-byte bank line and moves 4 consecutive rows by even amounts, so
// both read patterns above are conflict-free.
template <int RB>
struct Swz {
    static_assert(RB % 16 == 0 && RB <= 256, "rows of 16..256 bytes");
    static constexpr int NCH = RB / 16;
    static constexpr int RPL = 256 / RB;   // rows per 256-byte bank line
    __device__ static inline int perm(int r)
    {
        if constexpr (NCH < 4) {
            return 0;
        } else {
            const int u = r / RPL;
            return ((u & (NCH / 2 - 1)) << 1) | ((u / (NCH / 2)) & 1);
        }
    }
    __device__ static inline int off(int r, int b) { return r * RB + ((((b >> 4) ^ perm(r)) << 4) | (b & 15)); }
};

// LDS row stride (elements) of the padded key-dimension tile St.  In dwords it
// is a multiple of 4 with an odd quotient, so 16 rows read with 16-byte
// accesses hit 16 distinct bank groups.
template <typename E>
constexpr int key_row_stride(int dk)
{
    const int dw = dk * (int)sizeof(E) / 4;
    for (int s = (dw + 3) / 4 * 4;; s += 4)
        if ((s / 4) % 2 == 1)
            return s * 4 / (int)sizeof(E);
}

template <typename E, int C, int DK>
struct KtOperand;

// bf16: fragments of K^T straight from the staged K tile (LDS transpose read).
template <int C, int DK>
struct KtOperand<bf16, C, DK> {
    typedef typename MmaFor<bf16, C>::type M;
    typedef Swz<DK * 2> S;
    // A-fragment of K^T for output rows m0..m0+15 (key index), contraction slice
    // starting at chunk row k0.
    __device__ static inline typename M::frag load(const unsigned char *Kb, int m0, int k0, int lane)
    {
        const int g = lane >> 4, s = lane & 15, e = s >> 2, qd = s & 3;
        const int b = 2 * (m0 + 4 * qd);
        if constexpr (M::kPerLane == 8) {
            const int r0 = k0 + 8 * g + e;
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(r0, b)));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(r0 + 4, b)));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        } else {
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(k0 + 4 * g + e, b)));
            return __builtin_bit_cast(bf16x4, lo);
        }
    }
};

// fp32: every lane reads its element K[k0 + lane/16][m0 + lane%16].
template <int C, int DK>
struct KtOperand<float, C, DK> {
    typedef Mma<float> M;
    typedef Swz<DK * 4> S;
    __device__ static inline float load(const unsigned char *Kb, int m0, int k0, int lane)
    {
        return *reinterpret_cast<const float *>(Kb + S::off(k0 + (lane >> 4), 4 * (m0 + (lane & 15))));
    }
};

// Operand fragment (K-slice of one row) of a staged tile.
template <typename M, typename S, typename E>
__device__ inline typename M::frag staged_frag(const unsigned char *base, int row, int col)
{
    return M::load(reinterpret_cast<const E *>(base + S::off(row, col * (int)sizeof(E))));
}

constexpr int kScanThreads = 2 * kThreads;   // 4 compute waves + 4 loader waves

template <typename E, int C, int DK, int DVS>
__global__ __launch_bounds__(kScanThreads) void gdn_chunk_scan_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v, const int32_t *__restrict__ cu,
    SlotMap map, int32_t num_seqs, int64_t total_tokens, int32_t hqk, int32_t hv, int32_t dv,
    const E *__restrict__ tmat, const E *__restrict__ amat, const float *__restrict__ dec, const float *state_in,
    float *state_out, E *__restrict__ o, float scale)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int PAD = LdsPad<E>::value;
    constexpr int LDK = key_row_stride<E>(DK);
    constexpr int LDC = C + PAD;
    constexpr int LDV = DVS + PAD;
    constexpr int RT = C / 16, CT = DVS / 16, SR = DK / 16;
    constexpr int SR_PER = (SR + kWaves - 1) / kWaves;
    constexpr int RT_PER = (RT + kWaves - 1) / kWaves;
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;
    typedef KtOperand<E, C, DK> KT;
    typedef typename MmaFor<E, C>::type MC;
    typedef typename MmaFor<E, DK>::type MK;
    typedef Swz<DK * ES> SK;
    typedef Swz<C * ES> SC;
    typedef Swz<DVS * ES> SV;
    static_assert(C <= kWave, "one lane per token of a chunk");
    static_assert(DVS % 16 == 0 && DK % 16 == 0 && C % 16 == 0, "16x16 tiles");

    // stage buffer layout (bytes) and the 1 KB direct-load jobs that fill it
    constexpr int OFF_Q = 0;
    constexpr int OFF_K = OFF_Q + C * DK * ES;
    constexpr int OFF_T = OFF_K + C * DK * ES;
    constexpr int OFF_A = OFF_T + C * C * ES;
    constexpr int OFF_V = OFF_A + C * C * ES;
    constexpr int OFF_D = OFF_V + C * DVS * ES;
    constexpr int STAGE = OFF_D + 3 * C * 4;
    constexpr int NJ_QK = (C * DK * ES / 16 + 63) / 64;
    constexpr int NJ_TA = (C * C * ES / 16 + 63) / 64;
    constexpr int NJ_V = (C * DVS * ES / 16 + 63) / 64;
    constexpr int NJ_D = (3 * C * 4 / 16 + 63) / 64;
    constexpr int NJ = 2 * NJ_QK + 2 * NJ_TA + NJ_V + NJ_D;

    __shared__ __attribute__((aligned(1024))) unsigned char stage_mem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) E Xt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E Dt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E LDt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E St[DVS * LDK];
    __shared__ __attribute__((aligned(16))) E Os[C * LDV];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool loader = wave >= kWaves;              // waves 4..7 stage chunks, 0..3 compute
    const int lw = wave - kWaves;                    // loader index
    const int nv = dv / DVS;
    const int pairs = num_seqs * hv;
    const int bid = blockIdx.x;
    const int j8 = bid >> 3;
    const int pair = (j8 / nv) * 8 + (bid & 7);
    const int s = j8 % nv;
    if (pair >= pairs)
        return;
    const int n = pair / hv, h = pair - (pair / hv) * hv;
    const int hq = h / (hv / hqk);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int nch = seq_chunks(map, cu, n, total_tokens, C);
    const int c_begin = map.seg_first;
    const int c_end = min(nch, map.seg_first + map.seg_len);
    const size_t state_base = (size_t)(n * hv + h) * DK * dv + (size_t)s * DVS;
    if (c_begin >= c_end) {
        // No chunk of this sequence in this launch.  The first launch still owes the
        // sequence its final state (initial state passed through, or zeros).
        if (c_begin == 0 && state_in != state_out) {
            for (int i = tid; i < DK * DVS; i += kScanThreads) {
                const size_t off = state_base + (size_t)(i / DVS) * dv + (i % DVS);
                state_out[off] = state_in ? state_in[off] : 0.f;
            }
        }
        return;
    }

    // ---- state slice into accumulators (compute wave w owns key-row tiles w, w+4, ...) ----
    f32x4 sacc[SR_PER][CT];
#pragma unroll
    for (int u = 0; u < SR_PER; ++u) {
        const int sr = wave + u * kWaves;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            sacc[u][ct] = zero4();
            if (!loader && sr < SR) {
                if (state_in) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sacc[u][ct][i] = state_in[state_base + (size_t)(sr * 16 + tile_row(lane, i)) * dv +
                                                  ct * 16 + tile_col(lane)];
                }
                store4(St + (ct * 16 + tile_col(lane)) * LDK + sr * 16 + tile_row(lane, 0), sacc[u][ct][0],
                       sacc[u][ct][1], sacc[u][ct][2], sacc[u][ct][3]);
            }
        }
    }

    // ---- loaders: chunk c into registers (issue_loads), then into a stage buffer ----
    // Loader lw owns jobs lw, lw + 4, ... of 64 16-byte chunks each; lane l of a job
    // moves physical chunk 64 * idx + l of its tile.
    constexpr int NJ_PER = (NJ + kWaves - 1) / kWaves;
    V16 lbuf[NJ_PER];
    int ldst[NJ_PER];
    // The job list of each loader is fixed at compile time (one branch per loader), and
    // every load is unconditional: a lane past the end of a tile reloads the tile's last
    // chunk and only its LDS store is skipped.  This keeps all loads of a step in flight
    // together instead of behind per-job waits.
    auto issue_jobs = [&](auto lwc, int c) __attribute__((always_inline)) {
        constexpr int LW = decltype(lwc)::value;
        const int64_t t0 = a + (int64_t)c * C;
        const int last = (int)min<int64_t>(C, b - t0) - 1;   // >= 0 for every chunk of the sequence
        const size_t slot = slot_of(map, n, c);
        const size_t ent = (slot * hv + h) * C * C;
#pragma unroll
        for (int u = 0; u < NJ_PER; ++u) {
            const int job = LW + u * kWaves;
            const E *src;
            int dst, valid;
            if (job < 2 * NJ_QK) {
                const int which = job / NJ_QK, idx = job % NJ_QK;
                const int P = idx * 64 + lane;                     // physical chunk of the tile
                const int r = P / (DK * ES / 16), pos = P % (DK * ES / 16);
                const int j = pos ^ SK::perm(r);
                src = (which ? k : q) + ((size_t)(t0 + min(r, last)) * hqk + hq) * DK + j * VN;
                dst = (which ? OFF_K : OFF_Q) + P * 16;
                valid = 1;
            } else if (job < 2 * NJ_QK + 2 * NJ_TA) {
                constexpr int NCK = C * C * ES / 16;
                const int jj = job - 2 * NJ_QK;
                const int which = jj / NJ_TA, idx = jj % NJ_TA;
                const int P = idx * 64 + lane;
                valid = P < NCK;
                const int Pl = min(P, NCK - 1);
                const int r = Pl / (C * ES / 16), pos = Pl % (C * ES / 16);
                const int j = pos ^ SC::perm(r);
                src = (which ? amat : tmat) + ent + (size_t)r * C + j * VN;
                dst = (which ? OFF_A : OFF_T) + P * 16;
            } else if (job < 2 * NJ_QK + 2 * NJ_TA + NJ_V) {
                constexpr int NCK = C * DVS * ES / 16;
                const int P = (job - 2 * NJ_QK - 2 * NJ_TA) * 64 + lane;
                valid = P < NCK;
                const int Pl = min(P, NCK - 1);
                const int r = Pl / (DVS * ES / 16), pos = Pl % (DVS * ES / 16);
                const int j = pos ^ SV::perm(r);
                src = v + ((size_t)(t0 + min(r, last)) * hv + h) * dv + (size_t)s * DVS + j * VN;
                dst = OFF_V + P * 16;
            } else {
                constexpr int NCK = 3 * C * 4 / 16;
                const int P = job < NJ ? (job - 2 * NJ_QK - 2 * NJ_TA - NJ_V) * 64 + lane : NCK;
                valid = P < NCK;
                src = reinterpret_cast<const E *>(dec + (slot * hv + h) * 3 * C + min(P, NCK - 1) * 4);
                dst = OFF_D + P * 16;
            }
            ldst[u] = valid ? dst : -1;
            lbuf[u] = *reinterpret_cast<const V16 *>(src);
        }
    };
    auto issue_loads = [&](int c) __attribute__((always_inline)) {
        switch (lw) {
        case 0: issue_jobs(std::integral_constant<int, 0>{}, c); break;
        case 1: issue_jobs(std::integral_constant<int, 1>{}, c); break;
        case 2: issue_jobs(std::integral_constant<int, 2>{}, c); break;
        default: issue_jobs(std::integral_constant<int, 3>{}, c); break;
        }
    };
    auto write_stage = [&](int buf) __attribute__((always_inline)) {
        unsigned char *stg = stage_mem + buf * STAGE;
#pragma unroll
        for (int u = 0; u < NJ_PER; ++u)
            if (ldst[u] >= 0)
                *reinterpret_cast<V16 *>(stg + ldst[u]) = lbuf[u];
    };
    // Outputs of a finished chunk (staged in Os by the compute waves): coalesced
    // 16-byte rows to global, written by the loaders.
    auto flush = [&](int64_t t0, int len) __attribute__((always_inline)) {
        constexpr int O_VECS = C * DVS / VN;
        for (int i = tid - kThreads; i < O_VECS; i += kThreads) {
            const int r = i / (DVS / VN), c0 = (i % (DVS / VN)) * VN;
            if (r < len)
                *reinterpret_cast<V16 *>(o + ((size_t)(t0 + r) * hv + h) * dv + (size_t)s * DVS + c0) =
                    *reinterpret_cast<const V16 *>(Os + r * LDV + c0);
        }
    };

    // ---- compute waves: one chunk step on stage buffer `cur` (barriers B1 and B2 inside) ----
    auto step = [&](int cur) __attribute__((always_inline)) {
        const unsigned char *stg = stage_mem + cur * STAGE;
        const float *Gam = reinterpret_cast<const float *>(stg + OFF_D);
        const float *Lam = Gam + C;
        const float *Bet = Gam + 2 * C;

        // P1: Q S and K S for row tile rt (all column tiles); X = diag(beta)(V - diag(exp G) K S)
        //     goes to Xt (transposed); diag(exp G) Q S stays in oacc for P3.
        f32x4 oacc[RT_PER][CT];
        f32x4 kacc[RT_PER][CT];
#pragma unroll
        for (int u = 0; u < RT_PER; ++u) {
            const int rt = wave + u * kWaves;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                oacc[u][ct] = zero4();
                kacc[u][ct] = zero4();
            }
            if (rt < RT) {
                const int r = lane & 15, kk = (lane >> 4) * MK::kPerLane;
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += MK::kStep) {
                    const auto aq = staged_frag<MK, SK, E>(stg + OFF_Q, rt * 16 + r, k0 + kk);
                    const auto ak = staged_frag<MK, SK, E>(stg + OFF_K, rt * 16 + r, k0 + kk);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const typename MK::frag bs = MK::load(St + (ct * 16 + r) * LDK + k0 + kk);
                        oacc[u][ct] = MK::mma(aq, bs, oacc[u][ct]);
                        kacc[u][ct] = MK::mma(ak, bs, kacc[u][ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int col = ct * 16 + tile_col(lane);
                    float x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = rt * 16 + tile_row(lane, i);
                        const E vv = *reinterpret_cast<const E *>(stg + OFF_V + SV::off(rr, col * ES));
                        x[i] = Bet[rr] * (to_f32(vv) - Gam[rr] * kacc[u][ct][i]);
                        oacc[u][ct][i] *= Gam[rr];
                    }
                    store4(Xt + col * LDC + rt * 16 + tile_row(lane, 0), x[0], x[1], x[2], x[3]);
                }
            }
        }
        __syncthreads();   // B1

        // P2: D = T X -> Dt and (diag(lambda) D) -> LDt, both transposed
#pragma unroll
        for (int u = 0; u < RT_PER; ++u) {
            const int rt = wave + u * kWaves;
            if (rt < RT) {
                f32x4 dacc[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    dacc[ct] = zero4();
                const int r = lane & 15, kk = (lane >> 4) * MC::kPerLane;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += MC::kStep) {
                    const auto at = staged_frag<MC, SC, E>(stg + OFF_T, rt * 16 + r, k0 + kk);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        dacc[ct] = MC::mma(at, MC::load(Xt + (ct * 16 + r) * LDC + k0 + kk), dacc[ct]);
                }
                const int r0 = rt * 16 + tile_row(lane, 0);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int col = ct * 16 + tile_col(lane);
                    store4(Dt + col * LDC + r0, dacc[ct][0], dacc[ct][1], dacc[ct][2], dacc[ct][3]);
                    store4(LDt + col * LDC + r0, Lam[r0] * dacc[ct][0], Lam[r0 + 1] * dacc[ct][1],
                           Lam[r0 + 2] * dacc[ct][2], Lam[r0 + 3] * dacc[ct][3]);
                }
            }
        }
        __syncthreads();   // B2

        // P3: O = diag(exp G) Q S + A D, scaled, staged in Os
#pragma unroll
        for (int u = 0; u < RT_PER; ++u) {
            const int rt = wave + u * kWaves;
            if (rt < RT) {
                const int r = lane & 15, kk = (lane >> 4) * MC::kPerLane;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += MC::kStep) {
                    const auto aa = staged_frag<MC, SC, E>(stg + OFF_A, rt * 16 + r, k0 + kk);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        oacc[u][ct] = MC::mma(aa, MC::load(Dt + (ct * 16 + r) * LDC + k0 + kk), oacc[u][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Os[(rt * 16 + tile_row(lane, i)) * LDV + ct * 16 + tile_col(lane)] =
                            (E)(scale * oacc[u][ct][i]);
            }
        }
        // P4: S <- exp(G_last) S + K^T diag(lambda) D; refresh the transposed copy
        const float gl = Gam[C - 1];   // exp(G_last): G is flat past the last real token
#pragma unroll
        for (int u = 0; u < SR_PER; ++u) {
            const int sr = wave + u * kWaves;
            if (sr < SR) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    sacc[u][ct] = sacc[u][ct] * gl;
                const int r = lane & 15, kk = (lane >> 4) * MC::kPerLane;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += MC::kStep) {
                    const typename MC::frag akt = KT::load(stg + OFF_K, sr * 16, k0, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        sacc[u][ct] = MC::mma(akt, MC::load(LDt + (ct * 16 + r) * LDC + k0 + kk), sacc[u][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    store4(St + (ct * 16 + tile_col(lane)) * LDK + sr * 16 + tile_row(lane, 0), sacc[u][ct][0],
                           sacc[u][ct][1], sacc[u][ct][2], sacc[u][ct][3]);
            }
        }
    };

    // ---- pipeline: while the compute waves work on chunk c (stage c & 1), the loaders
    //      flush the outputs of chunk c - 1 and stage chunk c + 1 into the other buffer ----
    if (loader) {
        issue_loads(c_begin);
        write_stage(c_begin & 1);
    }
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        if (loader) {
            if (c > c_begin) {
                const int64_t pt0 = a + (int64_t)(c - 1) * C;
                flush(pt0, (int)min<int64_t>(C, b - pt0));
            }
            if (c + 1 < c_end)
                issue_loads(c + 1);
            __syncthreads();   // B1
            __syncthreads();   // B2
            if (c + 1 < c_end)
                write_stage((c + 1) & 1);
        } else {
            step(c & 1);
        }
        __syncthreads();       // end of step: St, Os and the next stage are complete
    }
    if (loader) {
        const int64_t pt0 = a + (int64_t)(c_end - 1) * C;
        flush(pt0, (int)min<int64_t>(C, b - pt0));
    } else {
        // ---- final state ----
#pragma unroll
        for (int u = 0; u < SR_PER; ++u) {
            const int sr = wave + u * kWaves;
            if (sr < SR) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        state_out[state_base + (size_t)(sr * 16 + tile_row(lane, i)) * dv + ct * 16 +
                                  tile_col(lane)] = sacc[u][ct][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------

// Widest dv slice that still gives the chip at least two workgroups per CU.
static int pick_dvs(int64_t pairs, int dv, int widest)
{
    const int64_t want = 512;
    if (widest >= 64 && dv % 64 == 0 && pairs * (dv / 64) >= want)
        return 64;
    if (dv % 32 == 0 && pairs * (dv / 32) >= want)
        return 32;
    return 16;
}

template <typename E, int C, int DK, int DVS>
static void launch_scan(const PrefillArgs &p, const SlotMap &map, const E *tmat, const E *amat, const float *dec,
                        const float *sin, float *sout, hipStream_t st)
{
    const int nv = p.dv / DVS;
    const int64_t pairs = (int64_t)p.num_seqs * p.hv;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * nv;
    const ProfEvents ev = prof_events(PROF_SCAN);
    hipExtLaunchKernelGGL((gdn_chunk_scan_kernel<E, C, DK, DVS>), dim3((unsigned)blocks), dim3(kScanThreads), 0, st,
                          ev.start, ev.stop, 0, static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                          static_cast<const E *>(p.v), p.cu_seqlens, map, p.num_seqs, p.total_tokens, p.hqk, p.hv,
                          p.dv, tmat, amat, dec, sin, sout, static_cast<E *>(p.o), p.scale);
}

template <typename E, int C, int DK>
static hipError_t launch_prefill_t(const PrefillArgs &p)
{
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    // workspace: [chunk table | T matrices | A matrices | decay records]
    int32_t *chunk_start = reinterpret_cast<int32_t *>(p.workspace);
    E *tmat = reinterpret_cast<E *>(static_cast<char *>(p.workspace) + p.table_bytes);
    E *amat = tmat + (size_t)p.max_chunks * p.hv * C * C;
    float *dec = reinterpret_cast<float *>(amat + (size_t)p.max_chunks * p.hv * C * C);
    const int64_t pairs = (int64_t)p.num_seqs * p.hv;
    // Two stage buffers of a chunk leave room for slices of at most 32 columns (bf16)
    // or 16 columns (fp32).
    constexpr bool kWide = sizeof(E) == 2;
    const int dvs = pick_dvs(pairs, p.dv, kWide ? 32 : 16);

    auto scan = [&](const SlotMap &map, const float *sin, float *sout) {
        if constexpr (kWide) {
            if (dvs == 32) {
                launch_scan<E, C, DK, 32>(p, map, tmat, amat, dec, sin, sout, st);
                return;
            }
        }
        launch_scan<E, C, DK, 16>(p, map, tmat, amat, dec, sin, sout, st);
    };
    auto prep = [&](const SlotMap &map, int64_t slots) {
        const ProfEvents ev = prof_events(PROF_PREP);
        hipExtLaunchKernelGGL((gdn_prep_kernel<E, C, DK>), dim3((unsigned)slots, p.hqk), dim3(kThreads), 0, st,
                              ev.start, ev.stop, 0, static_cast<const E *>(p.q), static_cast<const E *>(p.k), p.g,
                              p.beta, p.cu_seqlens, map, p.num_seqs, p.total_tokens, p.hqk, p.hv, tmat, amat, dec);
    };

    if (p.seg_len > 0) {
        // Segment mode: local chunks [s0, s0 + seg_len) of every sequence per step.
        for (int32_t s0 = 0; s0 < p.max_seq_chunks; s0 += p.seg_len) {
            const SlotMap map{nullptr, s0, p.seg_len};
            prep(map, (int64_t)p.num_seqs * p.seg_len);
            scan(map, s0 == 0 ? p.initial_state : p.final_state, p.final_state);
        }
        return hipGetLastError();
    }

    {
        const ProfEvents ev = prof_events(PROF_CHUNK_TABLE);
        hipExtLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                              p.cu_seqlens, p.num_seqs, p.total_tokens, (int32_t)C, p.max_chunks, chunk_start);
    }
    const SlotMap map{chunk_start, 0, INT32_MAX};
    if (p.max_chunks > 0)
        prep(map, p.max_chunks);
    scan(map, p.initial_state, p.final_state);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &p)
{
    const bool bf = p.io_dtype == 1;
#define GDN_PREFILL_CASE(E_, C_, D_)                 \
    if (p.chunk == C_ && p.dk == D_)                 \
        return launch_prefill_t<E_, C_, D_>(p);
    if (bf) {
        GDN_PREFILL_CASE(bf16, 16, 32)
        GDN_PREFILL_CASE(bf16, 16, 64)
        GDN_PREFILL_CASE(bf16, 64, 32)
        GDN_PREFILL_CASE(bf16, 64, 64)
        GDN_PREFILL_CASE(bf16, 64, 128)
    } else {
        GDN_PREFILL_CASE(float, 16, 32)
        GDN_PREFILL_CASE(float, 16, 64)
        GDN_PREFILL_CASE(float, 64, 32)
        GDN_PREFILL_CASE(float, 64, 64)
    }
#undef GDN_PREFILL_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
