// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The chunkwise-parallel form of the rule (NPU page "Qwen3.5-9B -- every
// component on the Intel NPU", section "How it works").  In this file's
// notation, for one chunk of C tokens of one value head entering with state
// S: G is the running sum of g inside the chunk, gamma_t = exp(G_t),
// lambda_t = exp(G_last - G_t), Gamma = exp(G_last); T is the inverse of the
// unit lower-triangular matrix with beta_t exp(G_t - G_j) k_t.k_j below the
// diagonal, and A holds exp(G_t - G_j) q_t.k_j on and below it.  Then
//   X = diag(beta) (V - diag(gamma) K S)     (what the decayed state misses)
//   D = T X                                  (the chunk's corrected writes)
//   O = scale (diag(gamma) Q S + A D)        (the chunk's outputs)
//   S <- Gamma S + K^T diag(lambda) D        (the state after the chunk)
// Everything that does not depend on the state (the Gram products, the
// decay matrix, the inverse of I + N, the decayed query-key matrix) is done
// for many chunks at once by the prep kernel; the scan kernel then walks the
// chunks of each sequence in order with the state slice held on chip (the
// state is carried from chunk to chunk in order, the work inside a chunk is
// batched products: Candle pull-request page, section Chunked GatedDeltaNet
// Scan).  Kernels:
//   gdn_chunk_table_kernel  chunk offsets of every sequence (integer scan), the
//                           longest-first order, each slot's first token and length
//   gdn_seq_order_kernel    the longest-first order alone (segment mode)
//   gdn_prep_kernel         per chunk: K K^T (and Q K^T) on the matrix cores; per
//                           value head: G, log-space-masked exp(G_t - G_j), N, the
//                           unit lower-triangular T = (I + N)^-1, then one of the
//                           forms of PrepForm (T and A; W and M; T alone as hi/lo)
//   gdn_chunk_scan_kernel   direct form (fp32 io, chunk 16): per (sequence, value
//                           head, dv-slice), for each chunk, [Q;K] S,
//                           X = diag(beta)(V - diag(exp G) K S), D = T X,
//                           O = diag(exp G) Q S + A D, S update
//   gdn_chunk_scan_rows_kernel   absorbed form, 16-column slices (few pairs)
//   gdn_chunk_scan_bf16_kernel   absorbed form, whole heads (split batches)
//   gdn_chunk_scan_tform_kernel  T form, whole heads (many pairs)
//
// Where the chunks' T and A live.  Global mode: one slot per chunk of the
// batch, slot = chunk_start[n] + c; or, for a batch whose longest sequences
// take the row-split scan, windows of W local chunks [w0, w0 + W) of every
// sequence, each with a chunk table of its own over the chunks that fall in it,
// slot = chunk_start[n] + (c - w0).  Segment mode (the host knows the
// sequence lengths): the launch is split into segments of M local chunk
// indices [s0, s0 + M) of every sequence, slot = n * M + (c - s0); prep and
// scan run per segment, the state is carried in final_state between
// segments, and a segment's T, A, q and k stay in the last-level cache
// between the two kernels.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_profile.hpp"

#include <algorithm>
#include <mutex>

namespace gdn {

// Order in which the scan kernels take the sequences: by decreasing length
// (ties by index), so that the workgroups of the longest chains of chunk steps
// are dispatched first and the short ones fill the compute units they free.
// order[rank] = n; the ranks form a permutation, so every entry is written
// once.  Quadratic in the number of sequences (used for small batches only).
__device__ inline void rank_sequence(const int32_t *__restrict__ cu, int32_t num_seqs, int64_t total_tokens,
                                     int32_t *__restrict__ order, int n)
{
    if (n >= num_seqs)
        return;
    auto length = [&](int m) {
        const int64_t a = min<int64_t>(max<int64_t>(cu[m], 0), total_tokens);
        const int64_t b = min<int64_t>(max<int64_t>(cu[m + 1], a), total_tokens);
        return b - a;
    };
    const int64_t len = length(n);
    int rank = 0;
    for (int m = 0; m < num_seqs; ++m) {
        const int64_t lm = length(m);
        rank += (lm > len || (lm == len && m < n)) ? 1 : 0;
    }
    order[rank] = n;
}

__global__ __launch_bounds__(kThreads) void gdn_seq_order_kernel(const int32_t *__restrict__ cu, int32_t num_seqs,
                                                               int64_t total_tokens, int32_t *__restrict__ order)
{
    rank_sequence(cu, num_seqs, total_tokens, order, blockIdx.x * kThreads + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Chunk table: chunk_start[n] = sum_{m<n} ceil(L_m / C), clamped to
// max_chunks; chunk_start[num_seqs] = total number of chunks.  Over a window
// of local chunks [win_first, win_first + win_len) a sequence counts only
// its chunks in the window, and a slot's entry is that of local chunk
// win_first + (slot - chunk_start[n]).  Offsets are
// clamped to [0, total_tokens] so that invalid input cannot send later
// kernels out of bounds.  Workgroup 0 builds the table; with `order` given, the
// grid has one thread per sequence and also ranks them (gdn_seq_order_kernel's
// work in the same launch).  With `slot_info` given, workgroup i also writes
// the entries of slots [i K, (i + 1) K) (K = kSlotsPerTableBlock, slots below
// max_chunks): the chunk's first token and its length, length 0 past the
// batch's chunks.  The prep then finds its chunk with one load instead of a
// search of the table.
// ---------------------------------------------------------------------------
constexpr int32_t kSlotsPerTableBlock = 2048;

__global__ __launch_bounds__(kThreads) void gdn_chunk_table_kernel(
    const int32_t *__restrict__ cu, int32_t num_seqs, int64_t total_tokens, int32_t chunk,
    int32_t max_chunks, int32_t *__restrict__ chunk_start, int32_t *__restrict__ order,
    int2 *__restrict__ slot_info, int32_t win_first, int32_t win_len)
{
    if (order)
        rank_sequence(cu, num_seqs, total_tokens, order, blockIdx.x * kThreads + threadIdx.x);
    const int64_t lo = (int64_t)blockIdx.x * kSlotsPerTableBlock;
    const int64_t hi = min<int64_t>(lo + kSlotsPerTableBlock, max_chunks);
    const bool info = slot_info && lo < hi;
    if (blockIdx.x != 0 && !info)
        return;
    __shared__ int64_t wave_tot[kWaves];
    // this block of sequences: first slot (kThreads + 1 entries), first token, end token
    __shared__ int64_t s_first[kThreads + 1], s_a[kThreads], s_b[kThreads];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int64_t carry = 0;
    for (int32_t base = 0; base < num_seqs; base += kThreads) {
        const int32_t n = base + tid;
        int64_t cnt = 0, a = 0, b = 0;
        if (n < num_seqs) {
            a = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
            b = min<int64_t>(max<int64_t>(cu[n + 1], a), total_tokens);
            cnt = min<int64_t>(max<int64_t>((b - a + chunk - 1) / chunk - win_first, 0), win_len);
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
        const int64_t first = before + incl - cnt;
        if (n < num_seqs && blockIdx.x == 0)
            chunk_start[n] = (int32_t)min<int64_t>(first, max_chunks);
        int64_t block = 0;
        for (int w = 0; w < kWaves; ++w)
            block += wave_tot[w];
        if (info) {
            // the slots of this block's sequences that fall among this workgroup's: each
            // thread takes slots in turn and finds the owning sequence in LDS (the last one
            // whose first slot is at most the slot: empty sequences own none)
            const int nb = min(kThreads, num_seqs - base);
            if (tid < nb) {
                s_first[tid] = first;
                s_a[tid] = a;
                s_b[tid] = b;
            }
            if (tid == 0)
                s_first[nb] = carry + block;
            __syncthreads();
            const int64_t e_end = min<int64_t>(hi, carry + block);
            for (int64_t e = max<int64_t>(lo, carry) + tid; e < e_end; e += kThreads) {
                int m0 = 0, m1 = nb;
                while (m1 - m0 > 1) {
                    const int mid = (m0 + m1) >> 1;
                    if (s_first[mid] <= e)
                        m0 = mid;
                    else
                        m1 = mid;
                }
                const int64_t t0 = s_a[m0] + (win_first + e - s_first[m0]) * chunk;
                slot_info[e] = make_int2((int)t0, (int)min<int64_t>(chunk, s_b[m0] - t0));
            }
        }
        carry += block;
        __syncthreads();
    }
    if (blockIdx.x == 0 && tid == 0)
        chunk_start[num_seqs] = (int32_t)min<int64_t>(carry, max_chunks);
    if (info)
        for (int64_t e = max<int64_t>(carry, lo) + tid; e < hi; e += kThreads)
            slot_info[e] = make_int2(0, 0);
}

__device__ inline void seq_range(const int32_t *cu, int n, int64_t total_tokens, int64_t &a, int64_t &b)
{
    a = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
    b = min<int64_t>(max<int64_t>(cu[n + 1], a), total_tokens);
}

// Placement of chunk slots in the workspace (see the file header).
struct SlotMap {
    const int32_t *chunk_start;  // global mode: per-sequence first slot; NULL in segment mode
    int32_t seg_first;           // first local chunk index of this launch (segment or window)
    int32_t seg_len;             // local chunks per sequence in this launch
    const int32_t *seq_order;    // scan kernels: the sequence of rank r is seq_order[r]; NULL: r
    int32_t rank0;               // scan kernels: first rank of this launch (its ranks: rank0 + i)
    int32_t ranks;               // scan launches: number of ranks (sequences) this launch covers
    const int2 *slot_info;       // global mode, prep: per slot, its chunk's first token and length
                                 // (the prep's only source in global mode)
};

// Sequence of the scan work item with rank index i of its launch.
__device__ inline int ranked_sequence(const SlotMap &m, int i)
{
    const int r = m.rank0 + i;
    return m.seq_order ? m.seq_order[r] : r;
}

// Number of chunks of sequence n (consistent with the clamping of the chunk table; in a window,
// the chunks up to the window's end).
__device__ inline int seq_chunks(const SlotMap &m, const int32_t *cu, int n, int64_t total_tokens, int chunk)
{
    if (m.chunk_start)
        return m.seg_first + (m.chunk_start[n + 1] - m.chunk_start[n]);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    return (int)((b - a + chunk - 1) / chunk);
}

__device__ inline size_t slot_of(const SlotMap &m, int n, int c)
{
    if (m.chunk_start)
        return (size_t)((int64_t)m.chunk_start[n] + (c - m.seg_first));
    return (size_t)n * m.seg_len + (c - m.seg_first);
}

// Block index -> (item, member) such that the `members` workgroups of one item run on
// one XCD, dispatched back to back: the 8 XCDs take workgroups round-robin (block b on
// XCD b % 8), so an item's members take blocks 8 apart.  Used so that the workgroups
// that read the same q and k rows (the value heads of a query/key group, and the
// column slices of each) share one XCD's L2.  A grid of ceil(items / 8) * 8 * members
// blocks covers every (item, member) once.
__device__ inline void xcd_group(int bid, int members, int &item, int &member)
{
    const int k = bid >> 3;
    member = k % members;
    item = (k / members) * 8 + (bid & 7);
}

// Byte layout of a staged tile with rows of RB bytes: row r holds its 16-byte
// chunk j at position j ^ perm(r).  perm is injective over 16 consecutive rows
// of one 256-byte line and moves 4 consecutive rows by even amounts, so that
// the 16 rows of an operand read (16 bytes per lane) and the 4 rows of a
// transpose read fall on distinct 16-byte bank groups if the 64 banks are taken
// as consecutive dwords.
//
// Measured LDS rates on gfx950 (8 waves of one workgroup reading in a loop;
// clocks per wave instruction): ds_read_b128 in lane order (lane i at 16 i),
// or permuted the same way inside each 16-lane group's 256-byte block: 34-35.
// This layout, the 272-byte rows of St and the 144-byte exchange tiles of the
// row-split kernel, and the K units of the wide-batch kernel: 64.  Unswizzled
// 128- and 256-byte rows: 102 and 192.  ds_read_b64_tr_b16 in lane order (lane
// i at 8 i): 21; the wide-batch kernel's K and V transpose reads: 32.  So the
// bank mapping is not plain address modulo 64 dwords, and only lane-order
// reads here run at the full rate.
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

// A operand fragment (kPerLane consecutive elements of one row) of a staged tile.
template <typename M, typename S, typename E>
__device__ inline typename M::frag staged_frag(const unsigned char *base, int row, int col)
{
    return M::load(reinterpret_cast<const E *>(base + S::off(row, col * (int)sizeof(E))));
}

// ---------------------------------------------------------------------------
// Register-resident chains of products.  Three products of the chunk step
// take their B operand from the accumulator tiles of an earlier product:
// [Q;K] S (S from the S update), T X and A D (X and D from the products
// before them), K^T (lambda D).  An accumulator tile gives lane l column
// l % 16 and rows 4 (l / 16) + {0..3}; a B fragment wants column l % 16 and
// kPerLane contraction indices per lane group.  Chain<M> (M = the consuming
// instruction) makes the two agree without moving data:
//   row(t, r)     the matrix row that the PRODUCER computes in row r of its
//                 output tile t (it reads that row of its own A operand);
//   b_frag(t, s)  the consumer's B fragment of contraction step s, taken from
//                 the accumulator tiles as they stand;
//   a_col(s, l)   first contraction index of lane l's A fragment at step s.
// ---------------------------------------------------------------------------
template <typename M>
struct Chain;

// 16x16x32 bf16: tiles 2s and 2s+1 hold, in lane group g, the contraction
// indices 32 s + 8 g + {0..3} and 32 s + 8 g + {4..7}.
template <>
struct Chain<Mma<bf16>> {
    __device__ static inline int row(int t, int r) { return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3); }
    __device__ static inline int a_col(int s, int lane) { return 32 * s + 8 * (lane >> 4); }
    __device__ static inline bf16x8 b_frag(const f32x4 *t, int s)
    {
        const f32x4 a = t[2 * s], b = t[2 * s + 1];
        return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    }
};

// 16x16x16 bf16: tile s holds the indices 16 s + 4 g + {0..3} as it stands.
template <>
struct Chain<MmaBf16K16> {
    __device__ static inline int row(int t, int r) { return 16 * t + r; }
    __device__ static inline int a_col(int s, int lane) { return 16 * s + 4 * (lane >> 4); }
    __device__ static inline bf16x4 b_frag(const f32x4 *t, int s)
    {
        const f32x4 a = t[s];
        return bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    }
};

// 16x16x4 fp32: step s = 4 t + i uses slot i of tile t, i.e. in lane group g
// the index 16 t + 4 g + i.
template <>
struct Chain<Mma<float>> {
    __device__ static inline int row(int t, int r) { return 16 * t + r; }
    __device__ static inline int a_col(int s, int lane) { return 16 * (s >> 2) + 4 * (lane >> 4) + (s & 3); }
    __device__ static inline float b_frag(const f32x4 *t, int s) { return t[s >> 2][s & 3]; }
};

// Round x to bf16 (hi) and the remainder to bf16 (lo): hi + lo carries about 16
// significant bits, and products of hi/lo pairs accumulated in fp32 give sums that
// cancel accurately.
__device__ inline void split_bf16(float x, bf16 &hi, bf16 &lo)
{
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
}

// split_bf16 of two values at once, as packed pairs (value 0 in the low half): one
// two-value conversion for the hi pair, one for the remainders.  Returns {hi, lo}.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ inline u32x2 split_bf16x2(float x0, float x1)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
    const f32x2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
    return u32x2{h, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2))};
}

// Which form the chunk matrices take for io type E and chunk C.  Direct form
// (fp32 io, chunk 16): T = (I + N)^-1 and A, and the scan forms D = T X.
// Absorbed form (bf16 io, chunk 64): the products with T are taken in the
// prep, in fp32-accurate arithmetic, as
//   W = K^T diag(lambda) T   (dk x C)  and   M = A T   (C x C),
// so that the scan's step is X = diag(beta)(V - diag(gamma) K S),
// O = scale diag(gamma) Q S + M X, S <- Gamma S + W X (the same products,
// associated differently).  With bf16 matrix-core operands this matters: the
// columns of T alternate in sign when keys are correlated, and D = T X would
// be rounded to bf16 as an operand before its large entries cancel in K^T D
// and A D; W and M are those cancelled sums, formed before any rounding.
template <typename E, int C>
struct AbsorbedForm {
    static constexpr bool value = sizeof(E) == 2 && C == 64;
};

// What the prep writes per (chunk, value head):
//   kPrepDirect    T and A (fp32 io, chunk 16; the scan forms D = T X)
//   kPrepAbsorbed  W and M (bf16 io, chunk 64; row-split and whole-head scans)
//   kPrepTForm     T alone, as hi/lo bf16 pairs (bf16 io, chunk 64, dk 128; the T-form
//                  whole-head scan forms A from its staged q and k and takes Y = T X with
//                  the hi/lo pairs, so the cancelling sums of T's columns stay fp32-accurate)
// and the decay record.  T-form record: [G log2(e) | exp(G_last - G) | beta | beta exp(G)]
// (the scan forms its decays as powers of two and masks exp(G_t - G_j) in log space
// itself); the others: [exp(G) | ... ].
enum PrepForm { kPrepDirect = 0, kPrepAbsorbed = 1, kPrepTForm = 2 };
constexpr float kLog2E = 1.44269504088896340736f;   // log2(e)
// T in the T form: 6 units of 16 rows x 32 columns per bf16 matrix (hi, then lo), the
// units of T's row tiles rt (rows Chain<Mma<bf16>>::row(rt, .)) and column halves st with
// st <= rt / 2 (the other two are zero: T is lower triangular); unit u(rt, st) holds at
// its 16-byte position p the row Chain row(rt, p % 16), columns 32 st + 8 (p / 16) .. +7.
constexpr int kTUnits = 6;
__host__ __device__ constexpr int tform_unit(int rt, int st) { return rt < 2 ? rt : 2 + 2 * (rt - 2) + st; }

template <int C, int DK, int PW, int HB, int NKEEP>
__device__ void absorb_products(const unsigned char *Ks, const float *Tf, float *Am, float (*Gv)[C],
                                f32x4 (&akeep)[NKEEP][HB], int nh, int wv, int lane, bf16 *wout, bf16 *mout);

// ---------------------------------------------------------------------------
// Prep kernel.  One workgroup per (chunk slot, query/key head), or per (chunk
// slot, value head) in the absorbed form; writes, for every value head h of the
// workgroup,
//   tmat[slot][h] = (I + N)^-1   (C x C, row-major, unit lower triangular)
//   amat[slot][h] = scale [exp(G_t - G_j) q_t.k_j]_{j<=t}  (C x C, zero above)
//   dec[slot][h]  = [exp(G) | exp(G_last - G) | beta | beta exp(G)]
// or, in the absorbed form (AbsorbedForm), W = K^T diag(lambda) T (dk x C,
// row-major) in place of T and M = A T (C x C, row-major) in place of A.
//
// All global reads are issued first: the chunk's q and k rows go straight
// into LDS (direct-to-LDS loads, rows in the Swz chunk order; rows past the
// end of the sequence repeat its last row, their products are masked), and
// g, beta of every value head of the pass into registers of every wave.
// Each wave forms the in-chunk cumulative sum G with a DPP lane scan and
// keeps its own LDS copy of G and beta (read back by itself, so no barrier).
// The Gram products K K^T and Q K^T are formed tile by tile on the matrix cores
// in transposed orientation (a lane holds one row t and four consecutive
// columns j), and the log-space mask and decay are applied to the tile in
// registers: N goes to LDS for the solve, A straight to global memory.
//
// The inverse is formed in 16 x 16 blocks: the diagonal blocks D_b by
// forward substitution (one lane per column), then the blocks below the
// diagonal, one block-diagonal at a time, by
//   T_{b,b'} = -D_b * sum_{b' <= m < b} N_{b,m} T_{m,b'}
// which is the exact block-doubling identity (D + C)^-1 = D^-1 - D^-1 C D^-1
// of the NPU page applied to the block-triangular split, in fp32 on the
// matrix cores.
// ---------------------------------------------------------------------------
// Waves of a prep workgroup: four, with one block column of T per wave in the products of
// the absorbed form.
template <typename E, int C>
struct PrepWaves {
    static constexpr int value = 4;
};

template <typename E, int C, int DK, int FORM>
__global__ __launch_bounds__((PrepWaves<E, C>::value * kWave)) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, SlotMap map, int32_t num_seqs,
    int64_t total_tokens, int32_t hqk, int32_t hv, E *__restrict__ tmat, E *__restrict__ amat,
    float *__restrict__ dec, float scale, int32_t nslots)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int LDF = C + 4;      // fp32 C x C rows
    constexpr int RT = C / 16;      // 16-row blocks
    // value heads per workgroup pass: the two of a query/key group share its Gram products
    // (direct form, two workgroups of about 74 KB per CU); in the absorbed form, whose pass
    // keeps k and T alive together, one value head per workgroup (about 53 KB, three per CU;
    // the grid runs over value heads and each computes its group's Gram products)
    constexpr int HB = AbsorbedForm<E, C>::value ? 1 : 2;
    static_assert((FORM != kPrepDirect) == AbsorbedForm<E, C>::value, "form of the io type and chunk");
    static_assert(FORM != kPrepTForm || DK == 128, "T form: dk 128");
    constexpr bool TFORM = FORM == kPrepTForm;   // k rows only, K K^T only, T out
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;
    typedef typename MmaFor<E, DK>::type MK;
    typedef Swz<DK * ES> SK;
    // bf16 io at chunk 64: the products with T are taken here (absorbed form, see absorb_products)
    constexpr bool ABSORB = FORM == kPrepAbsorbed;
    constexpr bool COLT = FORM != kPrepDirect;   // T kept column-major in LDS
    constexpr int TILE = C * DK * ES;                 // bytes of the staged q (or k) rows
    constexpr int F_BYTES = HB * C * LDF * (int)sizeof(float);
    // k, q rows, then T of HB heads: over both (direct form), or over q only (absorbed form,
    // whose products with T still read k)
    // (T form: k rows only, and T over them once the Gram products are done: about 36 KB,
    // four workgroups per CU)
    constexpr int U1 = TFORM   ? (TILE > F_BYTES ? TILE : F_BYTES)
                       : COLT ? TILE + (TILE > F_BYTES ? TILE : F_BYTES)
                              : (2 * TILE > F_BYTES ? 2 * TILE : F_BYTES);
    constexpr int NCK = TILE / 16;                    // 16-byte chunks of a staged tile
    constexpr int NJ1 = NCK / 64;                     // 64-lane load jobs (1 KB) per tile
    constexpr int PW = PrepWaves<E, C>::value, NT = PW * kWave;
    constexpr int NJOBS = TFORM ? NJ1 : 2 * NJ1;       // the T form stages k only
    constexpr int NJ_PER = (NJOBS + PW - 1) / PW;
    constexpr int RB = DK * ES;                       // bytes of a staged row
    constexpr int RPJ = 1024 / RB;                    // rows per load job
    constexpr int KPAT = 16 / RPJ;                    // jobs per period of the row permutation
    static_assert(RB >= 64 && RB <= 256, "staged rows of 64 .. 256 bytes");
    static_assert(NCK % 64 == 0 && NJ1 % KPAT == 0 && PW % KPAT == 0,
                  "whole jobs; every job of a wave has the same lane pattern");
    static_assert(C <= kWave, "one lane per token of a chunk");
    static_assert(!ABSORB || PW == RT * HB, "absorbed form: one (head, block column of T) per wave");

    __shared__ __attribute__((aligned(1024))) unsigned char smem_qk[U1];
    __shared__ __attribute__((aligned(16))) float Nm[HB * C * LDF];   // N; then A (absorbed form)
    __shared__ __attribute__((aligned(16))) float Gw[PW][HB][C];   // each wave's copy of G
    __shared__ __attribute__((aligned(16))) float Bw[PW][HB][C];   // and of beta
    const unsigned char *Ks = smem_qk;                  // staged k rows
    const unsigned char *Qs = smem_qk + TILE;           // staged q rows
    float *Tf = reinterpret_cast<float *>(smem_qk + (ABSORB ? TILE : 0));   // [HB][C][LDF], after the Gram products
    // element (row t, column j) of a head's T: row-major, or column-major in the absorbed and
    // T forms (whose products and unit writes read T by columns)
    auto tix = [](int t, int j) __attribute__((always_inline)) { return COLT ? j * LDF + t : t * LDF + j; };
    __attribute__((address_space(3))) unsigned char *const lds_qk =
        (__attribute__((address_space(3))) unsigned char *)smem_qk;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int group = hv / hqk;
    // chunk slot, query/key head, first value head and number of value heads of this
    // workgroup.  One value head per workgroup: a 1-D grid over (slot, query/key head)
    // items whose value heads share an XCD (their q and k rows then meet in its L2).
    int sidx, hq, hfirst, nheads;
    if constexpr (HB == 1) {
        int item, member;
        xcd_group(blockIdx.x, group, item, member);
        if (item >= nslots * hqk)
            return;
        sidx = item / hqk;
        hq = item - sidx * hqk;
        hfirst = hq * group + member;
        nheads = 1;
    } else {
        sidx = blockIdx.x;
        hq = blockIdx.y;
        hfirst = hq * group;
        nheads = group;
    }
    int64_t t0;
    int len;
    size_t slot;
    if (map.slot_info) {
        // the table launch's entry for this slot (length 0: past the batch), read as one
        // 64-bit load so that the first token is not fetched only after the length test
        const uint64_t si = *reinterpret_cast<const uint64_t *>(map.slot_info + sidx);
        len = (int)(uint32_t)(si >> 32);
        if (len <= 0)
            return;
        t0 = (int)(uint32_t)si;
        slot = sidx;
    } else {   // segment mode
        const int n = sidx / map.seg_len;
        const int c = map.seg_first + (int)(sidx - n * map.seg_len);
        if (n >= num_seqs || c >= seq_chunks(map, cu, n, total_tokens, C))
            return;
        slot = sidx;
        int64_t a, b;
        seq_range(cu, n, total_tokens, a, b);
        t0 = a + (int64_t)c * C;
        len = (int)min<int64_t>(C, b - t0);   // >= 1
    }

    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // q and k rows of the chunk into LDS.  Job idx of a tile moves 1 KB: lane i writes the 16
    // bytes at 16 i of the job's block, i.e. row r = RPJ idx + i / (RB / 16) of the tile, chunk
    // position i % (RB / 16), whose source is chunk (position ^ perm(r)) of that token row
    // (Swz).  perm has period 16 in r, and the jobs of this wave all start at rows
    // = RPJ (wv % KPAT) modulo 16, so one lane offset serves all of them; the rest of a job's
    // offset (16 rows per period) is uniform and goes into the scalar base.  In a ragged chunk
    // rows past its end repeat its last row.
    auto issue_qk = [&]() __attribute__((always_inline)) {
        const uint32_t rowb = (uint32_t)hqk * DK * ES;      // bytes between tokens of one head
        const char *kb = reinterpret_cast<const char *>(k + ((size_t)t0 * hqk + hq) * DK);
        const char *qb = reinterpret_cast<const char *>(q + ((size_t)t0 * hqk + hq) * DK);
        const int lr = lane / (RB / 16), lpos = lane % (RB / 16);
        const int r_in = RPJ * (wv % KPAT) + lr;            // row within the period of perm
        const uint32_t chunk_off = (uint32_t)((lpos ^ SK::perm(r_in)) * 16);
        const uint32_t lane_off = (uint32_t)r_in * rowb + chunk_off;
        const bool ragged = len < C;
#pragma unroll
        for (int u = 0; u < NJ_PER; ++u) {
            const int J = wv + u * PW;
            if (J < NJOBS) {
                const int idx = J % NJ1;
                const char *base = J >= NJ1 ? qb : kb;
                uint32_t off;
                if (!ragged) {
                    base += (size_t)(idx / KPAT) * 16 * rowb;
                    off = lane_off;
                } else {
                    off = (uint32_t)min(RPJ * idx + lr, len - 1) * rowb + chunk_off;
                }
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(base + off),
                    (__attribute__((address_space(3))) void *)(lds_qk + (J >= NJ1 ? TILE : 0) + idx * 1024), 16, 0, 0);
            }
        }
    };

    for (int hb = 0; hb < nheads; hb += HB) {
        const int nh = min(HB, nheads - hb);
        // g and beta of the pass's value heads, one token per lane, in every wave (issued
        // before the q, k rows); padding tokens carry g = 0, beta = 0
        float gv[HB], bv[HB];
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            gv[hh] = 0.f;
            bv[hh] = 0.f;
            if (hh < nh && lane < len) {
                const size_t at = (size_t)t0 * hv + hfirst + hb + hh;   // uniform base, lane offset
                gv[hh] = (g + at)[lane * hv];
                bv[hh] = (beta + at)[lane * hv];
            }
        }
        issue_qk();
        // the direct loads are not tracked by the compiler's LDS dependences
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // G = in-chunk inclusive cumulative sum of g (lanes >= len carry g = 0, so lane
        // C - 1 holds G at the last real token), and the decay record of the chunk
        float Gr[HB];
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            Gr[hh] = wave_inclusive_sum(gv[hh]);
            if (lane < C) {   // this wave's own copy: read back below by the same wave only
                Gw[wv][hh][lane] = Gr[hh];
                Bw[wv][hh][lane] = bv[hh];
            }
        }
        if (wv < nh && lane < C) {
            const int h = hfirst + hb + wv;
            const float G = wv == 0 ? Gr[0] : Gr[HB - 1];
            const float Glast = __shfl(G, C - 1, kWave);
            float *rec = dec + (slot * hv + h) * 4 * C;
            const float eg = expf(G);
            rec[lane] = TFORM ? G * kLog2E : eg;
            rec[C + lane] = expf(Glast - G);
            rec[2 * C + lane] = wv == 0 ? bv[0] : bv[HB - 1];
            rec[3 * C + lane] = (wv == 0 ? bv[0] : bv[HB - 1]) * eg;
        }

        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // Gram tiles, transposed: the tiles of block row tr (rows t) and block column tc
        // (columns j) are computed as K_j . K_t and K_j . Q_t, so lane l holds row
        // t = 16 tr + l % 16 and columns j = 16 tc + 4 (l / 16) + {0..3}.  The lower-triangle
        // tiles (tc <= tr) give N (to LDS; the solve reads nothing above the diagonal) and A
        // (to global memory); A tiles above the diagonal are stored as zeros.  The tiles are
        // dealt to the waves round-robin at compile time, so each wave runs its own items as
        // straight-line code (the reads of one item overlap the products of the previous).
        const int r16 = lane & 15, kq = (lane >> 4) * MK::kPerLane;
        // absorbed form: the wave's A tiles (fp32) stay in registers until T is complete
        constexpr int NKEEP = (RT * (RT + 1) / 2 + PW - 1) / PW;
        f32x4 akeep[NKEEP][HB];
        auto gram_items = [&](auto wc) __attribute__((always_inline)) {
          constexpr int W = decltype(wc)::value;
          static_for<RT * RT>([&](auto pc) {
            constexpr int P = decltype(pc)::value;
            constexpr int tr = P / RT, tc = P % RT;
            constexpr bool lower = tc <= tr;
            constexpr int idx = lower ? tr * (tr + 1) / 2 + tc : (tr * RT + tc) + 2;   // deal index
            if constexpr (idx % PW != W)
                return;
            const int t = tr * 16 + r16;
            const int j0 = tc * 16 + 4 * (lane >> 4);
            if constexpr (lower) {
                constexpr int NS = DK / MK::kStep;
                typename MK::frag fj[NS], fkt[NS], fqt[NS];
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    fj[st] = staged_frag<MK, SK, E>(Ks, tc * 16 + r16, st * MK::kStep + kq);
                    fkt[st] = staged_frag<MK, SK, E>(Ks, tr * 16 + r16, st * MK::kStep + kq);
                    if constexpr (!TFORM)
                        fqt[st] = staged_frag<MK, SK, E>(Qs, tr * 16 + r16, st * MK::kStep + kq);
                }
                f32x4 kk = zero4(), qk = zero4();
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    kk = MK::mma(fj[st], fkt[st], kk);
                    if constexpr (!TFORM)
                        qk = MK::mma(fj[st], fqt[st], qk);
                }
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    if (hh >= nh)
                        break;
                    const int h = hfirst + hb + hh;
                    const float gt = Gw[wv][hh][t], bt = Bw[wv][hh][t];
                    const float st = t < len ? scale : 0.f;   // rows past the chunk's end: A = 0
                    const f32x4 gj = *reinterpret_cast<const f32x4 *>(&Gw[wv][hh][j0]);
                    f32x4 nv, av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // exp(G_t - G_j) only for j <= t, where the exponent is <= 0 (log-space
                        // mask); below the diagonal tiles every j < t
                        const int j = j0 + e;
                        float ed;
                        if constexpr (tc < tr) {
                            ed = __expf(gt - gj[e]);
                            nv[e] = bt * ed * kk[e];
                        } else {
                            ed = (j <= t) ? __expf(gt - gj[e]) : 0.f;
                            nv[e] = (j < t) ? bt * ed * kk[e] : 0.f;
                        }
                        av[e] = st * ed * qk[e];
                    }
                    *reinterpret_cast<f32x4 *>(Nm + (hh * C + t) * LDF + j0) = nv;
                    if constexpr (ABSORB)
                        akeep[idx / PW][hh] = av;
                    else if constexpr (!TFORM)
                        store4(amat + (slot * hv + h) * C * C + t * C + j0, av[0], av[1], av[2], av[3]);
                }
            } else if constexpr (FORM == kPrepDirect) {
#pragma unroll
                for (int hh = 0; hh < HB; ++hh)
                    if (hh < nh)
                        store4(amat + (slot * hv + hfirst + hb + hh) * C * C + t * C + j0, 0.f, 0.f, 0.f, 0.f);
            }
          });
        };
        static_for<PW>([&](auto wc) {
            if (decltype(wc)::value == wv)
                gram_items(wc);
        });
        __syncthreads();   // the q, k rows are dead from here: their space holds T

        // Diagonal blocks D_b: one wave per head, lane = (block b, column j).
        if (wave < nh) {
            const int bb = lane >> 4, j = lane & 15;
            if (bb < RT) {
                const float *Nb = Nm + (wave * C + bb * 16) * LDF + bb * 16;
                float *Tb = Tf + wave * C * LDF + tix(bb * 16, bb * 16);
                float x[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float s = (t == j) ? 1.f : 0.f;
#pragma unroll
                    for (int u = 0; u < t; ++u)
                        s -= Nb[t * LDF + u] * x[u];
                    x[t] = s;
                }
                if constexpr (COLT) {   // column j of the block: 16 consecutive floats
#pragma unroll
                    for (int t = 0; t < 16; t += 4)
                        *reinterpret_cast<f32x4 *>(Tb + j * LDF + t) = f32x4{x[t], x[t + 1], x[t + 2], x[t + 3]};
                } else {
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        Tb[t * LDF + j] = x[t];
                }
            }
        }
        __syncthreads();

        // Blocks below the diagonal.  Block column b' of T depends on nothing but itself,
        // D and N:  T_{b',b'} = D_{b'},  T_{b,b'} = -D_b sum_{b' <= m < b} N_{b,m} T_{m,b'},
        // so each (head, block column) is one chain of products, run by one wave with the
        // column's blocks held in registers.  A block enters the next product as its B
        // operand as it stands in the accumulators: in step s, lane group g contributes the
        // contraction indices 4 g + s, whose B rows are its own accumulator slot s (and the
        // A operand takes the same columns).  The chains are dealt to the waves in snake
        // order, longest first.
        if constexpr (RT > 1) {
            const int nchains = nh * (RT - 1);
            const int r16 = lane & 15, g4 = 4 * (lane >> 4);
            for (int round = 0; round * PW < nchains; ++round) {
                const int ch = round * PW + ((round & 1) ? PW - 1 - wv : wv);
                if (ch >= nchains)
                    continue;
                const int bp = ch / nh, hh = ch % nh;
                const float *Nh = Nm + hh * C * LDF;
                float *Th = Tf + hh * C * LDF;
                static_for<RT - 1>([&](auto bpc) {
                    constexpr int BP = decltype(bpc)::value;
                    if (BP != bp)
                        return;
                    f32x4 tb[RT];
                    if constexpr (COLT) {
                        tb[BP] = *reinterpret_cast<const f32x4 *>(Th + tix(BP * 16 + g4, BP * 16 + r16));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            tb[BP][i] = Th[tix(BP * 16 + g4 + i, BP * 16 + r16)];
                    }
                    static_for<RT - 1 - BP>([&](auto dc) {
                        constexpr int B = BP + 1 + decltype(dc)::value;
                        f32x4 y = zero4();
                        static_for<B - BP>([&](auto mc) {
                            constexpr int M = BP + decltype(mc)::value;
                            const f32x4 av = *reinterpret_cast<const f32x4 *>(Nh + (B * 16 + r16) * LDF + M * 16 + g4);
#pragma unroll
                            for (int st = 0; st < 4; ++st)
                                y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], tb[M][st], y, 0, 0, 0);
                        });
                        f32x4 dv;   // row r16 of D_B, columns g4 .. g4 + 3
                        if constexpr (COLT) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                dv[i] = Th[tix(B * 16 + r16, B * 16 + g4 + i)];
                        } else {
                            dv = *reinterpret_cast<const f32x4 *>(Th + tix(B * 16 + r16, B * 16 + g4));
                        }
                        f32x4 t = zero4();
#pragma unroll
                        for (int st = 0; st < 4; ++st)
                            t = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[st], y[st], t, 0, 0, 0);
                        tb[B] = -t;
                        if constexpr (COLT) {
                            *reinterpret_cast<f32x4 *>(Th + tix(B * 16 + g4, BP * 16 + r16)) = tb[B];
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                Th[tix(B * 16 + g4 + i, BP * 16 + r16)] = tb[B][i];
                        }
                    });
                });
            }
            __syncthreads();
        }

        if constexpr (TFORM) {
            // T as hi/lo fragment units (see tform_unit): task = (unit, position); the 8
            // columns of a row come from the column-major T, with the blocks above the
            // diagonal (stale LDS) cleared
            static_assert(HB == 1 && RT == 4, "one value head, chunk 64");
            bf16 *tout = tmat + (slot * hv + hfirst + hb) * (2 * kTUnits * 512);
            for (int task = tid; task < kTUnits * kWave; task += NT) {
                const int u = task / kWave, pos = task % kWave;
                const int rt = u < 2 ? u : 2 + (u - 2) / 2, st = u < 2 ? 0 : (u - 2) % 2;
                const int t = Chain<Mma<bf16>>::row(rt, pos % 16), j0 = 32 * st + 8 * (pos / 16);
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = ((j0 + e) >> 4) <= (t >> 4) ? Tf[tix(t, j0 + e)] : 0.f;
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u32x2 pr = split_bf16x2(v[2 * e], v[2 * e + 1]);
                    hi[e] = pr[0];
                    lo[e] = pr[1];
                }
                *reinterpret_cast<u32x4 *>(tout + u * 512 + pos * 8) = hi;
                *reinterpret_cast<u32x4 *>(tout + (kTUnits + u) * 512 + pos * 8) = lo;
            }
            __syncthreads();
            continue;
        }
        if constexpr (ABSORB) {
            absorb_products<C, DK, PW, HB, NKEEP>(Ks, Tf, Nm, Gw[wv], akeep, nh, wv, lane,
                                                  tmat + (slot * hv + hfirst + hb) * DK * C,
                                                  amat + (slot * hv + hfirst + hb) * C * C);
            __syncthreads();
            continue;
        }
        // T to global, zero above the diagonal blocks.
        for (int idx = tid; idx < nh * C * C / VN; idx += NT) {
            const int hh = idx / (C * C / VN);
            const int rem = (idx - hh * (C * C / VN)) * VN;
            const int t = rem / C, j0 = rem - (rem / C) * C;
            const int h = hfirst + hb + hh;
            V16 tv;
#pragma unroll
            for (int e4 = 0; e4 < VN; e4 += 4) {
                const f32x4 tf = *reinterpret_cast<const f32x4 *>(Tf + (hh * C + t) * LDF + j0 + e4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    tv[e4 + e] = (E)((((j0 + e4 + e) >> 4) <= (t >> 4)) ? tf[e] : 0.f);
            }
            *reinterpret_cast<V16 *>(tmat + (slot * hv + h) * C * C + rem) = tv;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Scan kernel.  One workgroup per (sequence, value head, dv-slice of DVS =
// 16 NW columns), NW waves; wave w owns the 16 columns 16 w .. 16 w + 15 of
// the slice.  The dv columns of S evolve independently (each column of the
// state only ever meets the same column of v), so the waves never exchange
// data: each runs the whole chunk step on its own columns, with its fp32
// state columns held in matrix-core accumulators for the whole sequence.
// Per chunk the wave computes, on its columns,
//   [Q;K] S,  X = diag(beta)(V - diag(exp G) K S),  D = T X,
//   O = scale (diag(exp G) Q S + A D),  S <- exp(G_last) S + K^T diag(lambda) D
// entirely in registers (see Chain below): nothing but the staged chunk
// inputs goes through LDS, and the only barrier per chunk is the one that
// hands over the next chunk's stage buffer.
//
// Staging: while computing chunk c from one of two LDS stage buffers, the
// waves load chunk c + 1 (Q, K, T, A, the V slice, the decay record) into
// registers and store it into the other buffer after their compute.  Rows
// past the end of a sequence are loaded from its last row: every term they
// feed is multiplied by beta = 0 (their rows of X and D are zero) or by a
// zero column of A.  Within a staged row the 16-byte chunks are permuted
// (Swz) to spread the 16-row operand reads and the 4-row transpose reads over
// the LDS banks (measured rates at Swz).
//
// The S update contracts over the chunk index, so it needs K^T as a matrix
// operand: with bf16 it is read from the row-major K tile with the LDS
// transpose read (ds_read_b64_tr_b16: in every group of 16 lanes, input lane
// 4 e + q reads 4 consecutive elements of row e, and output lane j receives
// element j % 4 of input lane j / 4's read for each of the 4 rows); with fp32
// every lane reads its single element.
//
// Block index -> work (xcd_group): the value heads of one (sequence, query/key
// head) and all their dv slices are placed on one XCD, so that their shared Q
// and K reads (and a head's W and M, read by each of its slices) hit the same
// L2.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Tiles read in the row order of the 32-wide chain below: a 16-lane operand
// read takes rows r0 + 8 a + b (a, b < 4, r0 a multiple of 4), and the
// transpose read of K takes rows 8 g + e (e < 4) in 16-byte chunks 4 a + q
// (q < 4).  These chunk permutations put both patterns on distinct 16-byte
// bank groups of the plain modulo bank model (for 256-, 128- and 64-byte rows);
// measured rates at Swz.
template <int RB>
struct SwzChain {
    static_assert(RB == 64 || RB == 128 || RB == 256, "rows of 64, 128 or 256 bytes");
    __device__ static inline int perm(int r)
    {
        if constexpr (RB == 256)
            return ((r & 3) << 2) | ((r >> 3) & 3);
        else if constexpr (RB == 128)
            return (((r >> 1) & 1) << 2) | ((r >> 3) & 3);
        else
            return (r >> 3) & 3;
    }
    __device__ static inline int off(int r, int b) { return r * RB + ((((b >> 4) ^ perm(r)) << 4) | (b & 15)); }
};

// A operand of the S update: K^T, output rows = key indices in the order
// Chain<MK>::row(sr, .), contraction over chunk rows in the order of
// Chain<MC> (MK, MC: the instructions of the key and chunk contractions).
template <typename E, typename MC, typename MK, typename S>
struct KtOperand;

template <typename MC, typename MK, typename S>
struct KtOperand<bf16, MC, MK, S> {
    __device__ static inline typename MC::frag load(const unsigned char *Kb, int sr, int s, int lane)
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, qd = lane & 3;
        // input lane (e, qd) reads 4 consecutive key indices: output lanes 4 qd .. 4 qd + 3
        // receive them, i.e. rows Chain<MK>::row(sr, 4 qd + {0..3}) of the output tile
        const int b = 2 * Chain<MK>::row(sr, 4 * qd);
        if constexpr (MC::kPerLane == 8) {
            const int r0 = 32 * s + 8 * g + e;
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(r0, b)));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(r0 + 4, b)));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        } else {
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(Kb + S::off(16 * s + 4 * g + e, b)));
            return __builtin_bit_cast(bf16x4, lo);
        }
    }
};

template <typename MC, typename MK, typename S>
struct KtOperand<float, MC, MK, S> {
    __device__ static inline float load(const unsigned char *Kb, int sr, int s, int lane)
    {
        const int c = Chain<MC>::a_col(s, lane);
        return *reinterpret_cast<const float *>(Kb + S::off(c, 4 * Chain<MK>::row(sr, lane & 15)));
    }
};

// Orders this wave's LDS accesses before and after it (lanes of one wave).
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Absorbed form of the chunk matrices (see AbsorbedForm), run by the prep after the
// solve: T (fp32, [HB][C][LDF], column j at j LDF) is complete in Tf, K is still staged in Ks (Swz rows),
// and each wave holds its A tiles (fp32) in akeep, dealt as the Gram tiles were.
// Wave wv owns value head hh = wv / (C / 16) of the pass and block column jb = wv % (C / 16)
// of its T: the fp32 values, and those of diag(lambda) T, become hi/lo bf16 operand pairs, and
//   W^T (rows t of block jb, columns i) = (diag(lambda) T)^T K      (two products per step)
//   M^T (rows j of block jb, columns t) = T^T A^T                   (three: hi hi, hi lo, lo hi)
// are formed transposed (each lane holds four consecutive elements of one row of W or M)
// and written out as whole rows through LDS.  M is zero above its diagonal blocks, written
// as such.  A goes to the N region
// (which the solve no longer reads) as a hi and a lo bf16 matrix, C rows of C elements in
// the Swz chunk order, so that each operand fragment of A^T is one 16-byte read.
template <int C, int DK, int PW, int HB, int NKEEP>
__device__ void absorb_products(const unsigned char *Ks, const float *Tf, float *Am, float (*Gv)[C],
                                f32x4 (&akeep)[NKEEP][HB], int nh, int wv, int lane, bf16 *wout, bf16 *mout)
{
    constexpr int LDF = C + 4, RT = C / 16, NS = C / 32;
    typedef Mma<bf16> M;
    typedef KtOperand<bf16, M, MmaBf16K16, Swz<DK * 2>> KT;
    typedef Swz<C * 2> SA;
    constexpr int TILE_BYTES = C * DK * 2;   // the staged k rows (T follows them)
    static_assert(C % 32 == 0 && DK % 16 == 0, "32-wide chunk steps, 16-row key tiles");
    static_assert(HB * 2 * C * C * 2 <= HB * C * LDF * 4, "hi and lo A fit the N region");
    const int r16 = lane & 15, G = lane >> 4;
    unsigned char *const Ab = reinterpret_cast<unsigned char *>(Am);   // [HB][hi | lo][C rows of 2 C bytes]

    // A as hi/lo bf16 into the N region; tiles above the diagonal as zeros (the deal of the
    // Gram tiles decides which wave writes what)
    static_for<RT * RT>([&](auto pc) {
        constexpr int P = decltype(pc)::value;
        constexpr int tr = P / RT, tc = P % RT;
        constexpr bool lower = tc <= tr;
        constexpr int idx = lower ? tr * (tr + 1) / 2 + tc : (tr * RT + tc) + 2;
        if (idx % PW != wv)
            return;
        const int t = tr * 16 + r16, j0 = tc * 16 + 4 * G;
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            if (hh >= nh)
                break;
            f32x4 v = zero4();
            if constexpr (lower)
                v = akeep[idx / PW][hh];
            const u32x2 p0 = split_bf16x2(v[0], v[1]), p1 = split_bf16x2(v[2], v[3]);
            unsigned char *base = Ab + hh * 2 * C * C * 2;
            *reinterpret_cast<u32x2 *>(base + SA::off(t, 2 * j0)) = u32x2{p0[0], p1[0]};
            *reinterpret_cast<u32x2 *>(base + C * C * 2 + SA::off(t, 2 * j0)) = u32x2{p0[1], p1[1]};
        }
    });
    __syncthreads();

    const int hh = wv / RT, jb = wv % RT, j = 16 * jb + r16;
    f32x4 wres[DK / 16], mres[RT];
    if (hh < nh) {
        const float *Th = Tf + hh * C * LDF;
        const unsigned char *Ahi = Ab + hh * 2 * C * C * 2, *Alo = Ahi + C * C * 2;
        // lambda_m = exp(G_last - G_m) over this wave's own copy of G (read back by itself)
        {
            const float lam = __expf(Gv[hh][C - 1] - Gv[hh][lane & (C - 1)]);
            wave_lds_sync();
            if (lane < C)
                Gv[hh][lane] = lam;
            wave_lds_sync();
        }
        // column j of T (zero above the diagonal blocks) and of diag(lambda) T, contraction
        // rows 32 s + 8 G + {0..7}, as hi/lo pairs
        bf16x8 thi[NS], tlo[NS], lhi[NS], llo[NS];
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const f32x4 l0 = *reinterpret_cast<const f32x4 *>(&Gv[hh][32 * st + 8 * G]);
            const f32x4 l1 = *reinterpret_cast<const f32x4 *>(&Gv[hh][32 * st + 8 * G + 4]);
            // rows 32 st + 8 G .. + 7 of column j (consecutive in Tf); rows above the diagonal
            // blocks hold stale data and are cleared by a mask (the reads stay unconditional)
            const uint32_t keep = ((2 * st + (G >> 1)) >= jb) ? 0xffffffffu : 0u;
            const u32x4 m0 = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4 *>(Th + j * LDF + 32 * st + 8 * G)) & keep;
            const u32x4 m1 = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4 *>(Th + j * LDF + 32 * st + 8 * G + 4)) & keep;
            const f32x4 t0 = __builtin_bit_cast(f32x4, m0), t1 = __builtin_bit_cast(f32x4, m1);
            const f32x4 v0 = t0 * l0, v1 = t1 * l1;
            u32x4 th, tl, lh, ll;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 &tq = q < 2 ? t0 : t1;
                const f32x4 &vq = q < 2 ? v0 : v1;
                const u32x2 a = split_bf16x2(tq[2 * (q & 1)], tq[2 * (q & 1) + 1]);
                const u32x2 b = split_bf16x2(vq[2 * (q & 1)], vq[2 * (q & 1) + 1]);
                th[q] = a[0];
                tl[q] = a[1];
                lh[q] = b[0];
                ll[q] = b[1];
            }
            thi[st] = __builtin_bit_cast(bf16x8, th);
            tlo[st] = __builtin_bit_cast(bf16x8, tl);
            lhi[st] = __builtin_bit_cast(bf16x8, lh);
            llo[st] = __builtin_bit_cast(bf16x8, ll);
        }
        // W^T tiles (rows t of block jb, columns i of key block it): lane holds
        // W[16 it + l % 16][16 jb + 4 G .. + 3]
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
            f32x4 acc = zero4();
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const bf16x8 kf = KT::load(Ks, it, st, lane);
                acc = M::mma(lhi[st], kf, acc);
                acc = M::mma(llo[st], kf, acc);
            }
            wres[it] = acc;
        }
        // M^T tiles (rows j of block jb, columns t of block tt): lane holds
        // M[16 tt + l % 16][16 jb + 4 G .. + 3]; zero for tt < jb
#pragma unroll
        for (int tt = 0; tt < RT; ++tt) {
            f32x4 acc = zero4();
            if (tt >= jb) {
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const int off = SA::off(16 * tt + r16, 64 * st + 16 * G);
                    const bf16x8 ahi = *reinterpret_cast<const bf16x8 *>(Ahi + off);
                    const bf16x8 alo = *reinterpret_cast<const bf16x8 *>(Alo + off);
                    acc = M::mma(thi[st], ahi, acc);
                    acc = M::mma(thi[st], alo, acc);
                    acc = M::mma(tlo[st], ahi, acc);
                }
            }
            mres[tt] = acc;
        }
    }
    // W and M to global memory as whole rows: through LDS (K, T and A are dead once every
    // wave has passed the barrier), rows padded to 2 C + 16 bytes so that the 16 rows of a
    // tile fall on distinct banks, then 16-byte stores of consecutive lanes along each row
    __syncthreads();
    constexpr int LDW = C + 8;   // padded row, elements
    static_assert(DK * LDW * 2 <= TILE_BYTES + HB * C * LDF * 4, "W rows fit the k and T regions");
    static_assert(HB * C * LDW * 2 <= HB * C * LDF * 4, "M rows fit the N region");
    bf16 *Wl = reinterpret_cast<bf16 *>(const_cast<unsigned char *>(Ks));   // [DK][LDW], over k and T
    bf16 *Ml = reinterpret_cast<bf16 *>(Am);                                // [C][LDW], over A
    if (hh < nh) {
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
            *reinterpret_cast<bf16x4 *>(Wl + (16 * it + r16) * LDW + 16 * jb + 4 * G) =
                bf16x4{(bf16)wres[it][0], (bf16)wres[it][1], (bf16)wres[it][2], (bf16)wres[it][3]};
#pragma unroll
        for (int tt = 0; tt < RT; ++tt)
            *reinterpret_cast<bf16x4 *>(Ml + (16 * tt + r16) * LDW + 16 * jb + 4 * G) =
                bf16x4{(bf16)mres[tt][0], (bf16)mres[tt][1], (bf16)mres[tt][2], (bf16)mres[tt][3]};
    }
    __syncthreads();
    static_assert(HB == 1, "one value head per pass in the absorbed form");
    if (nh > 0) {
        constexpr int CPR = C * 2 / 16;              // 16-byte pieces per row
        constexpr int RPI = PW * kWave / CPR;        // rows per pass of the workgroup
        static_assert(DK % RPI == 0 && C % RPI == 0, "whole passes over W and M");
        const int r0 = wv * (kWave / CPR) + lane / CPR, qp = lane % CPR;
        char *wb = reinterpret_cast<char *>(wout), *mb = reinterpret_cast<char *>(mout);
        static_for<DK / RPI>([&](auto ic) {
            const int row = decltype(ic)::value * RPI + r0;
            *reinterpret_cast<bf16x8 *>(wb + (uint32_t)(row * C + qp * 8) * 2u) =
                *reinterpret_cast<const bf16x8 *>(Wl + row * LDW + qp * 8);
        });
        static_for<C / RPI>([&](auto ic) {
            const int row = decltype(ic)::value * RPI + r0;
            *reinterpret_cast<bf16x8 *>(mb + (uint32_t)(row * C + qp * 8) * 2u) =
                *reinterpret_cast<const bf16x8 *>(Ml + row * LDW + qp * 8);
        });
    }
}


template <typename E, int C, int DK, int NW>
__global__ __launch_bounds__(NW * kWave) void gdn_chunk_scan_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v, const int32_t *__restrict__ cu,
    SlotMap map, int32_t num_seqs, int64_t total_tokens, int32_t hqk, int32_t hv, int32_t dv,
    const E *__restrict__ tmat, const E *__restrict__ amat, const float *__restrict__ dec, const float *state_in,
    float *state_out, E *__restrict__ o, float scale)
{
    constexpr int DVS = 16 * NW;
    constexpr int NT = NW * kWave;
    constexpr int ES = (int)sizeof(E);
    constexpr int RT = C / 16, SR = DK / 16;
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;
    typedef typename MmaFor<E, C>::type MC;     // contractions over the chunk rows
    typedef typename MmaFor<E, DK>::type MK;    // contractions over the key index
    typedef Chain<MC> CC;
    typedef Chain<MK> CK;
    // Q and A are read in natural row order; K and T in the row order of CC (and K
    // also by the transpose read).
    constexpr bool kChain32 = MC::kPerLane == 8;
    typedef Swz<DK * ES> SQ;
    typedef typename std::conditional<kChain32, SwzChain<DK * ES>, Swz<DK * ES>>::type SK;
    typedef typename std::conditional<kChain32, SwzChain<C * ES>, Swz<C * ES>>::type ST;
    typedef Swz<C * ES> SA;
    typedef Swz<DVS * ES> SV;
    typedef KtOperand<E, MC, MK, SK> KT;
    constexpr int NSK = DK / MK::kStep;   // steps along the key index
    constexpr int NSC = C / MC::kStep;    // steps along the chunk rows
    static_assert(C <= kWave, "one lane per token of a chunk");
    static_assert(DK % 32 == 0 || sizeof(E) == 4, "bf16 key contractions use 32-wide steps");

    // stage buffer layout (bytes) and its 1 KB load jobs (64 lanes x 16 bytes)
    constexpr int OFF_Q = 0;
    constexpr int OFF_K = OFF_Q + C * DK * ES;
    constexpr int OFF_T = OFF_K + C * DK * ES;
    constexpr int OFF_A = OFF_T + C * C * ES;
    constexpr int OFF_V = OFF_A + C * C * ES;
    constexpr int OFF_D = OFF_V + C * DVS * ES;
    constexpr int STAGE = OFF_D + 4 * C * 4;
    constexpr int NCK_QK = C * DK * ES / 16;   // 16-byte chunks per tile
    constexpr int NCK_TA = C * C * ES / 16;
    constexpr int NCK_V = C * DVS * ES / 16;
    constexpr int NCK_D = 4 * C * 4 / 16;
    constexpr int NJ_QK = (NCK_QK + 63) / 64;
    constexpr int NJ_TA = (NCK_TA + 63) / 64;
    constexpr int NJ_V = (NCK_V + 63) / 64;
    constexpr int NJ_D = (NCK_D + 63) / 64;
    constexpr int J_T = 2 * NJ_QK, J_V = J_T + 2 * NJ_TA, J_D = J_V + NJ_V;
    constexpr int NJ = J_D + NJ_D;
    constexpr int NJ_PER = (NJ + NW - 1) / NW;

    __shared__ __attribute__((aligned(1024))) unsigned char stage_mem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) E Os[NW][C * 16];   // each wave's output columns

    // the stage buffers as LDS addresses (the direct loads write LDS by address)
    __attribute__((address_space(3))) unsigned char *const lds_stage =
        (__attribute__((address_space(3))) unsigned char *)stage_mem;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int r16 = lane & 15, g4 = 4 * (lane >> 4);
    const int nv = dv / DVS;
    const int pairs = num_seqs * hv;
    // item = (sequence rank, query/key head); its members are the group's value heads
    // times their column slices
    const int group = hv / hqk;
    int item, member;
    xcd_group(blockIdx.x, group * nv, item, member);
    const int pair = item * group + member / nv;
    const int s = member % nv;
    if (pair >= pairs)
        return;
    const int n = ranked_sequence(map, pair / hv), h = pair - (pair / hv) * hv;
    const int hq = h / (hv / hqk);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int nch = seq_chunks(map, cu, n, total_tokens, C);
    const int c_begin = map.seg_first;
    const int c_end = min(nch, map.seg_first + map.seg_len);
    const int col = s * DVS + 16 * w + r16;            // this lane's state / output column
    const size_t state_base = (size_t)(n * hv + h) * DK * dv;
    if (c_begin >= c_end) {
        // No chunk of this sequence in this launch.  The first launch still owes the
        // sequence its final state (initial state passed through, or zeros).
        if (c_begin == 0 && state_in != state_out) {
            for (int i = tid; i < DK * DVS; i += NT) {
                const size_t off = state_base + (size_t)(i / DVS) * dv + s * DVS + (i % DVS);
                state_out[off] = state_in ? state_in[off] : 0.f;
            }
        }
        return;
    }

    // ---- state columns into accumulators: tile sr, slot i holds key row CK::row(sr, g4 + i) ----
    f32x4 sacc[SR];
#pragma unroll
    for (int sr = 0; sr < SR; ++sr) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sacc[sr][i] = state_in ? state_in[state_base + (size_t)CK::row(sr, g4 + i) * dv + col] : 0.f;
    }
    typename MK::frag sb[NSK];   // B fragments of S for [Q;K] S
#pragma unroll
    for (int st = 0; st < NSK; ++st)
        sb[st] = CK::b_frag(sacc, st);

    // ---- staging ----
    // Job J (of NJ) moves 1 KB of the stage with one direct-to-LDS load: lane i writes
    // the 16 bytes at 16 i of the job's block.  Wave w runs jobs w, w + NW, ...; which
    // tile and rows a job covers is fixed at compile time, so each lane's source offset
    // (elements from the chunk's first row, for a full chunk) is computed once.
    const int qk_row = hqk * DK, v_row = hv * dv;
    auto job_row = [&](auto jc) __attribute__((always_inline)) -> int {   // source row of this lane
        constexpr int J = decltype(jc)::value;
        if constexpr (J < J_T) {
            return (((J % NJ_QK) * 64 + lane) / (DK * ES / 16));
        } else if constexpr (J < J_V) {
            return min(((J - J_T) % NJ_TA) * 64 + lane, NCK_TA - 1) / (C * ES / 16);
        } else if constexpr (J < J_D) {
            return min((J - J_V) * 64 + lane, NCK_V - 1) / (DVS * ES / 16);
        } else {
            return 0;
        }
    };
    // element offset of this lane's 16 bytes from the tile's origin, given its source row
    auto job_off = [&](auto jc, int row) __attribute__((always_inline)) -> int {
        constexpr int J = decltype(jc)::value;
        if constexpr (J < J_T) {
            const int P = (J % NJ_QK) * 64 + lane;
            const int r = P / (DK * ES / 16), pos = P % (DK * ES / 16);
            const int j = pos ^ (J >= NJ_QK ? SK::perm(r) : SQ::perm(r));
            return row * qk_row + j * VN;
        } else if constexpr (J < J_V) {
            const int P = min(((J - J_T) % NJ_TA) * 64 + lane, NCK_TA - 1);
            const int r = P / (C * ES / 16), pos = P % (C * ES / 16);
            const int j = pos ^ ((J - J_T) >= NJ_TA ? SA::perm(r) : ST::perm(r));
            return r * C + j * VN;
        } else if constexpr (J < J_D) {
            const int P = min((J - J_V) * 64 + lane, NCK_V - 1);
            const int r = P / (DVS * ES / 16), pos = P % (DVS * ES / 16);
            const int j = pos ^ SV::perm(r);
            return row * v_row + j * VN;
        } else {
            return min((J - J_D) * 64 + lane, NCK_D - 1) * 4;   // floats
        }
    };
    int loff[NJ_PER];   // per-lane source offsets of this wave's jobs, full chunks
    auto init_offsets = [&](auto wc) __attribute__((always_inline)) {
        constexpr int W = decltype(wc)::value;
        static_for<NJ_PER>([&](auto uc) {
            constexpr int J = W + decltype(uc)::value * NW;
            if constexpr (J < NJ)
                loff[decltype(uc)::value] = job_off(std::integral_constant<int, J>{},
                                                    job_row(std::integral_constant<int, J>{}));
        });
    };
    // Stage chunk c into buffer BUF.  `last` is the index of the chunk's last real row;
    // rows past it are loaded from it.
    auto issue_jobs = [&](auto wc, auto bufc, int c) __attribute__((always_inline)) {
        constexpr int W = decltype(wc)::value;
        __attribute__((address_space(3))) unsigned char *stg = lds_stage + decltype(bufc)::value * STAGE;
        const int64_t t0 = a + (int64_t)c * C;
        const int last = (int)min<int64_t>(C, b - t0) - 1;
        const size_t slot = slot_of(map, n, c);
        const E *qb = q + ((size_t)t0 * hqk + hq) * DK;
        const E *kb = k + ((size_t)t0 * hqk + hq) * DK;
        const E *vb = v + ((size_t)t0 * hv + h) * dv + (size_t)s * DVS;
        const E *tb = tmat + (slot * hv + h) * C * C;
        const E *ab = amat + (slot * hv + h) * C * C;
        const E *db = reinterpret_cast<const E *>(dec + (slot * hv + h) * 4 * C);
        const bool full = last == C - 1;
        static_for<NJ_PER>([&](auto uc) {
            constexpr int U = decltype(uc)::value;
            constexpr int J = W + U * NW;
            if constexpr (J < NJ) {
                constexpr std::integral_constant<int, J> jc{};
                const E *base;
                int off = loff[U];
                if constexpr (J < J_T) {
                    base = J >= NJ_QK ? kb : qb;
                    if (!full)
                        off = job_off(jc, min(job_row(jc), last));
                } else if constexpr (J < J_V) {
                    base = (J - J_T) >= NJ_TA ? ab : tb;
                } else if constexpr (J < J_D) {
                    base = vb;
                    if (!full)
                        off = job_off(jc, min(job_row(jc), last));
                } else {
                    base = db;
                    off *= (int)(sizeof(float) / sizeof(E));
                }
                // lanes of the job that carry data, and the job's block in the stage
                constexpr int NCK = J < J_T ? NCK_QK : J < J_V ? NCK_TA : J < J_D ? NCK_V : NCK_D;
                constexpr int IDX = J < J_T ? J % NJ_QK : J < J_V ? (J - J_T) % NJ_TA : J < J_D ? J - J_V : J - J_D;
                constexpr int NL = NCK - IDX * 64 < 64 ? NCK - IDX * 64 : 64;
                constexpr int BLK = (J < J_T ? (J >= NJ_QK ? OFF_K : OFF_Q)
                                             : J < J_V ? ((J - J_T) >= NJ_TA ? OFF_A : OFF_T)
                                                       : J < J_D ? OFF_V : OFF_D) + IDX * 1024;
                if (NL == 64 || lane < NL)
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                     (__attribute__((address_space(3))) void *)(stg + BLK), 16, 0, 0);
            }
        });
    };
    auto by_wave = [&](auto fn) __attribute__((always_inline)) {
        if constexpr (NW == 2) {
            if (w == 0) fn(std::integral_constant<int, 0>{});
            else fn(std::integral_constant<int, 1>{});
        } else {
            static_assert(NW == 4, "2 or 4 waves");
            switch (w) {
            case 0: fn(std::integral_constant<int, 0>{}); break;
            case 1: fn(std::integral_constant<int, 1>{}); break;
            case 2: fn(std::integral_constant<int, 2>{}); break;
            default: fn(std::integral_constant<int, 3>{}); break;
            }
        }
    };
    by_wave([&](auto wc) { init_offsets(wc); });
    auto issue_stage = [&](auto bufc, int c) __attribute__((always_inline)) {
        by_wave([&](auto wc) { issue_jobs(wc, bufc, c); });
    };
    // The direct loads are not tracked by the compiler's LDS dependences: wait for
    // them (and this wave's stores) explicitly before the barrier that publishes them.
    auto stage_done = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // ---- one chunk step of this wave's 16 columns on stage buffer BUF ----
    // Operand fragments are read from LDS one group of products ahead of their
    // use; the scheduling barriers keep the compiler from sinking each read next
    // to its product, where every product would wait out a full LDS latency.
    E *os = Os[w];
    auto step = [&](auto bufc, int64_t t0, int len) __attribute__((always_inline)) {
        const unsigned char *stg = stage_mem + decltype(bufc)::value * STAGE;
        const float *Gs = reinterpret_cast<const float *>(stg + OFF_D);   // exp(G)
        const float *Lam = Gs + C;                                         // exp(G_last - G)
        const float *Bet = Gs + 2 * C;                                     // beta
        const float *BGam = Gs + 3 * C;                                    // beta exp(G)
        typedef typename MK::frag FK;
        typedef typename MC::frag FC;

        // [Q;K] S.  Q rows in natural order (O tiles are only stored); K rows in the
        // order of CC, since X = f(K S) is the B operand of T X.
        FK fq[2][RT], fk[2][RT];
        auto load_qk = [&](int bsel, int st) __attribute__((always_inline)) {
            const int kc = CK::a_col(st, lane);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                fq[bsel][rt] = staged_frag<MK, SQ, E>(stg + OFF_Q, 16 * rt + r16, kc);
                fk[bsel][rt] = staged_frag<MK, SK, E>(stg + OFF_K, CC::row(rt, r16), kc);
            }
        };
        load_qk(0, 0);
        // X = beta V - beta exp(G) (K S) on this lane's rows
        float xp[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = CC::row(rt, g4 + i);
                xp[rt][i] = Bet[c] * to_f32(*reinterpret_cast<const E *>(stg + OFF_V + SV::off(c, (16 * w + r16) * ES)));
            }
        }
        f32x4 qacc[RT], xacc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            qacc[rt] = zero4();
            xacc[rt] = zero4();
        }
#pragma unroll
        for (int st = 0; st < NSK; ++st) {
            if (st + 1 < NSK)
                load_qk((st + 1) & 1, st + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                qacc[rt] = MK::mma(fq[st & 1][rt], sb[st], qacc[rt]);
                xacc[rt] = MK::mma(fk[st & 1][rt], sb[st], xacc[rt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // T fragments (rows in the order of CC: D feeds A D and the S update)
        FC ft[NSC][RT];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                ft[st][rt] = staged_frag<MC, ST, E>(stg + OFF_T, CC::row(rt, r16), CC::a_col(st, lane));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xacc[rt][i] = xp[rt][i] - BGam[CC::row(rt, g4 + i)] * xacc[rt][i];
        FC xb[NSC];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
            xb[st] = CC::b_frag(xacc, st);

        // K^T fragments of the S update
        FC fkt[SR][NSC];
#pragma unroll
        for (int sr = 0; sr < SR; ++sr)
#pragma unroll
            for (int st = 0; st < NSC; ++st)
                fkt[sr][st] = KT::load(stg + OFF_K, sr, st, lane);
        __builtin_amdgcn_sched_barrier(0);

        // D = T X
        f32x4 dacc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            dacc[rt] = zero4();
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                dacc[rt] = MC::mma(ft[st][rt], xb[st], dacc[rt]);
        __builtin_amdgcn_sched_barrier(0);

        // A fragments of the output product (A carries the output scale)
        FC fa[NSC][RT];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                fa[st][rt] = staged_frag<MC, SA, E>(stg + OFF_A, 16 * rt + r16, CC::a_col(st, lane));
        __builtin_amdgcn_sched_barrier(0);

        FC db[NSC], lb[NSC];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
            db[st] = CC::b_frag(dacc, st);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dacc[rt][i] *= Lam[CC::row(rt, g4 + i)];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
            lb[st] = CC::b_frag(dacc, st);

        // S <- exp(G_last) S + K^T (diag(lambda) D)
        const float gl = Gs[C - 1];   // exp(G_last): G is flat past the last real token
#pragma unroll
        for (int sr = 0; sr < SR; ++sr) {
            sacc[sr] = sacc[sr] * gl;
#pragma unroll
            for (int st = 0; st < NSC; ++st)
                sacc[sr] = MC::mma(fkt[sr][st], lb[st], sacc[sr]);
        }
#pragma unroll
        for (int st = 0; st < NSK; ++st)
            sb[st] = CK::b_frag(sacc, st);

        // O = scale diag(exp G) Q S + (scale A) D, natural row order
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qacc[rt][i] *= scale * Gs[16 * rt + g4 + i];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                qacc[rt] = MC::mma(fa[st][rt], db[st], qacc[rt]);
        // this wave's 16 output columns: through its own LDS rows to 16-byte stores
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                os[(16 * rt + g4 + i) * 16 + r16] = (E)qacc[rt][i];
        wave_lds_sync();
        constexpr int RV = 16 / VN;   // 16-byte vectors per row of 16 columns
        for (int idx = lane; idx < C * RV; idx += kWave) {
            const int r = idx / RV, cv = (idx % RV) * VN;
            if (r < len)
                *reinterpret_cast<V16 *>(o + ((size_t)(t0 + r) * hv + h) * dv + (size_t)s * DVS + 16 * w + cv) =
                    *reinterpret_cast<const V16 *>(os + r * 16 + cv);
        }
        wave_lds_sync();
    };

    // ---- pipeline: one barrier per chunk; chunk c_begin + 2 m uses buffer 0, the
    //      next one buffer 1 (the loop is unrolled by two so that both buffers'
    //      addresses are compile-time offsets) ----
    const std::integral_constant<int, 0> buf0;
    const std::integral_constant<int, 1> buf1;
    issue_stage(buf0, c_begin);
    stage_done();
    for (int c = c_begin;;) {
        if (c + 1 < c_end)
            issue_stage(buf1, c + 1);
        int64_t t0 = a + (int64_t)c * C;
        step(buf0, t0, (int)min<int64_t>(C, b - t0));
        stage_done();
        if (++c >= c_end)
            break;
        if (c + 1 < c_end)
            issue_stage(buf0, c + 1);
        t0 = a + (int64_t)c * C;
        step(buf1, t0, (int)min<int64_t>(C, b - t0));
        stage_done();
        if (++c >= c_end)
            break;
    }

    // ---- final state ----
#pragma unroll
    for (int sr = 0; sr < SR; ++sr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            state_out[state_base + (size_t)CK::row(sr, g4 + i) * dv + col] = sacc[sr][i];
}

// ---------------------------------------------------------------------------
// Scan kernel for few (sequence, head) pairs (bf16 io, chunk 64): one chunk
// step is spread over 4 compute waves by chunk rows (and key rows for the S
// update), exchanging X, D and the transposed bf16 copy of S through LDS, and
// storing the chunk's outputs straight from registers; 4 loader waves stage
// the chunks ahead of the compute waves: two steps ahead with three stage
// buffers for dk = 128, one step ahead with two for smaller dk (whose two
// buffers leave room for two workgroups per CU).  With few pairs the chip has
// more CUs than workgroups and the chain of chunk steps is latency-bound, which
// this split shortens.  (Wide batches use gdn_chunk_scan_bf16_kernel.)
// ---------------------------------------------------------------------------
// LDS row stride (elements) of the padded key-dimension tile St.  In dwords it
// is a multiple of 4 with an odd quotient, so 16 rows read with 16-byte
// accesses fall on 16 distinct bank groups of the plain modulo bank model
// (measured at half the lane-order rate: see Swz).
template <typename E>
constexpr int key_row_stride(int dk)
{
    const int dw = dk * (int)sizeof(E) / 4;
    for (int s = (dw + 3) / 4 * 4;; s += 4)
        if ((s / 4) % 2 == 1)
            return s * 4 / (int)sizeof(E);
}

constexpr int kScanThreads = 2 * kThreads;   // 4 compute waves + 4 loader waves

template <typename E, int C, int DK, int DVS, int NSTAGE>
__global__ __launch_bounds__(kScanThreads) void gdn_chunk_scan_rows_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v, const int32_t *__restrict__ cu,
    SlotMap map, int32_t num_seqs, int64_t total_tokens, int32_t hqk, int32_t hv, int32_t dv,
    const E *__restrict__ wmat, const E *__restrict__ mmat, const float *__restrict__ dec, const float *state_in,
    float *state_out, E *__restrict__ o, float scale)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int PAD = LdsPad<E>::value;
    constexpr int LDK = key_row_stride<E>(DK);
    constexpr int LDC = C + PAD;
    constexpr int RT = C / 16, CT = DVS / 16, SR = DK / 16;
    constexpr int SR_PER = (SR + kWaves - 1) / kWaves;
    constexpr int RT_PER = (RT + kWaves - 1) / kWaves;
    constexpr int VN = Vec16<E>::n;
    typedef typename MmaFor<E, C>::type MC;
    typedef typename MmaFor<E, DK>::type MK;
    typedef Swz<DK * ES> SK;
    typedef Swz<C * ES> SC;
    typedef Swz<DVS * ES> SV;
    static_assert(C <= kWave, "one lane per token of a chunk");
    static_assert(DVS % 16 == 0 && DK % 16 == 0 && C % 16 == 0, "16x16 tiles");

    // Stage buffers (bytes) and the 1 KB direct-to-LDS load jobs that fill them.  A chunk is
    // staged in two parts: part A, Q, K (C x DK) and the V slice (C x DVS), read only before
    // the step's first barrier; part B, W (DK x C), M (C x C) and the decay record, read
    // through the step.  Part A has NSTAGE buffers (it can be refilled two chunks ahead once
    // the step has passed its first barrier), part B two.
    constexpr int OFF_Q = 0;
    constexpr int OFF_K = OFF_Q + C * DK * ES;
    constexpr int OFF_V = OFF_K + C * DK * ES;
    constexpr int STAGE_A = OFF_V + C * DVS * ES;
    constexpr int OFF_W = 0;
    constexpr int OFF_M = OFF_W + DK * C * ES;
    constexpr int OFF_D = OFF_M + C * C * ES;
    constexpr int STAGE_B = OFF_D + 4 * C * 4;
    constexpr int NCK_QK = C * DK * ES / 16;   // 16-byte chunks per tile
    constexpr int NCK_W = DK * C * ES / 16;
    constexpr int NCK_M = C * C * ES / 16;
    constexpr int NCK_V = C * DVS * ES / 16;
    constexpr int NCK_D = 4 * C * 4 / 16;
    constexpr int NJ_QK = (NCK_QK + 63) / 64;
    constexpr int NJ_W = (NCK_W + 63) / 64;
    constexpr int NJ_M = (NCK_M + 63) / 64;
    constexpr int NJ_V = (NCK_V + 63) / 64;
    constexpr int NJ_D = (NCK_D + 63) / 64;
    constexpr int J_W = 2 * NJ_QK, J_M = J_W + NJ_W, J_V = J_M + NJ_M, J_D = J_V + NJ_V;
    constexpr int NJ = J_D + NJ_D;
    static_assert(STAGE_A % 1024 == 0 && STAGE_B % 16 == 0 && OFF_D % 16 == 0, "16-byte aligned stage blocks");
    static_assert(AbsorbedForm<E, C>::value, "the row-split scan reads the absorbed form");

    // While the compute waves work on chunk c, the loaders fill part B of chunk c + 1 and
    // part A of chunk c + NSTAGE - 1.
    static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three part-A buffers");
    static_assert(NSTAGE * STAGE_A + 2 * STAGE_B + DVS * LDC * ES + DVS * LDK * ES <= 163840,
                  "stage buffers and exchange tiles must fit the 160 KB of LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char stage_a[NSTAGE * STAGE_A];
    __shared__ __attribute__((aligned(1024))) unsigned char stage_b[2 * STAGE_B];
    __shared__ __attribute__((aligned(16))) E Xt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E St[DVS * LDK];

    // the stage buffers as LDS addresses (the direct loads write LDS by address)
    __attribute__((address_space(3))) unsigned char *const lds_a =
        (__attribute__((address_space(3))) unsigned char *)stage_a;
    __attribute__((address_space(3))) unsigned char *const lds_b =
        (__attribute__((address_space(3))) unsigned char *)stage_b;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool loader = wave >= kWaves;              // waves 4..7 stage chunks, 0..3 compute
    const int lw = wave - kWaves;                    // loader index
    const int nv = dv / DVS;
    const int pairs = num_seqs * hv;
    // item = (sequence rank, query/key head); its members are the group's value heads
    // times their column slices
    const int group = hv / hqk;
    int item, member;
    xcd_group(blockIdx.x, group * nv, item, member);
    const int pair = item * group + member / nv;
    const int s = member % nv;
    if (pair >= pairs)
        return;
    const int n = ranked_sequence(map, pair / hv), h = pair - (pair / hv) * hv;
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

    // ---- loaders: part A of chunk c into buffer c % NSTAGE of stage_a, part B into buffer
    //      c % 2 of stage_b (direct-to-LDS loads) ----
    // Job J (of NJ) moves 1 KB of the stage with one load: lane i writes the 16 bytes at
    // 16 i of the job's block.  Loader lw runs jobs lw, lw + 4, ...; which tile and rows a
    // job covers is fixed at compile time (one code path per loader), and all loads of a
    // chunk are in flight together without holding registers.
    constexpr int NJ_PER = (NJ + kWaves - 1) / kWaves;
    const int qk_row = hqk * DK, v_row = hv * dv;
    const size_t slot_begin = slot_of(map, n, c_begin);   // chunk c sits in slot slot_begin + c - c_begin
    auto job_row = [&](auto jc) __attribute__((always_inline)) -> int {   // source row of this lane
        constexpr int J = decltype(jc)::value;
        if constexpr (J < J_W)
            return min((J % NJ_QK) * 64 + lane, NCK_QK - 1) / (DK * ES / 16);
        else if constexpr (J >= J_V && J < J_D)
            return min((J - J_V) * 64 + lane, NCK_V - 1) / (DVS * ES / 16);
        else
            return 0;
    };
    // element offset of this lane's 16 bytes from the tile's origin, given its source row
    auto job_off = [&](auto jc, int row) __attribute__((always_inline)) -> int {
        constexpr int J = decltype(jc)::value;
        if constexpr (J < J_W) {
            const int P = min((J % NJ_QK) * 64 + lane, NCK_QK - 1);
            const int r = P / (DK * ES / 16), pos = P % (DK * ES / 16);
            return row * qk_row + (pos ^ SK::perm(r)) * VN;
        } else if constexpr (J < J_V) {   // W or M: rows of C elements
            constexpr int NCK_X = J < J_M ? NCK_W : NCK_M;
            constexpr int IDX = J < J_M ? J - J_W : J - J_M;
            const int P = min(IDX * 64 + lane, NCK_X - 1);
            const int r = P / (C * ES / 16), pos = P % (C * ES / 16);
            return r * C + (pos ^ SC::perm(r)) * VN;
        } else if constexpr (J < J_D) {
            const int P = min((J - J_V) * 64 + lane, NCK_V - 1);
            const int r = P / (DVS * ES / 16), pos = P % (DVS * ES / 16);
            return row * v_row + (pos ^ SV::perm(r)) * VN;
        } else {
            return min((J - J_D) * 64 + lane, NCK_D - 1) * 4;   // floats
        }
    };
    // Stage part PART (0: A, 1: B) of chunk c.  Rows past the chunk's last real row are
    // loaded from it.
    auto issue_jobs = [&](auto wc, auto partc, int c) __attribute__((always_inline)) {
        constexpr int W = decltype(wc)::value;
        constexpr int PART = decltype(partc)::value;
        __attribute__((address_space(3))) unsigned char *stg =
            PART == 0 ? lds_a + (c % NSTAGE) * STAGE_A : lds_b + (c & 1) * STAGE_B;
        const int64_t t0 = a + (int64_t)c * C;
        const int last = (int)min<int64_t>(C, b - t0) - 1;   // >= 0 for every chunk of the sequence
        const size_t slot = slot_begin + (size_t)(c - c_begin);
        const E *qb = q + ((size_t)t0 * hqk + hq) * DK;
        const E *kb = k + ((size_t)t0 * hqk + hq) * DK;
        const E *vb = v + ((size_t)t0 * hv + h) * dv + (size_t)s * DVS;
        const E *wb = wmat + (slot * hv + h) * DK * C;
        const E *mb = mmat + (slot * hv + h) * C * C;
        const E *db = reinterpret_cast<const E *>(dec + (slot * hv + h) * 4 * C);
        static_for<NJ_PER>([&](auto uc) {
            constexpr int J = W + decltype(uc)::value * kWaves;
            constexpr bool in_a = J < J_W || (J >= J_V && J < J_D);   // Q, K, V
            if constexpr (J < NJ && in_a == (PART == 0)) {
                constexpr std::integral_constant<int, J> jc{};
                const E *base;
                int off = job_off(jc, min(job_row(jc), last));
                if constexpr (J < J_W)
                    base = J >= NJ_QK ? kb : qb;
                else if constexpr (J < J_V)
                    base = J >= J_M ? mb : wb;
                else if constexpr (J < J_D)
                    base = vb;
                else {
                    base = db;
                    off *= (int)(sizeof(float) / sizeof(E));
                }
                // lanes of the job that carry data, and the job's block in the stage
                constexpr int NCK = J < J_W ? NCK_QK : J < J_M ? NCK_W : J < J_V ? NCK_M : J < J_D ? NCK_V : NCK_D;
                constexpr int IDX = J < J_W ? J % NJ_QK : J < J_M ? J - J_W : J < J_V ? J - J_M
                                  : J < J_D ? J - J_V : J - J_D;
                constexpr int NL = NCK - IDX * 64 < 64 ? NCK - IDX * 64 : 64;
                constexpr int BLK = (J < J_W ? (J >= NJ_QK ? OFF_K : OFF_Q)
                                             : J < J_M ? OFF_W : J < J_V ? OFF_M : J < J_D ? OFF_V : OFF_D) + IDX * 1024;
                if (NL == 64 || lane < NL)
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                     (__attribute__((address_space(3))) void *)(stg + BLK), 16, 0, 0);
            }
        });
    };
    auto by_loader = [&](auto fn) __attribute__((always_inline)) {
        switch (lw) {
        case 0: fn(std::integral_constant<int, 0>{}); break;
        case 1: fn(std::integral_constant<int, 1>{}); break;
        case 2: fn(std::integral_constant<int, 2>{}); break;
        default: fn(std::integral_constant<int, 3>{}); break;
        }
    };
    // ---- compute waves: one chunk step on stage buffer `cur` (barrier B1 inside) ----
    auto step = [&](int c, int64_t t0, int len) __attribute__((always_inline)) {
        const unsigned char *stg = stage_a + (c % NSTAGE) * STAGE_A;     // Q, K, V
        const unsigned char *stb = stage_b + (c & 1) * STAGE_B;          // W, M, record
        const float *Gs = reinterpret_cast<const float *>(stb + OFF_D);   // exp(G)
        const float *Bet = Gs + 2 * C;                                     // beta
        const float *BGam = Gs + 3 * C;                                    // beta exp(G)

        // P1: (Q S)^T and K S for row tile rt (all column tiles); X = diag(beta)(V - diag(exp G)
        //     K S) goes to Xt (transposed); (diag(exp G) Q S)^T stays in oacc for P3.
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
                        oacc[u][ct] = MK::mma(bs, aq, oacc[u][ct]);   // (Q S)^T: lane = token
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
                        x[i] = Bet[rr] * to_f32(vv) - BGam[rr] * kacc[u][ct][i];
                        oacc[u][ct][i] *= scale * Gs[rt * 16 + (lane & 15)];
                    }
                    store4(Xt + col * LDC + rt * 16 + tile_row(lane, 0), x[0], x[1], x[2], x[3]);
                }
            }
        }
        __syncthreads();   // B1

        // P3: O = scale diag(exp G) Q S + M X, computed transposed (O^T = (Q S)^T + X^T M^T,
        //     the same fragments with the operand roles swapped) so that each lane holds four
        //     consecutive output columns of one token and stores them at once
#pragma unroll
        for (int u = 0; u < RT_PER; ++u) {
            const int rt = wave + u * kWaves;
            if (rt < RT) {
                const int r = lane & 15, kk = (lane >> 4) * MC::kPerLane;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += MC::kStep) {
                    const auto am = staged_frag<MC, SC, E>(stb + OFF_M, rt * 16 + r, k0 + kk);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        oacc[u][ct] = MC::mma(MC::load(Xt + (ct * 16 + r) * LDC + k0 + kk), am, oacc[u][ct]);
                }
                // O^T tile: lane = token rt * 16 + l % 16, four consecutive output columns
                const int tok = rt * 16 + (lane & 15);
                if (tok < len) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        store4(o + ((size_t)(t0 + tok) * hv + h) * dv + (size_t)s * DVS + ct * 16 + 4 * (lane >> 4),
                               oacc[u][ct][0], oacc[u][ct][1], oacc[u][ct][2], oacc[u][ct][3]);
                }
            }
        }
        // P4: S <- exp(G_last) S + W X; refresh the transposed copy
        const float gl = Gs[C - 1];   // exp(G_last): G is flat past the last real token
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
                    const auto aw = staged_frag<MC, SC, E>(stb + OFF_W, sr * 16 + r, k0 + kk);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        sacc[u][ct] = MC::mma(aw, MC::load(Xt + (ct * 16 + r) * LDC + k0 + kk), sacc[u][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    store4(St + (ct * 16 + tile_col(lane)) * LDK + sr * 16 + tile_row(lane, 0), sacc[u][ct][0],
                           sacc[u][ct][1], sacc[u][ct][2], sacc[u][ct][3]);
            }
        }
    };

    // ---- pipeline: while the compute waves work on chunk c, the loaders stage part B of
    //      chunk c + 1 and then part A of chunk c + NSTAGE - 1 (part A of chunk c is dead
    //      once the step passes its first barrier, part B of chunk c - 1 once the previous
    //      step ended).  The direct loads are not tracked by the compiler's LDS dependences:
    //      before the barrier that ends a step, each loader waits until every load of chunk
    //      c + 1 has landed, leaving only its part-A loads of chunk c + 2 in flight (the
    //      counter retires loads in issue order).  The loaders take bare barriers: a fenced
    //      one would first wait for all their loads. ----
    // wait for all of this loader's loads but its part-A jobs of one chunk (jobs W, W + 4, ...)
    auto wait_all_but_part_a = [&](auto wc) __attribute__((always_inline)) {
        constexpr int W = decltype(wc)::value;
        constexpr int cnt = [] {
            int n = 0;
            for (int J = W; J < NJ; J += kWaves)
                n += (J < J_W || (J >= J_V && J < J_D)) ? 1 : 0;
            return n;
        }();
        static_assert(cnt < 64, "vmcnt holds at most 63");
        __builtin_amdgcn_s_waitcnt((cnt & 15) | ((cnt >> 4) << 14) | 0x0f70);   // vmcnt(cnt) only
        asm volatile("" ::: "memory");
    };
    constexpr std::integral_constant<int, 0> part_a{};
    constexpr std::integral_constant<int, 1> part_b{};
    constexpr int AHEAD = NSTAGE - 1;   // chunks of lead of part A
    if (loader) {
        by_loader([&](auto wc) {
            issue_jobs(wc, part_a, c_begin);
            issue_jobs(wc, part_b, c_begin);
        });
        if (AHEAD == 2 && c_begin + 1 < c_end)
            by_loader([&](auto wc) {
                issue_jobs(wc, part_a, c_begin + 1);
                wait_all_but_part_a(wc);
            });
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    for (int c = c_begin; c < c_end; ++c) {
        if (loader) {
            if (c + 1 < c_end)
                by_loader([&](auto wc) { issue_jobs(wc, part_b, c + 1); });
            if (c + AHEAD < c_end)
                by_loader([&](auto wc) { issue_jobs(wc, part_a, c + AHEAD); });
            // B1 of the compute waves: the loaders publish nothing there
            __builtin_amdgcn_s_barrier();
            if (AHEAD == 2 && c + 2 < c_end)
                by_loader([&](auto wc) { wait_all_but_part_a(wc); });
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();   // end of step: chunk c + 1 is staged
        } else {
            const int64_t ct0 = a + (int64_t)c * C;
            step(c, ct0, (int)min<int64_t>(C, b - ct0));
            __syncthreads();   // end of step: St is complete
        }
    }
    if (!loader) {
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
// Scan kernel for bf16 io and chunk 64 (the Qwen3.5 shapes): the chunk step
// of the absorbed form (see AbsorbedForm), with the chunk's matrix operands
// staged in FRAGMENT ORDER.  Every operand tile is a sequence of 1 KB units of 16
// rows x 32 contraction indices; in a unit, the 16 bytes at position p belong
// to matrix-core lane m(p): row m % 16 of the unit's rows, contraction indices
// 8 (m / 16) .. +7.  One direct-to-LDS load fills one unit (lane i of the load
// fetches the 16 bytes of position i), and one LDS read of 16 bytes at 16 l
// gives lane l its operand fragment: neither side computes addresses beyond a
// per-lane constant and instruction offsets, and a unit read is a 1 KB read in
// lane order, the fastest LDS read pattern measured (see Swz).
//   Q, M units (rt, kb): rows 16 rt + r (natural order), m(p) = p.
//   W units (sr, kb):    key rows Chain row(sr, r), chunk rows 32 kb + 8 (p / 16)
//                        .. +7, m(p) = p (W replaces T: absorbed form).
//   K units (rt, kb):    rows Chain row(rt, r); m(p) = r + 16 g with g = p / 16,
//                        r = (p % 16) ^ 4 g (measured: the fragment read at
//                        about half its lane-order rate; see Swz).
//   V (the dv slice):    row-major; the 16-byte chunks of a row are permuted
//                        (XOR with 2 (r % 4) for 256-byte rows, 2 ((r / 2) % 2)
//                        for 128-byte rows), which spreads the transpose read
//                        of 4 consecutive rows of one column block over the
//                        banks (without it that read runs 3x slower).
//   decay record:        [exp(G) | exp(G_last - G) | beta | beta exp(G)].
// Each wave owns CT tiles of 16 state columns: every operand fragment read
// from LDS then feeds CT matrix instructions.  The output is computed
// transposed (O^T = (Q S)^T ... with S^T and X^T as the A operands, whose
// registers are the B fragments as they stand), so that each lane holds 4
// consecutive columns of one token row and stores them as one 8-byte write.
// ---------------------------------------------------------------------------
template <int DK, int NW, int CT>
__global__ __launch_bounds__(NW * kWave) void gdn_chunk_scan_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const int32_t *__restrict__ cu, SlotMap map, int32_t num_seqs, int64_t total_tokens, int32_t hqk, int32_t hv,
    int32_t dv, const bf16 *__restrict__ wmat, const bf16 *__restrict__ mmat, const float *__restrict__ dec,
    const float *state_in, float *state_out, bf16 *__restrict__ o, float scale)
{
    constexpr int C = 64;
    constexpr int WC = 16 * CT;                   // columns per wave
    constexpr int DVS = WC * NW;                  // columns per workgroup
    constexpr int NT = NW * kWave;
    constexpr int RT = C / 16, SR = DK / 16;
    constexpr int NSK = DK / 32, NSC = C / 32;
    typedef Mma<bf16> M;
    typedef Chain<M> CH;
    static_assert(DK % 32 == 0, "32-wide contraction steps");

    // stage layout (bytes): 1 KB units
    constexpr int NU_QK = RT * NSK, NU_W = SR * NSC, NU_M = RT * NSC;
    constexpr int VRB = DVS * 2;                   // bytes per row of the V slice
    constexpr int NU_V = C * VRB / 1024;
    constexpr int OFF_Q = 0;
    constexpr int OFF_K = OFF_Q + NU_QK * 1024;
    constexpr int OFF_W = OFF_K + NU_QK * 1024;
    constexpr int OFF_M = OFF_W + NU_W * 1024;
    constexpr int OFF_V = OFF_M + NU_M * 1024;
    constexpr int OFF_D = OFF_V + NU_V * 1024;
    constexpr int STAGE = OFF_D + 1024;
    static_assert(C * VRB % 1024 == 0 && 4 * C * 4 == 1024, "whole units");
    static_assert(VRB == 64 || VRB == 128 || VRB == 256, "V slice rows of 64, 128 or 256 bytes");

    // The two stage buffers are separate objects, so that the compiler can tell the
    // direct loads into one from the reads of the other (a single array would make
    // every read of the current chunk wait for the loads of the next).
    __shared__ __attribute__((aligned(1024))) unsigned char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1[STAGE];
    auto stage_ptr = [&](auto bufc) __attribute__((always_inline)) -> unsigned char * {
        return decltype(bufc)::value ? stage1 : stage0;
    };
    auto stage_lds = [&](auto bufc) __attribute__((always_inline)) {
        return (__attribute__((address_space(3))) unsigned char *)(decltype(bufc)::value ? stage1 : stage0);
    };

    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int r16 = lane & 15, G = lane >> 4, g4 = 4 * G;
    const int nv = dv / DVS;
    const int pairs = num_seqs * hv;
    // item = (sequence rank, query/key head); its members are the group's value heads
    // times their column slices
    const int group = hv / hqk;
    int item, member;
    xcd_group(blockIdx.x, group * nv, item, member);
    const int pair = item * group + member / nv;
    const int s = member % nv;
    if (pair >= pairs)
        return;
    const int n = ranked_sequence(map, pair / hv), h = pair - (pair / hv) * hv;
    const int hq = h / (hv / hqk);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int nch = seq_chunks(map, cu, n, total_tokens, C);
    const int c_begin = map.seg_first;
    const int c_end = min(nch, map.seg_first + map.seg_len);
    const int col0 = s * DVS + WC * w;                  // first state / output column of this wave
    const size_t state_base = (size_t)(n * hv + h) * DK * dv;
    if (c_begin >= c_end) {
        if (c_begin == 0 && state_in != state_out) {
            for (int i = tid; i < DK * DVS; i += NT) {
                const size_t off = state_base + (size_t)(i / DVS) * dv + s * DVS + (i % DVS);
                state_out[off] = state_in ? state_in[off] : 0.f;
            }
        }
        return;
    }

    // ---- state columns in accumulators: tile (sr, ct), slot i holds key row
    //      CH::row(sr, g4 + i), column col0 + 16 ct + l % 16 ----
    f32x4 sacc[SR][CT];
#pragma unroll
    for (int sr = 0; sr < SR; ++sr)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sacc[sr][ct][i] = state_in ? state_in[state_base + (size_t)CH::row(sr, g4 + i) * dv + col0 + 16 * ct +
                                                      r16]
                                           : 0.f;
    auto pack_s = [&](bf16x8 (&sb)[NSK][CT]) __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 t[SR];
#pragma unroll
            for (int sr = 0; sr < SR; ++sr)
                t[sr] = sacc[sr][ct];
#pragma unroll
            for (int st = 0; st < NSK; ++st)
                sb[st][ct] = CH::b_frag(t, st);
        }
    };

    // ---- staging ----
    // chunk c of the sequence sits in workspace slot slot0 + c (in either launch mode)
    const size_t slot0 = slot_of(map, n, 0);
    // The stage is filled in rounds of NW units: in round R every wave loads one unit of
    // the same tile (unit (R - first round of the tile) NW + w), so all waves run the same
    // code and each lane's source offsets are computed once.  Rounds: Q, K, T, A, the V
    // slice, then the decay record (wave 0 only).  (RT0 and RA0 begin the W and M rounds.)
    constexpr int R_Q = NU_QK / NW, R_W = NU_W / NW, R_M = NU_M / NW, R_V = NU_V / NW;
    static_assert(NU_QK % NW == 0 && NU_W % NW == 0 && NU_M % NW == 0 && NU_V % NW == 0, "whole rounds");
    constexpr int RK0 = R_Q, RT0 = 2 * R_Q, RA0 = RT0 + R_W, RV0 = RA0 + R_M, RD0 = RV0 + R_V;
    constexpr int NR = RD0 + 1;
    const int qk_row = hqk * DK, v_row = hv * dv;
    // (row in the chunk, element column, stage offset of the unit) of this lane's 16
    // bytes in round R
    auto round_src = [&](auto rc, int &row, int &ecol, int &blk) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
        if constexpr (R < RT0) {                       // Q or K unit (rt, kb)
            const int u = (R < RK0 ? R : R - RK0) * NW + w;
            const int rt = u / NSK, kb = u % NSK;
            row = R < RK0 ? 16 * rt + r16 : CH::row(rt, r16 ^ g4);
            ecol = 32 * kb + 8 * G;
            blk = (R < RK0 ? OFF_Q : OFF_K) + u * 1024;
        } else if constexpr (R < RV0) {                // W unit (sr, kb) or M unit (rt, kb)
            const int u = (R < RA0 ? R - RT0 : R - RA0) * NW + w;
            const int rt = u / NSC, kb = u % NSC;
            row = R < RA0 ? CH::row(rt, r16) : 16 * rt + r16;
            ecol = 32 * kb + 8 * G;
            blk = (R < RA0 ? OFF_W : OFF_M) + u * 1024;
        } else if constexpr (R < RD0) {                // 1 KB of rows of the V slice
            const int u = (R - RV0) * NW + w;
            const int P = u * 64 + lane;                  // physical 16-byte chunk
            row = P / (VRB / 16);
            int j = P % (VRB / 16);
            if constexpr (VRB == 256)
                j ^= 2 * (row & 3);
            else if constexpr (VRB == 128)
                j ^= 2 * ((row >> 1) & 1);
            ecol = j * 8;
            blk = OFF_V + u * 1024;
        } else {                                       // decay record, 4 floats per lane
            row = 0;
            ecol = lane * 4;
            blk = OFF_D;
        }
    };
    // byte offset of this lane's 16 bytes from the chunk's base of the tile
    auto round_bytes = [&](auto rc, int row, int ecol) __attribute__((always_inline)) -> uint32_t {
        constexpr int R = decltype(rc)::value;
        if constexpr (R < RT0)
            return (uint32_t)(row * qk_row + ecol) * 2u;
        else if constexpr (R < RV0)
            return (uint32_t)(row * C + ecol) * 2u;
        else if constexpr (R < RD0)
            return (uint32_t)(row * v_row + ecol) * 2u;
        else
            return (uint32_t)ecol * 4u;
    };
    uint32_t loff[NR];
    int lblk[NR];
    static_for<NR>([&](auto rc) __attribute__((always_inline)) {
        int row, ecol, blk;
        round_src(rc, row, ecol, blk);
        loff[decltype(rc)::value] = round_bytes(rc, row, ecol);
        lblk[decltype(rc)::value] = blk;
    });
    // Rounds [LO, HI) of the staging of chunk c into buffer BUF.
    auto issue_rounds = [&](auto bufc, int c, auto loc, auto hic) __attribute__((always_inline)) {
        constexpr int LO = decltype(loc)::value, HI = decltype(hic)::value;
        __attribute__((address_space(3))) unsigned char *stg = stage_lds(bufc);
        const int64_t t0 = a + (int64_t)c * C;
        const int last = (int)min<int64_t>(C, b - t0) - 1;
        const size_t slot = slot0 + c;
        // wave-uniform bases: the loads take them as a scalar base plus a 32-bit lane offset
        const char *qb = reinterpret_cast<const char *>(q + ((size_t)t0 * hqk + hq) * DK);
        const char *kb = reinterpret_cast<const char *>(k + ((size_t)t0 * hqk + hq) * DK);
        const char *vb = reinterpret_cast<const char *>(v + ((size_t)t0 * hv + h) * dv + (size_t)s * DVS);
        const char *tb = reinterpret_cast<const char *>(wmat + (slot * hv + h) * DK * C);
        const char *ab = reinterpret_cast<const char *>(mmat + (slot * hv + h) * C * C);
        const char *db = reinterpret_cast<const char *>(dec + (slot * hv + h) * 4 * C);
        const bool full = last == C - 1;
        static_for<NR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;
            if constexpr (R < LO || R >= HI)
                return;
            uint32_t off = loff[R];
            if constexpr (R < RT0 || (R >= RV0 && R < RD0)) {
                if (!full) {   // ragged last chunk: rows past its end repeat its last row
                    int row, ecol, blk;
                    round_src(rc, row, ecol, blk);
                    off = round_bytes(rc, min(row, last), ecol);
                }
            }
            const char *base = R < RK0 ? qb : R < RT0 ? kb : R < RA0 ? tb : R < RV0 ? ab : R < RD0 ? vb : db;
            if (R < RD0 || w == 0)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                 (__attribute__((address_space(3))) void *)(stg + lblk[R]), 16, 0,
                                                 0);
        });
    };
    auto issue_stage = [&](auto bufc, int c) __attribute__((always_inline)) {
        issue_rounds(bufc, c, std::integral_constant<int, 0>{}, std::integral_constant<int, NR>{});
    };
    // The next chunk's staging is issued in four parts spread over the step (q and k
    // rounds first, the decay record last): issued at once, the last waves to issue would
    // stall for the whole transfer before starting their products.
    constexpr int kPartEnd[4] = {RT0, RV0, RD0, NR};
    auto stage_part = [&](auto bufc, int c, auto pc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        issue_rounds(bufc, c, std::integral_constant<int, P == 0 ? 0 : kPartEnd[P == 0 ? 0 : P - 1]>{},
                     std::integral_constant<int, kPartEnd[P]>{});
    };
    auto stage_done = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // per-lane LDS byte offsets (everything else is an instruction offset)
    const int lin = 16 * lane;                                   // Q, T, A units
    const int kperm = 16 * (16 * G + (r16 ^ g4));                 // K units, fragment read
    const int e = (lane >> 2) & 3, qd = lane & 3;
    // V slice, transpose read of column block ct of this wave: rows 8 G + e (+ the
    // tile's first row), logical chunk 2 (CT w + ct) + qd / 2, physical = logical ^ X(row)
    auto vtr = [&](int ct) __attribute__((always_inline)) -> int {
        int chunk = 2 * (CT * w + ct) + (qd >> 1);
        if constexpr (VRB == 256)
            chunk ^= 2 * e;
        else if constexpr (VRB == 128)
            chunk ^= 2 * (e >> 1);
        return (8 * G + e) * VRB + 16 * chunk + 8 * (qd & 1);
    };
    int vtro[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        vtro[ct] = vtr(ct);

    // ---- one chunk step of this wave's WC columns on stage buffer BUF ----
    auto step = [&](auto bufc, int64_t t0, int len, auto &&stage_hook) __attribute__((always_inline)) {
        const unsigned char *stg = stage_ptr(bufc);
        auto frag = [&](int off) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8 *>(stg + off);
        };
        auto rec4 = [&](int arr, int row0) __attribute__((always_inline)) {
            return *reinterpret_cast<const f32x4 *>(stg + OFF_D + 4 * (arr * C + row0));
        };
        auto tr4 = [&](int off) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(stage_lds(bufc) + off));
        };

        // [Q;K] S: (Q S)^T with S^T as the A operand; K S with K rows in the order of CH
        stage_hook(std::integral_constant<int, 0>{});
        bf16x8 sb[NSK][CT];
        pack_s(sb);
        f32x4 qacc[RT][CT], xacc[RT][CT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                qacc[rt][ct] = zero4();
                xacc[rt][ct] = zero4();
            }
#pragma unroll
        for (int st = 0; st < NSK; ++st) {
            bf16x8 fq[RT], fk[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                fq[rt] = frag(OFF_Q + (rt * NSK + st) * 1024 + lin);
                fk[rt] = frag(OFF_K + (rt * NSK + st) * 1024 + kperm);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    qacc[rt][ct] = M::mma(sb[st][ct], fq[rt], qacc[rt][ct]);
                    xacc[rt][ct] = M::mma(fk[rt], sb[st][ct], xacc[rt][ct]);
                }
        }

        stage_hook(std::integral_constant<int, 1>{});
        // X = beta v - beta exp(G) (K S) on this lane's rows CH::row(rt, g4 + i) (the bit
        // cast is of the whole vector: a bit cast of one element of a vector reads element 0)
        bf16x8 xb[NSC][CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 t[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x4 vv = __builtin_bit_cast(bf16x4, tr4(OFF_V + CH::row(rt, 0) * VRB + vtro[ct]));
                const f32x4 vf = {(float)vv[0], (float)vv[1], (float)vv[2], (float)vv[3]};
                t[rt] = rec4(2, CH::row(rt, g4)) * vf - rec4(3, CH::row(rt, g4)) * xacc[rt][ct];
            }
#pragma unroll
            for (int st = 0; st < NSC; ++st)
                xb[st][ct] = CH::b_frag(t, st);
        }
        __builtin_amdgcn_sched_barrier(0);

        stage_hook(std::integral_constant<int, 2>{});
        // S <- exp(G_last) S + W X.  W fragments: key rows CH::row(sr, .), chunk rows
        // 32 st + 8 G + {0..7}, read one key tile ahead of their products.
        auto load_w = [&](int sr, bf16x8 (&f)[NSC]) __attribute__((always_inline)) {
#pragma unroll
            for (int st = 0; st < NSC; ++st)
                f[st] = frag(OFF_W + (sr * NSC + st) * 1024 + lin);
        };
        const float gl = *reinterpret_cast<const float *>(stg + OFF_D + 4 * (C - 1));
        bf16x8 fw[2][NSC];
        load_w(0, fw[0]);
#pragma unroll
        for (int sr = 0; sr < SR; ++sr) {
            if (sr + 1 < SR)
                load_w(sr + 1, fw[(sr + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                sacc[sr][ct] = sacc[sr][ct] * gl;
#pragma unroll
                for (int st = 0; st < NSC; ++st)
                    sacc[sr][ct] = M::mma(fw[sr & 1][st], xb[st][ct], sacc[sr][ct]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_hook(std::integral_constant<int, 3>{});
        // M fragments (M carries the output scale)
        bf16x8 fm[NSC][RT];
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                fm[st][rt] = frag(OFF_M + (rt * NSC + st) * 1024 + lin);

        // O^T = scale (Q S)^T diag(exp G) + X^T M^T: lane l holds token row 16 rt + l % 16
        // and the four columns 16 ct + 4 (l / 16) .. +3 of this wave's
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float gs = scale * *reinterpret_cast<const float *>(stg + OFF_D + 4 * (16 * rt + r16));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                qacc[rt][ct] *= gs;
        }
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    qacc[rt][ct] = M::mma(xb[st][ct], fm[st][rt], qacc[rt][ct]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = 16 * rt + r16;
            if (r < len) {
                bf16 *orow = o + ((size_t)(t0 + r) * hv + h) * dv + col0 + g4;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    *reinterpret_cast<bf16x4 *>(orow + 16 * ct) =
                        bf16x4{(bf16)qacc[rt][ct][0], (bf16)qacc[rt][ct][1], (bf16)qacc[rt][ct][2],
                               (bf16)qacc[rt][ct][3]};
            }
        }
    };

    // ---- pipeline: one barrier per chunk; buffers alternate from buffer 0 ----
    const std::integral_constant<int, 0> buf0;
    const std::integral_constant<int, 1> buf1;
    issue_stage(buf0, c_begin);
    stage_done();
    for (int c = c_begin;;) {
        bool more = c + 1 < c_end;
        int64_t t0 = a + (int64_t)c * C;
        step(buf0, t0, (int)min<int64_t>(C, b - t0), [&](auto pc) __attribute__((always_inline)) {
            if (more)
                stage_part(buf1, c + 1, pc);
        });
        stage_done();
        if (++c >= c_end)
            break;
        more = c + 1 < c_end;
        t0 = a + (int64_t)c * C;
        step(buf1, t0, (int)min<int64_t>(C, b - t0), [&](auto pc) __attribute__((always_inline)) {
            if (more)
                stage_part(buf0, c + 1, pc);
        });
        stage_done();
        if (++c >= c_end)
            break;
    }

    // ---- final state ----
#pragma unroll
    for (int sr = 0; sr < SR; ++sr)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                state_out[state_base + (size_t)CH::row(sr, g4 + i) * dv + col0 + 16 * ct + r16] = sacc[sr][ct][i];
}

// ---------------------------------------------------------------------------
// Whole-head scan of the T form (bf16 io, chunk 64, dk = dv = 128; see PrepForm): one
// workgroup of 8 waves per (sequence, value head), each wave owning 16 state columns held in
// matrix-core accumulators, as in gdn_chunk_scan_bf16_kernel.  The prep hands over T as hi/lo
// bf16 units and the decay record; per chunk the step computes
//   A   = scale exp(G_t - G_j) q_t.k_j for j <= t: 12 tiles of 16 query rows by 16 key rows
//         (key rows in Chain order), dealt to the waves round-robin and formed inside the
//         [Q;K] S products from the same fragments, then left in LDS as a hi and a lo matrix
//   X   = beta v - beta exp(G) (K S)
//   Y   = T X = T_hi X + T_lo X
//   S  <- exp(G_last) S + K^T (lambda Y)_hi + K^T (lambda Y)_lo
//   O   = scale exp(G) Q S + A_hi Y_hi + A_hi Y_lo + A_lo Y_hi
// Every product that meets T, Y or A takes hi/lo pairs of the fp32 values, so the cancelling
// sums of T's alternating columns (correlated keys) are carried at about 16 significant bits;
// q, k, X and S enter as bf16.  K^T comes from the K units with the LDS transpose read: for
// the contraction rows 32 st + 8 g + {0..7} and key rows Chain row(sr, .), input lane
// (e, quarter) of a 16-lane group reads 4 keys of chunk row 32 st + 8 g + e (+ 4).
// The output leaves through LDS: each wave holds 16 columns of the chunk's 64 rows, which
// written straight out would be 32-byte pieces of each row (partial-line writes, about a
// sixth of the kernel's time on a long batch); the waves write their pieces into one bf16
// row buffer, and after the barrier that ends the step each wave stores 8 whole rows.
// ---------------------------------------------------------------------------
template <int DK, int NW>
__global__ __launch_bounds__(NW * kWave) void gdn_chunk_scan_tform_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const int32_t *__restrict__ cu, SlotMap map, int32_t num_seqs, int64_t total_tokens, int32_t hqk, int32_t hv,
    int32_t dv, const bf16 *__restrict__ tmat, const float *__restrict__ dec, const float *state_in,
    float *state_out, bf16 *__restrict__ o, float scale)
{
    constexpr int C = 64;
    constexpr int WC = 16;                        // columns per wave
    constexpr int DVS = WC * NW;                  // columns per workgroup
    constexpr int NT = NW * kWave;
    constexpr int RT = C / 16, SR = DK / 16;
    constexpr int NSK = DK / 32, NSC = C / 32;
    typedef Mma<bf16> M;
    typedef Chain<M> CH;
    static_assert(DK == 128 && DVS == 128, "whole heads of 128 columns");

    // stage layout (bytes): 1 KB units
    constexpr int NU_QK = RT * NSK, NU_T = 2 * kTUnits;
    constexpr int VRB = DVS * 2;                   // bytes per row of the V slice
    constexpr int NU_V = C * VRB / 1024;
    constexpr int OFF_Q = 0;
    constexpr int OFF_K = OFF_Q + NU_QK * 1024;
    constexpr int OFF_T = OFF_K + NU_QK * 1024;
    constexpr int OFF_V = OFF_T + NU_T * 1024;
    constexpr int OFF_D = OFF_V + NU_V * 1024;
    constexpr int STAGE = OFF_D + 1024;
    constexpr int AB = C * C * 2;                  // bytes of one bf16 A matrix
    static_assert(C * VRB % 1024 == 0 && 4 * C * 4 == 1024 && VRB == 256, "whole units, 256-byte V rows");

    __shared__ __attribute__((aligned(1024))) unsigned char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1[STAGE];
    // A hi, A lo, each in 1 KB fragment units: unit 2 rt + st holds at 16-byte position p the
    // query row 16 rt + p % 16, keys 32 st + 8 (p / 16) .. +7
    __shared__ __attribute__((aligned(1024))) unsigned char abuf[2 * AB];
    // the chunk's output rows (bf16, rows of ORB bytes): each wave writes its 16 columns, and
    // after the barrier that ends the step each wave stores 8 whole rows (full-line writes)
    constexpr int ORB = DVS * 2 + 16;
    __shared__ __attribute__((aligned(16))) unsigned char obuf[C * ORB];
    auto stage_ptr = [&](auto bufc) __attribute__((always_inline)) -> unsigned char * {
        return decltype(bufc)::value ? stage1 : stage0;
    };
    auto stage_lds = [&](auto bufc) __attribute__((always_inline)) {
        return (__attribute__((address_space(3))) unsigned char *)(decltype(bufc)::value ? stage1 : stage0);
    };

    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int r16 = lane & 15, G = lane >> 4, g4 = 4 * G;
    const int nv = dv / DVS;
    const int pairs = num_seqs * hv;
    const int group = hv / hqk;
    int item, member;
    xcd_group(blockIdx.x, group * nv, item, member);
    const int pair = item * group + member / nv;
    const int s = member % nv;
    if (pair >= pairs)
        return;
    const int n = ranked_sequence(map, pair / hv), h = pair - (pair / hv) * hv;
    const int hq = h / (hv / hqk);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int nch = seq_chunks(map, cu, n, total_tokens, C);
    const int c_begin = map.seg_first;
    const int c_end = min(nch, map.seg_first + map.seg_len);
    const int col0 = s * DVS + WC * w;                  // first state / output column of this wave
    const size_t state_base = (size_t)(n * hv + h) * DK * dv;
    if (c_begin >= c_end) {
        if (c_begin == 0 && state_in != state_out) {
            for (int i = tid; i < DK * DVS; i += NT) {
                const size_t off = state_base + (size_t)(i / DVS) * dv + s * DVS + (i % DVS);
                state_out[off] = state_in ? state_in[off] : 0.f;
            }
        }
        return;
    }

    // ---- state columns in accumulators: tile sr, slot i holds key row CH::row(sr, g4 + i),
    //      column col0 + l % 16 ----
    f32x4 sacc[SR];
#pragma unroll
    for (int sr = 0; sr < SR; ++sr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sacc[sr][i] = state_in ? state_in[state_base + (size_t)CH::row(sr, g4 + i) * dv + col0 + r16] : 0.f;

    // ---- staging (as in gdn_chunk_scan_bf16_kernel; T units are contiguous 1 KB blocks) ----
    const size_t slot0 = slot_of(map, n, 0);
    constexpr int R_Q = NU_QK / NW, R_T = (NU_T + NW - 1) / NW, R_V = NU_V / NW;
    static_assert(NU_QK % NW == 0 && NU_V % NW == 0, "whole rounds");
    constexpr int RK0 = R_Q, RT0 = 2 * R_Q, RV0 = RT0 + R_T, RD0 = RV0 + R_V;
    constexpr int NR = RD0 + 1;
    const int qk_row = hqk * DK, v_row = hv * dv;
    auto round_src = [&](auto rc, int &row, int &ecol, int &blk) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
        if constexpr (R < RT0) {                       // Q or K unit (rt, kb)
            const int u = (R < RK0 ? R : R - RK0) * NW + w;
            const int rt = u / NSK, kb = u % NSK;
            row = R < RK0 ? 16 * rt + r16 : CH::row(rt, r16 ^ g4);
            ecol = 32 * kb + 8 * G;
            blk = (R < RK0 ? OFF_Q : OFF_K) + u * 1024;
        } else if constexpr (R < RV0) {                // T unit (hi units, then lo)
            const int u = min((R - RT0) * NW + w, NU_T - 1);
            row = u;
            ecol = 8 * lane;
            blk = OFF_T + u * 1024;
        } else if constexpr (R < RD0) {                // 1 KB of rows of the V slice
            const int u = (R - RV0) * NW + w;
            const int P = u * 64 + lane;
            row = P / (VRB / 16);
            const int j = (P % (VRB / 16)) ^ (2 * (row & 3));
            ecol = j * 8;
            blk = OFF_V + u * 1024;
        } else {                                       // decay record, 4 floats per lane
            row = 0;
            ecol = lane * 4;
            blk = OFF_D;
        }
    };
    auto round_bytes = [&](auto rc, int row, int ecol) __attribute__((always_inline)) -> uint32_t {
        constexpr int R = decltype(rc)::value;
        if constexpr (R < RT0)
            return (uint32_t)(row * qk_row + ecol) * 2u;
        else if constexpr (R < RV0)
            return (uint32_t)(row * 512 + ecol) * 2u;
        else if constexpr (R < RD0)
            return (uint32_t)(row * v_row + ecol) * 2u;
        else
            return (uint32_t)ecol * 4u;
    };
    uint32_t loff[NR];
    int lblk[NR];
    static_for<NR>([&](auto rc) __attribute__((always_inline)) {
        int row, ecol, blk;
        round_src(rc, row, ecol, blk);
        loff[decltype(rc)::value] = round_bytes(rc, row, ecol);
        lblk[decltype(rc)::value] = blk;
    });
    auto issue_rounds = [&](auto bufc, int c, auto loc, auto hic) __attribute__((always_inline)) {
        constexpr int LO = decltype(loc)::value, HI = decltype(hic)::value;
        __attribute__((address_space(3))) unsigned char *stg = stage_lds(bufc);
        const int64_t t0 = a + (int64_t)c * C;
        const int last = (int)min<int64_t>(C, b - t0) - 1;
        const size_t slot = slot0 + c;
        const char *qb = reinterpret_cast<const char *>(q + ((size_t)t0 * hqk + hq) * DK);
        const char *kb = reinterpret_cast<const char *>(k + ((size_t)t0 * hqk + hq) * DK);
        const char *vb = reinterpret_cast<const char *>(v + ((size_t)t0 * hv + h) * dv + (size_t)s * DVS);
        const char *tb = reinterpret_cast<const char *>(tmat + (slot * hv + h) * (NU_T * 512));
        const char *db = reinterpret_cast<const char *>(dec + (slot * hv + h) * 4 * C);
        const bool full = last == C - 1;
        static_for<NR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;
            if constexpr (R < LO || R >= HI)
                return;
            uint32_t off = loff[R];
            if constexpr (R < RT0 || (R >= RV0 && R < RD0)) {
                if (!full) {   // ragged last chunk: rows past its end repeat its last row
                    int row, ecol, blk;
                    round_src(rc, row, ecol, blk);
                    off = round_bytes(rc, min(row, last), ecol);
                }
            }
            const char *base = R < RK0 ? qb : R < RT0 ? kb : R < RV0 ? tb : R < RD0 ? vb : db;
            const bool on = R < RT0 || (R >= RV0 && R < RD0) ? true
                            : R < RV0 ? (R - RT0) * NW + w < NU_T : w == 0;
            if (on)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                 (__attribute__((address_space(3))) void *)(stg + lblk[R]), 16, 0,
                                                 0);
        });
    };
    auto issue_stage = [&](auto bufc, int c) __attribute__((always_inline)) {
        issue_rounds(bufc, c, std::integral_constant<int, 0>{}, std::integral_constant<int, NR>{});
    };
    // the next chunk's loads in two parts: its Q and K units once this chunk's [Q;K] S products
    // have read theirs, the rest (T, V, record) just before the state update.  Measured on a
    // long varlen batch against other placements: 760-775 us per step's scans, against 855 with
    // the four parts issued at the start of the step's phases (Q, K first).
    constexpr int kPartEnd[2] = {RT0, NR};
    auto stage_part = [&](auto bufc, int c, auto pc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        issue_rounds(bufc, c, std::integral_constant<int, P == 0 ? 0 : kPartEnd[0]>{},
                     std::integral_constant<int, kPartEnd[P]>{});
    };
    auto stage_done = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // per-lane LDS byte offsets
    const int lin = 16 * lane;                                   // Q, T units
    const int kperm = 16 * (16 * G + (r16 ^ g4));                 // K units, fragment read
    const int e = (lane >> 2) & 3, qd = lane & 3;
    const int vtro = (8 * G + e) * VRB + 16 * ((2 * w + (qd >> 1)) ^ (2 * e)) + 8 * (qd & 1);
    // K^T transpose read: position of (chunk row 4 g + e of a unit, key quarter qd)
    const int ktpos = 16 * (16 * qd + ((g4 + e) ^ (4 * qd)));

    // A tiles: tile index -> (query row tile tr, key tile tc in Chain order)
    constexpr int NA = 12;
    auto a_tile = [](int idx, int &tr, int &tc) __attribute__((always_inline)) {
        tr = idx < 4 ? idx / 2 : 2 + (idx - 4) / 4;
        tc = idx < 4 ? idx % 2 : (idx - 4) % 4;
    };
    constexpr int NA_W = (NA + NW - 1) / NW;                     // tiles per wave, at most
    // the wave index as a scalar: the per-wave branches around matrix instructions must be
    // scalar branches (a matrix instruction runs for the whole wave whatever the exec mask,
    // so an exec-masked branch would let every wave run every tile's product)
    const int wu = __builtin_amdgcn_readfirstlane(w);

    // the output scale as a power of two, added to the record's G log2(e)
    const float log2_scale = __log2f(scale);
    // the previous chunk's output rows, from obuf to o: rows 8 w .. 8 w + 7 of this wave, lane l
    // moving 16 bytes of row 8 w + 4 u + l / 16 (u = 0, 1); rows past the chunk's end skipped
    const uint32_t olane = (uint32_t)(lane >> 4) * (uint32_t)(hv * dv) + (uint32_t)(8 * (lane & 15));
    int64_t t0c = 0;
    int lenc = 0;
    auto store_rows = [&]() __attribute__((always_inline)) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        bf16 *ob = o + ((size_t)t0c * hv + h) * dv + (size_t)s * DVS;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 8 * wu + 4 * u + (lane >> 4);
            const u32x4 v4 = *reinterpret_cast<const u32x4 *>(obuf + r * ORB + 16 * (lane & 15));
            if (r < lenc)
                *reinterpret_cast<u32x4 *>(ob + (size_t)(8 * wu + 4 * u) * hv * dv + olane) = v4;
        }
    };

    auto step = [&](auto bufc, int64_t t0, int len, bool carried, auto &&stage_hook) __attribute__((always_inline)) {
        const unsigned char *stg = stage_ptr(bufc);
        unsigned char *abw = abuf;
        auto frag = [&](int off) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8 *>(stg + off);
        };
        auto rec4 = [&](int arr, int row0) __attribute__((always_inline)) {
            return *reinterpret_cast<const f32x4 *>(stg + OFF_D + 4 * (arr * C + row0));
        };
        auto rec1 = [&](int arr, int row) __attribute__((always_inline)) {
            return *reinterpret_cast<const float *>(stg + OFF_D + 4 * (arr * C + row));
        };
        auto tr4 = [&](int off) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(stage_lds(bufc) + off));
        };

        // ---- the previous chunk's output rows (obuf was filled before the last barrier) ----
        if (carried)
            store_rows();
        // ---- [Q;K] S, and this wave's A tiles from the same fragments ----
        bf16x8 sb[NSK];
#pragma unroll
        for (int st = 0; st < NSK; ++st)
            sb[st] = CH::b_frag(sacc, st);
        f32x4 qacc[RT], xacc[RT], aacc[NA_W];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            qacc[rt] = zero4();
            xacc[rt] = zero4();
        }
#pragma unroll
        for (int i = 0; i < NA_W; ++i)
            aacc[i] = zero4();
#pragma unroll
        for (int st = 0; st < NSK; ++st) {
            bf16x8 fq[RT], fk[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                fq[rt] = frag(OFF_Q + (rt * NSK + st) * 1024 + lin);
                fk[rt] = frag(OFF_K + (rt * NSK + st) * 1024 + kperm);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                qacc[rt] = M::mma(sb[st], fq[rt], qacc[rt]);
                xacc[rt] = M::mma(fk[rt], sb[st], xacc[rt]);
            }
            // A^T tile (key rows CH::row(tc, .), query rows 16 tr + .) = K_tc . Q_tr
            static_for<NW>([&](auto wc) __attribute__((always_inline)) {
                constexpr int W = decltype(wc)::value;
                if (W != wu)
                    return;
                static_for<NA_W>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int I = decltype(ic)::value, IDX = W + I * NW;
                    if constexpr (IDX < NA) {
                        constexpr int TR = IDX < 4 ? IDX / 2 : 2 + (IDX - 4) / 4;
                        constexpr int TC = IDX < 4 ? IDX % 2 : (IDX - 4) % 4;
                        aacc[I] = M::mma(fk[TC], fq[TR], aacc[I]);
                    }
                });
            });
        }
        stage_hook(std::integral_constant<int, 0>{});
        // A: lane holds query row t = 16 tr + l % 16 and the 4 consecutive keys j0 .. j0 + 3,
        // j0 = CH::row(tc, 4 g); exp(G_t - G_j) is formed only for j <= t (log-space mask)
        static_for<NA_W>([&](auto ic) __attribute__((always_inline)) {
            constexpr int I = decltype(ic)::value;
            const int idx = wu + I * NW;
            if (idx < NA) {
                int tr, tc;
                a_tile(idx, tr, tc);
                const int t = 16 * tr + r16, j0 = CH::row(tc, g4);
                const float gt = rec1(0, t) + log2_scale;
                const f32x4 gj = rec4(0, j0);
                f32x4 av;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    av[i] = (j0 + i <= t) ? __builtin_amdgcn_exp2f(gt - gj[i]) * aacc[I][i] : 0.f;
                const u32x2 p0 = split_bf16x2(av[0], av[1]), p1 = split_bf16x2(av[2], av[3]);
                // keys j0 .. j0 + 3 = 32 (tc / 2) + 8 g + 4 (tc % 2) + {0..3}: unit (tr, tc / 2),
                // position r16 + 16 g, half tc % 2
                const int off = (2 * tr + (tc >> 1)) * 1024 + 16 * lane + 8 * (tc & 1);
                *reinterpret_cast<u32x2 *>(abw + off) = u32x2{p0[0], p1[0]};
                *reinterpret_cast<u32x2 *>(abw + AB + off) = u32x2{p0[1], p1[1]};
            }
        });

        // X = beta v - beta exp(G) (K S) on this lane's rows CH::row(rt, g4 + i)
        bf16x8 xb[NSC];
        {
            f32x4 t[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x4 vv = __builtin_bit_cast(bf16x4, tr4(OFF_V + CH::row(rt, 0) * VRB + vtro));
                const f32x4 vf = {(float)vv[0], (float)vv[1], (float)vv[2], (float)vv[3]};
                t[rt] = rec4(2, CH::row(rt, g4)) * vf - rec4(3, CH::row(rt, g4)) * xacc[rt];
            }
#pragma unroll
            for (int st = 0; st < NSC; ++st)
                xb[st] = CH::b_frag(t, st);
        }
        __builtin_amdgcn_sched_barrier(0);

        // Y = T_hi X + T_lo X (rows CH::row(rt, .)); T is zero in units (rt < 2, st = 1)
        f32x4 yacc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            yacc[rt] = zero4();
#pragma unroll
            for (int st = 0; st < NSC; ++st) {
                if (rt < 2 && st == 1)
                    continue;
                const int u = tform_unit(rt, st);
                const bf16x8 th = frag(OFF_T + u * 1024 + lin), tl = frag(OFF_T + (kTUnits + u) * 1024 + lin);
                yacc[rt] = M::mma(th, xb[st], yacc[rt]);
                yacc[rt] = M::mma(tl, xb[st], yacc[rt]);
            }
        }
        // hi/lo B fragments of Y and of lambda Y (contraction rows 32 st + 8 g + {0..7})
        bf16x8 yh[NSC], yl[NSC], dh[NSC], dl[NSC];
        {
            f32x4 ly[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                ly[rt] = rec4(1, CH::row(rt, g4)) * yacc[rt];
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int st = 0; st < NSC; ++st) {
                u32x4 a0, a1, b0, b1;
#pragma unroll
                for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const f32x4 &ty = yacc[2 * st + hlf], &tl = ly[2 * st + hlf];
                        const u32x2 sy = split_bf16x2(ty[2 * pr], ty[2 * pr + 1]);
                        const u32x2 sl = split_bf16x2(tl[2 * pr], tl[2 * pr + 1]);
                        a0[2 * hlf + pr] = sy[0];
                        a1[2 * hlf + pr] = sy[1];
                        b0[2 * hlf + pr] = sl[0];
                        b1[2 * hlf + pr] = sl[1];
                    }
                yh[st] = __builtin_bit_cast(bf16x8, a0);
                yl[st] = __builtin_bit_cast(bf16x8, a1);
                dh[st] = __builtin_bit_cast(bf16x8, b0);
                dl[st] = __builtin_bit_cast(bf16x8, b1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        stage_hook(std::integral_constant<int, 1>{});
        // S <- exp(G_last) S + K^T (lambda Y)_hi + K^T (lambda Y)_lo
        const float gl = __builtin_amdgcn_exp2f(rec1(0, C - 1));
#pragma unroll
        for (int sr = 0; sr < SR; ++sr) {
            sacc[sr] = sacc[sr] * gl;
#pragma unroll
            for (int st = 0; st < NSC; ++st) {
                const int u0 = OFF_K + ((2 * st) * NSK + (sr >> 1)) * 1024 + ktpos + 8 * (sr & 1);
                const s16x4 k0 = tr4(u0), k1 = tr4(u0 + NSK * 1024);
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const bf16x8 kt = __builtin_bit_cast(bf16x8, s16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]});
                sacc[sr] = M::mma(kt, dh[st], sacc[sr]);
                sacc[sr] = M::mma(kt, dl[st], sacc[sr]);
            }
        }

        // every wave's A tiles are in LDS, and every wave has stored the previous chunk's rows
        // from obuf (an LDS-only barrier: the next chunk's staging loads stay in flight)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // O^T = scale (Q S)^T diag(exp G) + Y^T A^T: lane l holds token row 16 rt + l % 16 and the
        // four columns 4 (l / 16) .. +3 of this wave's.  Key half 0 meets all four row tiles,
        // half 1 the last two (the others are zero): the fragments of a half are read together
        // and the row tiles' products interleaved.
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            qacc[rt] *= __builtin_amdgcn_exp2f(rec1(0, 16 * rt + r16) + log2_scale);
        static_for<NSC>([&](auto sc) __attribute__((always_inline)) {
            constexpr int ST = decltype(sc)::value, R0 = ST == 0 ? 0 : 2;
            bf16x8 ah[RT], al[RT];
#pragma unroll
            for (int rt = R0; rt < RT; ++rt) {
                const int off = (2 * rt + ST) * 1024 + 16 * lane;
                ah[rt] = *reinterpret_cast<const bf16x8 *>(abuf + off);
                al[rt] = *reinterpret_cast<const bf16x8 *>(abuf + AB + off);
            }
#pragma unroll
            for (int rt = R0; rt < RT; ++rt)
                qacc[rt] = M::mma(yh[ST], ah[rt], qacc[rt]);
#pragma unroll
            for (int rt = R0; rt < RT; ++rt)
                qacc[rt] = M::mma(yl[ST], ah[rt], qacc[rt]);
#pragma unroll
            for (int rt = R0; rt < RT; ++rt)
                qacc[rt] = M::mma(yh[ST], al[rt], qacc[rt]);
        });
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            *reinterpret_cast<bf16x4 *>(obuf + (16 * rt + r16) * ORB + 2 * (WC * wu + g4)) =
                bf16x4{(bf16)qacc[rt][0], (bf16)qacc[rt][1], (bf16)qacc[rt][2], (bf16)qacc[rt][3]};
        t0c = t0;
        lenc = len;
    };

    // ---- pipeline: buffers alternate from buffer 0; the barrier that ends a step also
    //      publishes its output rows in obuf to the next step ----
    const std::integral_constant<int, 0> buf0;
    const std::integral_constant<int, 1> buf1;
    issue_stage(buf0, c_begin);
    stage_done();
    for (int c = c_begin;;) {
        bool more = c + 1 < c_end;
        int64_t t0 = a + (int64_t)c * C;
        step(buf0, t0, (int)min<int64_t>(C, b - t0), c != c_begin, [&](auto pc) __attribute__((always_inline)) {
            if (more)
                stage_part(buf1, c + 1, pc);
        });
        stage_done();
        if (++c >= c_end) {
            store_rows();
            break;
        }
        more = c + 1 < c_end;
        t0 = a + (int64_t)c * C;
        step(buf1, t0, (int)min<int64_t>(C, b - t0), true, [&](auto pc) __attribute__((always_inline)) {
            if (more)
                stage_part(buf0, c + 1, pc);
        });
        stage_done();
        if (++c >= c_end) {
            store_rows();
            break;
        }
    }

    // ---- final state ----
#pragma unroll
    for (int sr = 0; sr < SR; ++sr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            state_out[state_base + (size_t)CH::row(sr, g4 + i) * dv + col0 + r16] = sacc[sr][i];
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------

template <typename E, int C, int DK, int NW>
static void launch_scan(const PrefillArgs &p, const SlotMap &map, const E *tmat, const E *amat, const float *dec,
                        const float *sin, float *sout, hipStream_t st)
{
    const int nv = p.dv / (16 * NW);
    const int64_t items = (int64_t)map.ranks * p.hqk;                  // (sequence, query/key head)
    const int64_t blocks = ((items + 7) / 8) * 8 * (p.hv / p.hqk) * nv;
    const ProfEvents ev = prof_events(PROF_SCAN, PROF_SCAN_PLAIN);
    hipExtLaunchKernelGGL((gdn_chunk_scan_kernel<E, C, DK, NW>), dim3((unsigned)blocks), dim3(NW * kWave), 0, st,
                          ev.start, ev.stop, 0, static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                          static_cast<const E *>(p.v), p.cu_seqlens, map, map.ranks, p.total_tokens, p.hqk, p.hv,
                          p.dv, tmat, amat, dec, sin, sout, static_cast<E *>(p.o), p.scale);
}

template <int DK, int DVS>
static void launch_scan_rows(const PrefillArgs &p, const SlotMap &map, const bf16 *wmat, const bf16 *mmat,
                             const float *dec, const float *sin, float *sout, hipStream_t st)
{
    const int nv = p.dv / DVS;
    const int64_t items = (int64_t)map.ranks * p.hqk;                  // (sequence, query/key head)
    const int64_t blocks = ((items + 7) / 8) * 8 * (p.hv / p.hqk) * nv;
    const ProfEvents ev = prof_events(PROF_SCAN, PROF_SCAN_ROWS);
    // part-A (Q, K, V) buffers: three where one workgroup per CU is the occupancy anyway
    // (dk = 128), two for smaller dk (two workgroups per CU)
    constexpr int NSTAGE = DK >= 128 ? 3 : 2;
    hipExtLaunchKernelGGL((gdn_chunk_scan_rows_kernel<bf16, 64, DK, DVS, NSTAGE>), dim3((unsigned)blocks),
                          dim3(kScanThreads), 0, st, ev.start, ev.stop, 0, static_cast<const bf16 *>(p.q),
                          static_cast<const bf16 *>(p.k), static_cast<const bf16 *>(p.v), p.cu_seqlens, map,
                          map.ranks, p.total_tokens, p.hqk, p.hv, p.dv, wmat, mmat, dec, sin, sout,
                          static_cast<bf16 *>(p.o), p.scale);
}

template <int DK, int NW, int CT>
static void launch_scan_bf16(const PrefillArgs &p, const SlotMap &map, const bf16 *wmat, const bf16 *mmat,
                             const float *dec, const float *sin, float *sout, hipStream_t st)
{
    const int nv = p.dv / (16 * CT * NW);
    const int64_t items = (int64_t)map.ranks * p.hqk;                  // (sequence, query/key head)
    const int64_t blocks = ((items + 7) / 8) * 8 * (p.hv / p.hqk) * nv;
    const ProfEvents ev = prof_events(PROF_SCAN, PROF_SCAN_WIDE);
    hipExtLaunchKernelGGL((gdn_chunk_scan_bf16_kernel<DK, NW, CT>), dim3((unsigned)blocks), dim3(NW * kWave), 0,
                          st, ev.start, ev.stop, 0, static_cast<const bf16 *>(p.q), static_cast<const bf16 *>(p.k),
                          static_cast<const bf16 *>(p.v), p.cu_seqlens, map, map.ranks, p.total_tokens, p.hqk, p.hv,
                          p.dv, wmat, mmat, dec, sin, sout, static_cast<bf16 *>(p.o), p.scale);
}

template <int DK, int NW>
static void launch_scan_tform(const PrefillArgs &p, const SlotMap &map, const bf16 *tmat, const float *dec,
                              const float *sin, float *sout, hipStream_t st)
{
    const int nv = p.dv / (16 * NW);
    const int64_t items = (int64_t)map.ranks * p.hqk;                  // (sequence, query/key head)
    const int64_t blocks = ((items + 7) / 8) * 8 * (p.hv / p.hqk) * nv;
    const ProfEvents ev = prof_events(PROF_SCAN, PROF_SCAN_TFORM);
    hipExtLaunchKernelGGL((gdn_chunk_scan_tform_kernel<DK, NW>), dim3((unsigned)blocks), dim3(NW * kWave), 0, st,
                          ev.start, ev.stop, 0, static_cast<const bf16 *>(p.q), static_cast<const bf16 *>(p.k),
                          static_cast<const bf16 *>(p.v), p.cu_seqlens, map, map.ranks, p.total_tokens, p.hqk, p.hv,
                          p.dv, tmat, dec, sin, sout, static_cast<bf16 *>(p.o), p.scale);
}

// Batches of at most this many sequences are scanned longest first.
constexpr int32_t kMaxOrderedSeqs = 4096;

// The gated RMSNorm of a prefill's output rows, if asked for: in place, after the scans.
static hipError_t launch_prefill_norm(const PrefillArgs &p)
{
    if (p.norm_z && p.total_tokens > 0) {
        NormArgs n{};
        n.hv = p.hv;
        n.dv = p.dv;
        n.io_dtype = p.io_dtype;
        n.o = p.o;
        n.z = p.norm_z;
        n.weight = p.norm_weight;
        n.y = p.o;
        n.tokens = p.total_tokens;
        n.eps = p.norm_eps;
        n.stream = p.stream;
        const hipError_t e = launch_norm(n);
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

template <typename E, int C, int DK>
static hipError_t launch_prefill_t(const PrefillArgs &p)
{
    hipStream_t st = static_cast<hipStream_t>(p.stream);
    // workspace: [chunk table, scan order, slot entries | T (or W) matrices | A (or M) matrices |
    // decay records]
    constexpr bool kAbsorbed = AbsorbedForm<E, C>::value;
    static_assert(kAbsorbed == (std::is_same<E, bf16>::value && C == 64), "matches prefill_absorbed()");
    int32_t *chunk_start = reinterpret_cast<int32_t *>(p.workspace);
    E *tmat = reinterpret_cast<E *>(static_cast<char *>(p.workspace) + p.table_bytes);
    E *amat = tmat + (size_t)p.max_chunks * p.hv * (kAbsorbed ? DK : C) * C;
    float *dec = reinterpret_cast<float *>(amat + (size_t)p.max_chunks * p.hv * C * C);
    // The gated RMSNorm of the output rows, if asked for: in place, after the scans.
    auto finish = [&]() -> hipError_t { return launch_prefill_norm(p); };

    // Whole-head batches (many (sequence, head) pairs, no split by length) take the T form:
    // the prep writes T alone and the whole-head scan forms A and Y = T X itself.
    const bool mixed = p.long_ranks > 0 && p.long_ranks < p.num_seqs;
    const bool tform = kAbsorbed && DK == 128 && (int64_t)p.num_seqs * p.hv > 64 && !mixed;
    auto scan = [&](const SlotMap &map, const float *sin, float *sout) {
        if constexpr (std::is_same<E, bf16>::value && C == 64) {
            // 32 columns per wave; a whole 128-column head per workgroup when the batch
            // has enough (sequence, head) pairs to fill the chip, else 64 columns
            // Few (sequence, head) pairs: the chain of chunk steps is latency-bound, so a
            // step is spread over the rows of 4 waves (16-column slices, 8 workgroups per
            // pair).  More pairs: whole 128-column heads per workgroup, 8 waves of 16
            // columns each (two waves per SIMD hide each other's latencies).  Measured
            // crossover: 64 pairs (1024-token sequences, 16 chunk steps).
            const int64_t pairs = (int64_t)p.num_seqs * p.hv;
            if constexpr (DK == 128) {
                if (tform) {
                    launch_scan_tform<DK, 8>(p, map, tmat, dec, sin, sout, st);
                    return;
                }
                if (mixed) {
                    // Mixed batch (host offsets: a few sequences whose chains would bound a
                    // whole-head scan): its longest sequences (the first ranks) in the
                    // row-split scan, the rest in the whole-head scan.
                    // (In segments or windows past the rest's chunks only the first.)
                    SlotMap lm = map, rm = map;
                    lm.ranks = p.long_ranks;
                    rm.rank0 = map.rank0 + p.long_ranks;
                    rm.ranks = map.ranks - p.long_ranks;
                    launch_scan_rows<DK, 16>(p, lm, tmat, amat, dec, sin, sout, st);
                    if (p.rest_chunks < 0 || map.seg_first < p.rest_chunks || map.seg_first == 0)
                        launch_scan_bf16<DK, 8, 1>(p, rm, tmat, amat, dec, sin, sout, st);
                    return;
                }
                if (pairs > 64) {
                    launch_scan_bf16<DK, 8, 1>(p, map, tmat, amat, dec, sin, sout, st);
                    return;
                }
            }
            launch_scan_rows<DK, 16>(p, map, tmat, amat, dec, sin, sout, st);
        } else {
            launch_scan<E, C, DK, 2>(p, map, tmat, amat, dec, sin, sout, st);
        }
    };
    auto prep = [&](const SlotMap &map, int64_t slots) {
        const ProfEvents ev = prof_events(PROF_PREP);
        // grid: (chunk slot, query/key head); in the absorbed form (one value head per
        // workgroup) 1-D, ceil(slots * HQK / 8) * 8 * group blocks (xcd_group)
        const int64_t items = slots * p.hqk;
        const dim3 grid = AbsorbedForm<E, C>::value
                              ? dim3((unsigned)(((items + 7) / 8) * 8 * (p.hv / p.hqk)))
                              : dim3((unsigned)slots, (unsigned)p.hqk);
        auto go = [&](auto kern) {
            hipExtLaunchKernelGGL(kern, grid, dim3(PrepWaves<E, C>::value * kWave), 0, st, ev.start, ev.stop, 0,
                                  static_cast<const E *>(p.q), static_cast<const E *>(p.k), p.g, p.beta,
                                  p.cu_seqlens, map, p.num_seqs, p.total_tokens, p.hqk, p.hv, tmat, amat, dec,
                                  p.scale, (int32_t)slots);
        };
        if constexpr (!kAbsorbed) {
            go(gdn_prep_kernel<E, C, DK, kPrepDirect>);
        } else {
            if constexpr (DK == 128) {
                if (tform) {
                    go(gdn_prep_kernel<E, C, DK, kPrepTForm>);
                    return;
                }
            }
            go(gdn_prep_kernel<E, C, DK, kPrepAbsorbed>);
        }
    };

    // Longest sequences first in the scans (their chains of chunk steps bound the time),
    // unless the host offsets show the batch in that order already.  In the single launch
    // over the chunk table the ranking runs in the table's launch.
    int32_t *order = nullptr;
    if (p.num_seqs > 1 && p.num_seqs <= kMaxOrderedSeqs && !p.ordered)
        order = chunk_start + p.num_seqs + 1;   // after the chunk table
    const unsigned rank_blocks = (unsigned)((p.num_seqs + kThreads - 1) / kThreads);

    if (p.seg_len > 0) {
        if (order) {
            const ProfEvents ev = prof_events(PROF_CHUNK_TABLE);
            hipExtLaunchKernelGGL(gdn_seq_order_kernel, dim3(rank_blocks), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                                  p.cu_seqlens, p.num_seqs, p.total_tokens, order);
        }
        // Segment mode: local chunks [s0, s0 + seg_len) of every sequence per step.
        for (int32_t s0 = 0; s0 < p.max_seq_chunks; s0 += p.seg_len) {
            const SlotMap map{nullptr, s0, p.seg_len, order, 0, p.num_seqs};
            prep(map, (int64_t)p.num_seqs * p.seg_len);
            scan(map, s0 == 0 ? p.initial_state : p.final_state, p.final_state);
        }
        return finish();
    }

    int2 *slot_info = reinterpret_cast<int2 *>(static_cast<char *>(p.workspace) + prefill_slot_info_offset(p.num_seqs));
    // One window over every chunk, or (host offsets, long ranks) windows of win_len local chunks
    // of every sequence, with win_slots[j] slots each: table, prep and scans per window, the
    // state carried in final_state between windows.
    const bool windows = p.win_len > 0 && p.win_slots;
    const int32_t win = windows ? p.win_len : INT32_MAX;
    for (int32_t w0 = 0, j = 0;; w0 += win, ++j) {
        const int32_t slots = windows ? (int32_t)p.win_slots[j] : p.max_chunks;
        {
            const ProfEvents ev = prof_events(PROF_CHUNK_TABLE);
            const unsigned info_blocks = (unsigned)((slots + kSlotsPerTableBlock - 1) / kSlotsPerTableBlock);
            int32_t *const rank = w0 == 0 ? order : nullptr;   // the order stays for later windows
            const unsigned blocks = std::max(std::max(rank ? rank_blocks : 1u, info_blocks), 1u);
            hipExtLaunchKernelGGL(gdn_chunk_table_kernel, dim3(blocks), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                                  p.cu_seqlens, p.num_seqs, p.total_tokens, (int32_t)C, slots, chunk_start, rank,
                                  slot_info, w0, win);
        }
        const SlotMap map{chunk_start, w0, win, order, 0, p.num_seqs, slot_info};
        if (slots > 0)
            prep(map, slots);
        scan(map, w0 == 0 ? p.initial_state : p.final_state, p.final_state);
        if (!windows || w0 + win >= p.max_seq_chunks)
            break;
    }
    return finish();
}

// The library's own device scratch behind gdn_prefill_chunked_noalloc: one copy per device,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the kernels are given the address that hipGetSymbolAddress returns for
// the device, looked up once per device with that device current.
__device__ __align__(256) unsigned char scratch[kPrefillScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
void *g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t prefill_scratch(hipStream_t stream, void **ptr, size_t *bytes)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = kPrefillScratchBytes;
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs &p)
{
    // Every sequence at most kShortPrefillTokens long (known from host offsets), or fp32 io at
    // dk = 128 (no chunked kernel): one token-recurrent launch, no chunk matrices; then the
    // norm, if asked for.
    const bool short_batch = p.max_len >= 0 && p.max_len <= kShortPrefillTokens;
    const bool fp32_wide = p.io_dtype == 0 && p.dk == 128;
    if ((short_batch || fp32_wide) && short_prefill_supported(p.dk, p.dv)) {
        const hipError_t e = launch_short_prefill(p);
        if (e != hipSuccess)
            return e;
        return launch_prefill_norm(p);
    }
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
