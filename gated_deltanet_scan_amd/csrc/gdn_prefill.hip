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
// decay matrix, the solve of (I + N), the decayed query-key matrix) is done
// for all chunks at once by the prep kernel; the scan kernel then walks the
// chunks of each sequence in order with the state slice held on chip
// ("state propagated sequentially between chunks, intra-chunk work as
// batched products": Candle pull-request page, section Chunked GatedDeltaNet
// Scan).  Three kernels per call:
//   gdn_chunk_table_kernel  chunk offsets of every sequence (integer scan)
//   gdn_prep_kernel         per (chunk, query/key head): K K^T and Q K^T on
//                           the matrix cores; per value head of the group:
//                           G, log-space-masked exp(G_t - G_j), N, the unit
//                           lower-triangular inverse T = (I + N)^-1 by
//                           forward substitution, A = decayed Q K^T
//   gdn_chunk_scan_kernel   per (sequence, value head, dv-slice): for each
//                           chunk, [Q;K] S, X = diag(beta)(V - diag(exp G) K S),
//                           D = T X, O = diag(exp G) Q S + A D, S update.
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

// ---------------------------------------------------------------------------
// Prep kernel.  Grid (max_chunks, HQK); entries past the real chunk count
// exit at once.  Writes, for every value head h of the group and chunk e,
//   tmat[e][h] = (I + N)^-1   (C x C, row-major, unit lower triangular)
//   amat[e][h] = [exp(G_t - G_j) q_t.k_j]_{j<=t}  (C x C, zero above)
// ---------------------------------------------------------------------------
template <int C>
__device__ inline void solve_unit_lower_column(const float *Nm, int ldf, int col, float (&x)[C])
{
    // Column `col` of (I + N)^-1: x_t = [t == col] - sum_{j<t} N[t][j] x_j.
#pragma unroll
    for (int t = 0; t < C; ++t) {
        float s = (t == col) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < t; ++j)
            s -= Nm[t * ldf + j] * x[j];
        x[t] = s;
    }
}

template <typename E, int C, int DK>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_start, int32_t num_seqs, int64_t total_tokens, int32_t hqk,
    int32_t hv, E *__restrict__ tmat, E *__restrict__ amat)
{
    constexpr int PAD = LdsPad<E>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDF = C + 4;
    constexpr int RT = C / 16;
    constexpr int HB = 2;  // value heads per pass
    constexpr int IN_BYTES = 2 * C * LDK * (int)sizeof(E);
    constexpr int N_BYTES = HB * C * LDF * (int)sizeof(float);
    constexpr int U_BYTES = IN_BYTES > N_BYTES ? IN_BYTES : N_BYTES;
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;

    __shared__ __attribute__((aligned(16))) unsigned char smem_u[U_BYTES];
    __shared__ __attribute__((aligned(16))) float KK[C * LDF];
    __shared__ __attribute__((aligned(16))) float QK[C * LDF];
    __shared__ float Gs[HB][C];
    __shared__ float Bs[HB][C];
    E *Ks = reinterpret_cast<E *>(smem_u);
    E *Qs = Ks + C * LDK;
    float *Nm = reinterpret_cast<float *>(smem_u);  // reused once the Gram products are done

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int32_t e = blockIdx.x;
    const int hq = blockIdx.y;
    if (e >= chunk_start[num_seqs])
        return;
    const int n = find_sequence(chunk_start, num_seqs, e);
    int64_t a, b;
    seq_range(cu, n, total_tokens, a, b);
    const int64_t t0 = a + (int64_t)(e - chunk_start[n]) * C;
    const int len = (int)min<int64_t>(C, b - t0);

    // Q and K rows of this query/key head; rows past the end are zero.
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

    // K K^T and Q K^T, lower block triangle only (tile row >= tile column).
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

    const int group = hv / hqk;
    for (int hb = 0; hb < group; hb += HB) {
        const int nh = min(HB, group - hb);
        // G = in-chunk inclusive cumulative sum of g; padding tokens carry g = 0, beta = 0.
        if (wave < nh) {
            const int h = hq * group + hb + wave;
            float gv = 0.f, bv = 0.f;
            if (lane < len) {
                gv = g[(size_t)(t0 + lane) * hv + h];
                bv = beta[(size_t)(t0 + lane) * hv + h];
            }
            const float G = wave_inclusive_sum(gv, lane);
            if (lane < C) {
                Gs[wave][lane] = G;
                Bs[wave][lane] = bv;
            }
        }
        __syncthreads();
        // exp(G_t - G_j) only for j <= t, where the exponent is <= 0 (log-space mask).
        for (int idx = tid; idx < nh * C * C; idx += kThreads) {
            const int hh = idx / (C * C);
            const int rem = idx - hh * C * C;
            const int t = rem / C, j = rem - (rem / C) * C;
            const int h = hq * group + hb + hh;
            float ed = 0.f;
            if (j <= t)
                ed = __expf(Gs[hh][t] - Gs[hh][j]);
            Nm[(hh * C + t) * LDF + j] = (j < t) ? Bs[hh][t] * ed * KK[t * LDF + j] : 0.f;
            amat[((size_t)e * hv + h) * C * C + rem] = (E)(ed * QK[t * LDF + j]);
        }
        __syncthreads();
        if (wave < nh && lane < C) {
            const int h = hq * group + hb + wave;
            float x[C];
            solve_unit_lower_column<C>(Nm + wave * C * LDF, LDF, lane, x);
            E *out = tmat + ((size_t)e * hv + h) * C * C + lane;
#pragma unroll
            for (int t = 0; t < C; ++t)
                out[t * C] = (E)x[t];
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
// Block index -> work: the 8 XCDs take workgroups round-robin, so the dv
// slices of one (sequence, head) are placed on one XCD (shared Q, K, T, A
// reads then hit the same L2).
// ---------------------------------------------------------------------------
template <typename E, int C, int DK, int DVS>
__global__ __launch_bounds__(kThreads) void gdn_chunk_scan_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_start, int32_t num_seqs, int64_t total_tokens, int32_t hqk,
    int32_t hv, int32_t dv, const E *__restrict__ tmat, const E *__restrict__ amat,
    const float *initial_state, float *final_state, E *__restrict__ o, float scale)
{
    constexpr int PAD = LdsPad<E>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int RT = C / 16, CT = DVS / 16, SR = DK / 16;
    constexpr int NO = (RT * CT + kWaves - 1) / kWaves;
    constexpr int NS = (SR * CT + kWaves - 1) / kWaves;
    constexpr int VN = Vec16<E>::n;
    typedef typename Vec16<E>::type V16;
    constexpr int QK_VECS = C * DK / VN, QK_PER = (QK_VECS + kThreads - 1) / kThreads;
    constexpr int CC_VECS = C * C / VN, CC_PER = (CC_VECS + kThreads - 1) / kThreads;
    constexpr int V_VECS = C * DVS / VN, V_PER = (V_VECS + kThreads - 1) / kThreads;
    static_assert(C <= kWave, "one lane per token of a chunk");

    __shared__ __attribute__((aligned(16))) E Ks[C * LDK];
    __shared__ __attribute__((aligned(16))) E Qs[C * LDK];
    __shared__ __attribute__((aligned(16))) E Kt[DK * LDC];
    __shared__ __attribute__((aligned(16))) E Ts[C * LDC];
    __shared__ __attribute__((aligned(16))) E As[C * LDC];
    __shared__ __attribute__((aligned(16))) E Vs[C * DVS];
    __shared__ __attribute__((aligned(16))) E Xt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E Dt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E LDt[DVS * LDC];
    __shared__ __attribute__((aligned(16))) E St[DVS * LDK];
    __shared__ float Gam[C], Lam[C], Bet[C];
    __shared__ float GamL;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
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
    const int32_t cs0 = chunk_start[n];
    const int nchunks = chunk_start[n + 1] - cs0;
    const size_t state_base = (size_t)(n * hv + h) * DK * dv + (size_t)s * DVS;

    // ---- state slice into accumulators, bf16 copy into St ----
    f32x4 sacc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int st = wave + u * kWaves;
        sacc[u] = zero4();
        if (st < SR * CT) {
            const int sr = st / CT, ct = st % CT;
            if (initial_state) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[u][i] = initial_state[state_base + (size_t)(sr * 16 + tile_row(lane, i)) * dv +
                                               ct * 16 + tile_col(lane)];
            }
            store4(St + (ct * 16 + tile_col(lane)) * LDK + sr * 16 + tile_row(lane, 0), sacc[u][0],
                   sacc[u][1], sacc[u][2], sacc[u][3]);
        }
    }

    // ---- chunk inputs: global -> registers (prefetch) -> LDS ----
    V16 rq[QK_PER], rk[QK_PER], rtm[CC_PER], ram[CC_PER], rv[V_PER];
    float rg = 0.f, rb = 0.f;
    int64_t pre_t0 = a;
    int pre_len = 0;

    auto load_chunk = [&](int c) {
        const int64_t t0 = a + (int64_t)c * C;
        const int len = (int)min<int64_t>(C, b - t0);
        pre_t0 = t0;
        pre_len = len;
        const size_t ent = ((size_t)(cs0 + c) * hv + h) * C * C;
#pragma unroll
        for (int u = 0; u < QK_PER; ++u) {
            const int i = tid + u * kThreads;
            rq[u] = (V16)(E)0.f;
            rk[u] = (V16)(E)0.f;
            if (i < QK_VECS) {
                const int r = i / (DK / VN), c0 = (i % (DK / VN)) * VN;
                if (r < len) {
                    const size_t off = ((size_t)(t0 + r) * hqk + hq) * DK + c0;
                    rq[u] = *reinterpret_cast<const V16 *>(q + off);
                    rk[u] = *reinterpret_cast<const V16 *>(k + off);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < CC_PER; ++u) {
            const int i = tid + u * kThreads;
            if (i < CC_VECS) {
                rtm[u] = *reinterpret_cast<const V16 *>(tmat + ent + (size_t)i * VN);
                ram[u] = *reinterpret_cast<const V16 *>(amat + ent + (size_t)i * VN);
            }
        }
#pragma unroll
        for (int u = 0; u < V_PER; ++u) {
            const int i = tid + u * kThreads;
            rv[u] = (V16)(E)0.f;
            if (i < V_VECS) {
                const int r = i / (DVS / VN), c0 = (i % (DVS / VN)) * VN;
                if (r < len)
                    rv[u] = *reinterpret_cast<const V16 *>(v + ((size_t)(t0 + r) * hv + h) * dv +
                                                           (size_t)s * DVS + c0);
            }
        }
        rg = 0.f;
        rb = 0.f;
        if (wave == 0 && lane < len) {
            rg = g[(size_t)(t0 + lane) * hv + h];
            rb = beta[(size_t)(t0 + lane) * hv + h];
        }
    };

    auto store_chunk = [&]() {
#pragma unroll
        for (int u = 0; u < QK_PER; ++u) {
            const int i = tid + u * kThreads;
            if (i < QK_VECS) {
                const int r = i / (DK / VN), c0 = (i % (DK / VN)) * VN;
                *reinterpret_cast<V16 *>(Qs + r * LDK + c0) = rq[u];
                *reinterpret_cast<V16 *>(Ks + r * LDK + c0) = rk[u];
#pragma unroll
                for (int j = 0; j < VN; ++j)
                    Kt[(c0 + j) * LDC + r] = rk[u][j];
            }
        }
#pragma unroll
        for (int u = 0; u < CC_PER; ++u) {
            const int i = tid + u * kThreads;
            if (i < CC_VECS) {
                const int r = (i * VN) / C, c0 = (i * VN) % C;
                *reinterpret_cast<V16 *>(Ts + r * LDC + c0) = rtm[u];
                *reinterpret_cast<V16 *>(As + r * LDC + c0) = ram[u];
            }
        }
#pragma unroll
        for (int u = 0; u < V_PER; ++u) {
            const int i = tid + u * kThreads;
            if (i < V_VECS)
                *reinterpret_cast<V16 *>(Vs + i * VN) = rv[u];
        }
        if (wave == 0) {
            const float G = wave_inclusive_sum(rg, lane);   // lanes >= len add 0
            const float Glast = __shfl(G, kWave - 1, kWave);
            if (lane < C) {
                Gam[lane] = expf(G);
                Lam[lane] = expf(Glast - G);
                Bet[lane] = rb;
            }
            if (lane == 0)
                GamL = expf(Glast);
        }
    };

    if (nchunks > 0) {
        load_chunk(0);
        store_chunk();
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = pre_t0;
        const int len = pre_len;
        if (c + 1 < nchunks)
            load_chunk(c + 1);

        // P1: Q S and K S; X = diag(beta)(V - diag(exp G) K S) -> Xt (transposed)
        f32x4 oacc[NO];
#pragma unroll
        for (int u = 0; u < NO; ++u) {
            const int it = wave + u * kWaves;
            oacc[u] = zero4();
            if (it < RT * CT) {
                const int rt = it / CT, ct = it % CT;
                const f32x4 qs = mma_tile<E, DK>(zero4(), Qs + rt * 16 * LDK, LDK, St + ct * 16 * LDK, LDK, lane);
                const f32x4 ks = mma_tile<E, DK>(zero4(), Ks + rt * 16 * LDK, LDK, St + ct * 16 * LDK, LDK, lane);
                const int col = ct * 16 + tile_col(lane);
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + tile_row(lane, i);
                    x[i] = Bet[r] * (to_f32(Vs[r * DVS + col]) - Gam[r] * ks[i]);
                    oacc[u][i] = Gam[r] * qs[i];
                }
                store4(Xt + col * LDC + rt * 16 + tile_row(lane, 0), x[0], x[1], x[2], x[3]);
            }
        }
        __syncthreads();

        // P2: D = T X -> Dt and (diag(lambda) D) -> LDt, both transposed
#pragma unroll
        for (int u = 0; u < NO; ++u) {
            const int it = wave + u * kWaves;
            if (it < RT * CT) {
                const int rt = it / CT, ct = it % CT;
                const f32x4 d = mma_tile<E, C>(zero4(), Ts + rt * 16 * LDC, LDC, Xt + ct * 16 * LDC, LDC, lane);
                const int col = ct * 16 + tile_col(lane);
                const int r0 = rt * 16 + tile_row(lane, 0);
                store4(Dt + col * LDC + r0, d[0], d[1], d[2], d[3]);
                store4(LDt + col * LDC + r0, Lam[r0] * d[0], Lam[r0 + 1] * d[1], Lam[r0 + 2] * d[2],
                       Lam[r0 + 3] * d[3]);
            }
        }
        __syncthreads();

        // P3: O = diag(exp G) Q S + A D, scaled, to global
#pragma unroll
        for (int u = 0; u < NO; ++u) {
            const int it = wave + u * kWaves;
            if (it < RT * CT) {
                const int rt = it / CT, ct = it % CT;
                oacc[u] = mma_tile<E, C>(oacc[u], As + rt * 16 * LDC, LDC, Dt + ct * 16 * LDC, LDC, lane);
                const int col = s * DVS + ct * 16 + tile_col(lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + tile_row(lane, i);
                    if (r < len)
                        o[((size_t)(t0 + r) * hv + h) * dv + col] = (E)(scale * oacc[u][i]);
                }
            }
        }
        // P4: S <- exp(G_last) S + K^T diag(lambda) D; refresh the transposed copy
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int st = wave + u * kWaves;
            if (st < SR * CT) {
                const int sr = st / CT, ct = st % CT;
                f32x4 acc = sacc[u] * GamL;
                acc = mma_tile<E, C>(acc, Kt + sr * 16 * LDC, LDC, LDt + ct * 16 * LDC, LDC, lane);
                sacc[u] = acc;
                store4(St + (ct * 16 + tile_col(lane)) * LDK + sr * 16 + tile_row(lane, 0), acc[0], acc[1],
                       acc[2], acc[3]);
            }
        }
        __syncthreads();
        if (c + 1 < nchunks)
            store_chunk();
        __syncthreads();
    }

    // ---- final state ----
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int st = wave + u * kWaves;
        if (st < SR * CT) {
            const int sr = st / CT, ct = st % CT;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[state_base + (size_t)(sr * 16 + tile_row(lane, i)) * dv + ct * 16 + tile_col(lane)] =
                    sacc[u][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------
template <typename E, int C, int DK>
static hipError_t launch_prefill_t(const PrefillArgs &p)
{
    constexpr int DVS = 16;
    int32_t *chunk_start = reinterpret_cast<int32_t *>(p.workspace);
    E *tmat = reinterpret_cast<E *>(static_cast<char *>(p.workspace) + p.table_bytes);
    E *amat = tmat + (size_t)p.max_chunks * p.hv * C * C;
    hipStream_t st = static_cast<hipStream_t>(p.stream);

    prof_begin(PROF_CHUNK_TABLE, st);
    hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(kThreads), 0, st, p.cu_seqlens,
                       p.num_seqs, p.total_tokens, (int32_t)C, p.max_chunks, chunk_start);
    prof_end(st);
    if (p.max_chunks > 0) {
        prof_begin(PROF_PREP, st);
        hipLaunchKernelGGL((gdn_prep_kernel<E, C, DK>), dim3(p.max_chunks, p.hqk), dim3(kThreads), 0, st,
                           static_cast<const E *>(p.q), static_cast<const E *>(p.k), p.g, p.beta,
                           p.cu_seqlens, chunk_start, p.num_seqs, p.total_tokens, p.hqk, p.hv, tmat, amat);
        prof_end(st);
    }
    const int nv = p.dv / DVS;
    const int64_t pairs = (int64_t)p.num_seqs * p.hv;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * nv;
    if (blocks > 0) {
        prof_begin(PROF_SCAN, st);
        hipLaunchKernelGGL((gdn_chunk_scan_kernel<E, C, DK, DVS>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           static_cast<const E *>(p.q), static_cast<const E *>(p.k),
                           static_cast<const E *>(p.v), p.g, p.beta, p.cu_seqlens, chunk_start, p.num_seqs,
                           p.total_tokens, p.hqk, p.hv, p.dv, tmat, amat, p.initial_state, p.final_state,
                           static_cast<E *>(p.o), p.scale);
        prof_end(st);
    }
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
