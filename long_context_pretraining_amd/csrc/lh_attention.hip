// Causal softmax attention on the gathered sub-sequence (page "skillsmp.com
// ... lighthouse-attention", Stage 3: dense attention with the standard S x S
// causal mask; gist.science Methodology 2C), forward and backward, on the
// gfx950 matrix cores.  This is the only dense contraction of the layer.
//
// Design (wave64, v_mfma_f32_32x32x16_bf16; f32 uses v_mfma_f32_32x32x2_f32):
//  * Forward and dQ compute the TRANSPOSED score tile S^T = K Q^T, so each lane
//    owns one query column: the softmax row statistics are per-lane scalars
//    plus one exchange with the lane 32 away.  P^T is then fed straight back
//    as the B operand of O^T += V^T P^T (see the k-order note in lh_device.h),
//    with V^T read from a transposed copy made by the gather.
//  * dK/dV computes S = Q K^T (each lane owns one key column) and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS, again without moving P or dS across
//    lanes.  dQ is a separate pass over key tiles (recomputing P), so every
//    output is written exactly once: deterministic, no atomics.
//  * K/V (or Q/dO) tiles are staged through LDS, double buffered with a
//    register prefetch of the next tile; rows padded against bank conflicts.
//  * Blocks are ordered longest-first (causal work grows with the block
//    index), heads interleaved.
#include <math.h>

#include "lh_device.h"
#include "lh_internal.h"

namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kBN = 64;         // keys (fwd, dQ) or queries (dK/dV) per LDS tile
constexpr int kWaveRows = 64;   // queries (fwd, dQ) or keys (dK/dV) per wave
constexpr int kBlockRows = 4 * kWaveRows;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDkdvNW = 8;      // waves per dK/dV block (32 keys each; d = 128: 4)

// Blocks per CU the forward and dQ kernels are built for: two (two waves per
// SIMD) where a wave's registers fit in 256, one for d = 128, whose
// accumulators and fragments need the whole register file of a SIMD.
template <typename T, int D> constexpr int kBlocksPerCu = D * (int)sizeof(T) > 128 ? 1 : 2;

struct AttnK {
    int64_t BH, S, S_pad;
    float scale, scale_log2;
    int nblk;   // row blocks per head
};

__device__ __forceinline__ void block_order(const AttnK& a, bool longest_last_rows, int64_t& bh, int& blk) {
    const int64_t x = blockIdx.x;
    bh = x % a.BH;
    const int i = (int)(x / a.BH);
    blk = longest_last_rows ? (a.nblk - 1 - i) : i;
}

// The bf16 forward multiplies V by P in two parts, P = hi + lo with hi the
// bf16 rounding of P and lo the bf16 rounding of the remainder (split_frag),
// so that the f32 output carries P to about 2^-17 relative.  Without it the
// output would use P rounded to 8 bits while the backward recomputes P in
// f32, and D = rowsum(dO * O) would then be off by ~2^-9 |dP| in rows
// dominated by a few keys -- an error the products with K and Q magnify.
template <typename T> constexpr bool kSplitP = sizeof(T) == 2;
// bf16 products that contract over the sequence read their operand across the
// rows of a row-major tile (tile_frag_tr); f32 reads a transposed copy.
template <typename T> constexpr bool kTr = sizeof(T) == 2;

// ---------------------------------------------------------------------------
// Forward: O = softmax(scale Q K^T, causal) V and LSE, per 256-query block.
// The output is written in f32 (and, when Ot is given, also in T).  Vop is V
// row-major [S][D] for bf16 and V^T [D][S_pad] for f32.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, (kBlocksPerCu<T, D>)) void attn_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                            const T* __restrict__ Vop, float* __restrict__ O32,
                                                            T* __restrict__ Ot, float* __restrict__ LSE, AttnK a) {
    typedef typename Frag<T>::type F;
    constexpr int KROWB = D * (int)sizeof(T), VROWB = kTr<T> ? KROWB : kBN * (int)sizeof(T);
    constexpr int KBYTES = kBN * KROWB, VBYTES = kTr<T> ? KBYTES : D * VROWB, BUF = KBYTES + VBYTES;
    extern __shared__ __align__(16) unsigned char smem[];

    int64_t bh; int qb;
    block_order(a, true, bh, qb);
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 31, h = lane >> 5;
    const int64_t S = a.S;
    const T* Qh = Q + bh * S * D;
    const T* Kh = K + bh * S * D;
    const T* Vh = Vop + (kTr<T> ? bh * S * D : bh * D * a.S_pad);

    const int64_t q_blk0 = (int64_t)qb * kBlockRows;
    const int64_t q_base = q_blk0 + wave * kWaveRows;
    const int64_t q_last_blk = (q_blk0 + kBlockRows < S ? q_blk0 + kBlockRows : S) - 1;
    const int64_t q_last_w = (q_base + kWaveRows < S ? q_base + kWaveRows : S) - 1;
    const int ntiles = (int)(q_last_blk / kBN) + 1;

    F qf[2][D / 16];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int64_t q = q_base + 32 * cb + col;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qf[cb][c] = load8_or_zero(Qh + q * D + 16 * c + 8 * h, q < S);
    }
    floatx16 o[2][D / 32];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[cb][db] = floatx16{};
    // Running reference max (log2 units) and row sum per query.  The output is
    // rescaled only when the max grows by more than 2^8, so P stays below 256.
    float m_i[2] = {-INFINITY, -INFINITY}, l_i[2] = {0.f, 0.f};
    const float c = a.scale_log2;
    // last key each query may see, as an int32 offset from the tile
    const int q_lim0 = (int)((q_base + col < S - 1 ? q_base + col : S - 1) - 4 * h);
    const int q_lim1 = (int)((q_base + 32 + col < S - 1 ? q_base + 32 + col : S - 1) - 4 * h);

    const uint32_t last_row = (uint32_t)(S - 1);
    const uint32_t col_stride = (uint32_t)(a.S_pad * sizeof(T));
    auto stage = [&](int t, unsigned char* b) {
        const uint32_t r0 = (uint32_t)t * kBN;
        auto rows = [&](int r) {   // rows past S repeat row S - 1
            const uint32_t row = r0 + r < last_row ? r0 + r : last_row;
            return row * (uint32_t)KROWB;
        };
        stage_tile<KROWB, KBYTES, 4>(b, Kh, rows);
        if constexpr (kTr<T>)
            stage_tile<KROWB, KBYTES, 4>(b + KBYTES, Vh, rows);
        else
            stage_tile<VROWB, VBYTES, 4>(b + KBYTES, reinterpret_cast<const unsigned char*>(Vh) + (int64_t)t * VROWB,
                                         [&](int r) { return (uint32_t)r * col_stride; });
    };
    stage(0, smem);
    wait_tiles_and_sync();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) stage(t + 1, smem + (buf ^ 1) * BUF);
        const unsigned char* lk = smem + buf * BUF;
        const unsigned char* lv = lk + KBYTES;
        const int kt0 = t * kBN;
        if (kt0 <= q_last_w) {   // this wave sees at least one key of the tile
            // S^T for both 32-key halves of the tile, then one max/rescale per 64 keys
            floatx16 s[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                s[ks][0] = floatx16{};
                s[ks][1] = floatx16{};
#pragma unroll
                for (int cc = 0; cc < D / 16; ++cc) {
                    const F kf = tile_frag<T, KROWB>(lk, 32 * ks + col, 16 * cc + 8 * h);
                    mma_k16(s[ks][0], kf, qf[0][cc]);
                    mma_k16(s[ks][1], kf, qf[1][cc]);
                }
            }
            if (kt0 + kBN - 1 > q_base || kt0 + kBN - 1 >= S) {   // diagonal or tail: key > query / key >= S
                keep_branch();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int l0 = q_lim0 - kt0 - 32 * ks, l1 = q_lim1 - kt0 - 32 * ks;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        if (c_row0(j) > l0) s[ks][0][j] = -INFINITY;
                        if (c_row0(j) > l1) s[ks][1][j] = -INFINITY;
                    }
                }
            }
            float neg[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const float mx = max_halves(__builtin_fmaxf(max16(s[0][cb]), max16(s[1][cb]))) * c;
                // Each query moves its own reference only when its own max grew by more
                // than 2^8 (others scale by exactly 1), so a query's result never depends
                // on the other queries of the wave.
                const bool need = mx > m_i[cb] + 8.f;
                if (wave_any(need)) {
                    keep_branch();
                    const float m_new = need ? mx : m_i[cb];
                    const float alpha = need ? fast_exp2(m_i[cb] - m_new) : 1.f;
                    m_i[cb] = m_new;
                    l_i[cb] *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) o[cb][db] *= alpha;
                }
                neg[cb] = m_i[cb] == -INFINITY ? 0.f : -m_i[cb];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    float rs = 0.f;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float pv = fast_exp2(fmaf(s[ks][cb][j], c, neg[cb]));
                        s[ks][cb][j] = pv;
                        rs += pv;
                    }
                    l_i[cb] += rs;
                }
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    F p0, p1, r0, r1;
                    split_frag_vec<T>(s[ks][0], c2, p0, r0);
                    split_frag_vec<T>(s[ks][1], c2, p1, r1);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        F vf;
                        if constexpr (kTr<T>) vf = tile_frag_tr<KROWB>(lv, 32 * ks + 16 * c2, 32 * db);
                        else vf = tile_frag<T, VROWB>(lv, 32 * db + col, 32 * ks + 16 * c2 + 8 * h);
                        mma_k16(o[0][db], vf, p0);
                        mma_k16(o[1][db], vf, p1);
                        if (kSplitP<T>) {
                            mma_k16(o[0][db], vf, r0);
                            mma_k16(o[1][db], vf, r1);
                        }
                    }
                }
            }
        }
        wait_tiles_and_sync();
    }

#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int64_t q = q_base + 32 * cb + col;
        const float l = sum_halves(l_i[cb]);
        const float inv = 1.f / l;
        if (q < S) {
            float* orow = O32 + (bh * S + q) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    floatx4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = o[cb][db][4 * m + i] * inv;
                    *reinterpret_cast<floatx4*>(orow + 32 * db + 8 * m + 4 * h) = w;
                    if (Ot) {
                        typename Frag<T>::half wt;
#pragma unroll
                        for (int i = 0; i < 4; ++i) wt[i] = static_cast<T>(w[i]);
                        *reinterpret_cast<typename Frag<T>::half*>(Ot + (bh * S + q) * D + 32 * db + 8 * m + 4 * h) = wt;
                    }
                }
            if (h == 0) LSE[bh * S + q] = (m_i[cb] + log2f(l)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ: per 256-query block, over key tiles: S^T = K Q^T, P^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// Each row of dS sums to zero, so dQ = scale sum_j dS_j K_j is a cancelling
// sum; with dS rounded to 8 bits the remainder would carry 2^-9 |dS| |K| of
// noise.  bf16 therefore feeds dS as hi + lo parts (as P in the forward).
// ---------------------------------------------------------------------------
template <typename T, int D>
constexpr size_t dq_buf_bytes() {   // K and V row tiles (+ the K^T column tile for f32)
    return 2 * kBN * D * sizeof(T) + (kTr<T> ? 0 : D * kBN * sizeof(T));
}

// KT (K^T [D][S_pad]) is read only by the f32 kernel; bf16 reads the K tile across its rows.
template <typename T, int D, typename OutT>
__global__ __launch_bounds__(kThreads, (kBlocksPerCu<T, D>)) void attn_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const T* __restrict__ V, const T* __restrict__ KT,
                                                           const T* __restrict__ dO, const float* __restrict__ NL,
                                                           const float* __restrict__ ND, OutT* __restrict__ dQ,
                                                           AttnK a) {
    typedef typename Frag<T>::type F;
    constexpr int RROWB = D * (int)sizeof(T), CROWB = kBN * (int)sizeof(T);
    constexpr int RBYTES = kBN * RROWB, BUF = (int)dq_buf_bytes<T, D>();
    extern __shared__ __align__(16) unsigned char smem[];

    int64_t bh; int qb;
    block_order(a, true, bh, qb);
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 31, h = lane >> 5;
    const int64_t S = a.S;
    const T* Qh = Q + bh * S * D;
    const T* Kh = K + bh * S * D;
    const T* Vh = V + bh * S * D;
    const T* KTh = kTr<T> ? nullptr : KT + bh * D * a.S_pad;
    const T* dOh = dO + bh * S * D;

    const int64_t q_blk0 = (int64_t)qb * kBlockRows;
    const int64_t q_base = q_blk0 + wave * kWaveRows;
    const int64_t q_last_blk = (q_blk0 + kBlockRows < S ? q_blk0 + kBlockRows : S) - 1;
    const int64_t q_last_w = (q_base + kWaveRows < S ? q_base + kWaveRows : S) - 1;
    const int ntiles = (int)(q_last_blk / kBN) + 1;

    F qf[2][D / 16], df[2][D / 16];
    float nlc[2], nd[2];   // -LSE in log2 units, -D
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int64_t q = q_base + 32 * cb + col;
        const bool ok = q < S;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            qf[cb][c] = load8_or_zero(Qh + q * D + 16 * c + 8 * h, ok);
            df[cb][c] = load8_or_zero(dOh + q * D + 16 * c + 8 * h, ok);
        }
        nlc[cb] = ok ? NL[bh * S + q] * a.scale_log2 : 0.f;
        nd[cb] = ok ? ND[bh * S + q] : 0.f;
    }
    floatx16 acc[2][D / 32];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[cb][db] = floatx16{};
    const int q_lim0 = (int)((q_base + col < S - 1 ? q_base + col : S - 1) - 4 * h);
    const int q_lim1 = (int)((q_base + 32 + col < S - 1 ? q_base + 32 + col : S - 1) - 4 * h);

    const uint32_t last_row = (uint32_t)(S - 1);
    const uint32_t col_stride = (uint32_t)(a.S_pad * sizeof(T));
    auto stage = [&](int t, unsigned char* b) {
        const uint32_t r0 = (uint32_t)t * kBN;
        auto rows = [&](int r) {   // rows past S repeat row S - 1
            const uint32_t row = r0 + r < last_row ? r0 + r : last_row;
            return row * (uint32_t)RROWB;
        };
        stage_tile<RROWB, RBYTES, 4>(b, Kh, rows);
        stage_tile<RROWB, RBYTES, 4>(b + RBYTES, Vh, rows);
        if constexpr (!kTr<T>)
            stage_tile<CROWB, D * CROWB, 4>(b + 2 * RBYTES,
                                            reinterpret_cast<const unsigned char*>(KTh) + (int64_t)t * CROWB,
                                            [&](int r) { return (uint32_t)r * col_stride; });
    };
    stage(0, smem);
    wait_tiles_and_sync();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) stage(t + 1, smem + (buf ^ 1) * BUF);
        const unsigned char* lk = smem + buf * BUF;
        const unsigned char* lv = lk + RBYTES;
        const unsigned char* lkt = lk + 2 * RBYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t kbase = (int64_t)t * kBN + 32 * ks;
            if (kbase > q_last_w) continue;
            floatx16 s[2] = {floatx16{}, floatx16{}}, dp[2] = {floatx16{}, floatx16{}};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const F kf = tile_frag<T, RROWB>(lk, 32 * ks + col, 16 * c + 8 * h);
                const F vf = tile_frag<T, RROWB>(lv, 32 * ks + col, 16 * c + 8 * h);
                mma_k16(s[0], kf, qf[0][c]);
                mma_k16(s[1], kf, qf[1][c]);
                mma_k16(dp[0], vf, df[0][c]);
                mma_k16(dp[1], vf, df[1][c]);
            }
            if (kbase + 31 > q_base || kbase + 31 >= S) {   // diagonal or tail
                keep_branch();
                const int l0 = q_lim0 - (int)kbase, l1 = q_lim1 - (int)kbase;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (c_row0(j) > l0) s[0][j] = -INFINITY;
                    if (c_row0(j) > l1) s[1][j] = -INFINITY;
                }
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float pv = fast_exp2(fmaf(s[cb][j], a.scale_log2, nlc[cb]));
                    s[cb][j] = pv * (dp[cb][j] + nd[cb]);
                }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                F g0, g1, r0, r1;
                split_frag<T>(s[0], c2, g0, r0);
                split_frag<T>(s[1], c2, g1, r1);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    F kf;
                    if constexpr (kTr<T>) kf = tile_frag_tr<RROWB>(lk, 32 * ks + 16 * c2, 32 * db);
                    else kf = tile_frag<T, CROWB>(lkt, 32 * db + col, 32 * ks + 16 * c2 + 8 * h);
                    mma_k16(acc[0][db], kf, g0);
                    mma_k16(acc[1][db], kf, g1);
                    if (kSplitP<T>) {
                        mma_k16(acc[0][db], kf, r0);
                        mma_k16(acc[1][db], kf, r1);
                    }
                }
            }
        }
        wait_tiles_and_sync();
    }

#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int64_t q = q_base + 32 * cb + col;
        if (q >= S) continue;
        OutT* row = dQ + (bh * S + q) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    row[32 * db + 8 * m + 4 * h + i] = static_cast<OutT>(acc[cb][db][4 * m + i] * a.scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: per block of 32*NW keys (each wave owns 32 key columns), over the
// queries from the diagonal on, in steps of 32 queries:
// S = Q K^T - LSE/scale, P = exp(scale S), dP' = dO V^T - D, dS = P dP',
// dV^T += dO^T P, dK^T += Q^T dS  (P and dS as bf16 hi + lo parts).
// The -LSE/scale and -D terms enter as the initial accumulators of the two
// products, so they cost no vector instruction.
//
// Software pipeline: while a wave turns step u's scores into P and dS and
// accumulates dV and dK (vector work plus 16 matrix products), it already
// computes step u+1's two score products (8 independent matrix products), so
// the matrix cores and the vector units have independent work side by side.
// LDS: query tiles of TQ rows.  Row tiles (Q, dO, -LSE/scale, -D) are needed
// one step ahead and live in three buffers; for f32, column tiles (Q^T, dO^T)
// in two (bf16 reads the Q and dO row tiles across their rows instead).
// Tile t + 2's rows and tile t + 1's columns are loaded while tile t is used;
// one barrier per tile.
// ---------------------------------------------------------------------------
template <typename T, int D, int TQ>
struct DkdvLds {
    static constexpr int RROWB = D * (int)sizeof(T);   // bytes per row of a row tile
    static constexpr int CROWB = TQ * (int)sizeof(T);  // bytes per row of a column tile
    static constexpr int RT = TQ * RROWB;              // one row tile
    static constexpr int CT = D * CROWB;               // one column tile
    static constexpr int RBUF = 2 * RT + 2 * 256;      // Q, dO, -LSE/scale, -D
    static constexpr int CBUF = kTr<T> ? 0 : 2 * CT;  // Q^T, dO^T (f32 only)
    static constexpr int BYTES = 3 * RBUF + 2 * CBUF;
};

template <typename T, int D, typename OutT, int NW, int TQ>
__global__ __launch_bounds__(64 * NW, 1) void attn_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                               const T* __restrict__ V, const T* __restrict__ QT,
                                                               const T* __restrict__ dO, const T* __restrict__ dOT,
                                                               const float* __restrict__ NL,
                                                               const float* __restrict__ ND, OutT* __restrict__ dK,
                                                               OutT* __restrict__ dV, AttnK a) {
    typedef typename Frag<T>::type F;
    typedef DkdvLds<T, D, TQ> L;
    constexpr int NSTEP = TQ / 32;
    constexpr int RROWB = L::RROWB, CROWB = L::CROWB;
    extern __shared__ __align__(16) unsigned char smem[];

    int64_t bh; int kb;
    block_order(a, false, bh, kb);
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 31, h = lane >> 5;
    const int64_t S = a.S;
    const T* Qh = Q + bh * S * D;
    const T* Kh = K + bh * S * D;
    const T* Vh = V + bh * S * D;
    const T* QTh = kTr<T> ? nullptr : QT + bh * D * a.S_pad;
    const T* dOh = dO + bh * S * D;
    const T* dOTh = kTr<T> ? nullptr : dOT + bh * D * a.S_pad;
    const float* NLh = NL + bh * S;
    const float* NDh = ND + bh * S;

    const int64_t k_blk0 = (int64_t)kb * (32 * NW);
    const int64_t k_base = k_blk0 + 32 * wave;
    const int t0 = (int)(k_blk0 / TQ);
    const int ntiles = (int)((S + TQ - 1) / TQ);
    const int u_first = (int)(k_base / 32);       // the diagonal step (queries k_base .. k_base + 31)

    F kf[D / 16], vf[D / 16];
    {
        const int64_t key = k_base + col;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            kf[c] = load8_or_zero(Kh + key * D + 16 * c + 8 * h, key < S);
            vf[c] = load8_or_zero(Vh + key * D + 16 * c + 8 * h, key < S);
        }
    }
    floatx16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dk[db] = floatx16{};
        dv[db] = floatx16{};
    }

    const uint32_t last_row = (uint32_t)(S - 1);
    const uint32_t col_stride = (uint32_t)(a.S_pad * sizeof(T));
    auto rbuf = [&](int t) { return smem + (t % 3) * L::RBUF; };
    auto cbuf = [&](int t) { return smem + 3 * L::RBUF + (t & 1) * L::CBUF; };
    auto stage_rows = [&](int t) {
        unsigned char* b = rbuf(t);
        const uint32_t r0 = (uint32_t)t * TQ;
        auto rows = [&](int r) {   // rows past S repeat row S - 1
            const uint32_t row = r0 + r < last_row ? r0 + r : last_row;
            return row * (uint32_t)RROWB;
        };
        stage_tile<RROWB, L::RT, NW>(b, Qh, rows);
        stage_tile<RROWB, L::RT, NW>(b + L::RT, dOh, rows);
        // 64 values of -LSE/scale (wave 0) and -D (wave 1), 4 bytes per lane
        if (wave < 2) {
            const uint32_t row = r0 + lane < last_row ? r0 + lane : last_row;
            __builtin_amdgcn_global_load_lds((wave == 0 ? NLh : NDh) + row, (lds_void*)(b + 2 * L::RT + wave * 256),
                                             4, 0, 0);
        }
    };
    auto stage_cols = [&](int t) {
        if constexpr (kTr<T>) return;
        unsigned char* b = cbuf(t);
        auto cols = [&](int r) { return (uint32_t)r * col_stride; };
        stage_tile<CROWB, L::CT, NW>(b, reinterpret_cast<const unsigned char*>(QTh) + (int64_t)t * CROWB, cols);
        stage_tile<CROWB, L::CT, NW>(b + L::CT, reinterpret_cast<const unsigned char*>(dOTh) + (int64_t)t * CROWB,
                                     cols);
    };

    // Score products of one step: S' = Q K^T - LSE/scale and dP' = dO V^T - D
    // for the 32 queries at row r0 of row tile rb.
    auto scores = [&](const unsigned char* rb, int r0, floatx16& sp, floatx16& dp) {
        const float* nl = reinterpret_cast<const float*>(rb + 2 * L::RT);
        const float* nd = nl + 64;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const floatx4 l4 = *reinterpret_cast<const floatx4*>(nl + r0 + 8 * m + 4 * h);
            const floatx4 d4 = *reinterpret_cast<const floatx4*>(nd + r0 + 8 * m + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sp[4 * m + i] = l4[i];
                dp[4 * m + i] = d4[i];
            }
        }
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            const F qa = tile_frag<T, RROWB>(rb, r0 + col, 16 * cc + 8 * h);
            const F da = tile_frag<T, RROWB>(rb + L::RT, r0 + col, 16 * cc + 8 * h);
            mma_k16(sp, qa, kf[cc]);
            mma_k16(dp, da, vf[cc]);
        }
    };
    // P, dS and the dV / dK products of one step: queries c0 .. c0+31 of tile t,
    // read across the rows of its row tile rb (bf16) or from its column tile cb (f32).
    auto grads = [&](const unsigned char* rb, const unsigned char* cb, int c0, floatx16& sp, floatx16& dp) {
        const float c = a.scale_log2;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = fast_exp2(sp[8 * c2 + e] * c);
                sp[8 * c2 + e] = pv;
                dp[8 * c2 + e] = pv * dp[8 * c2 + e];
            }
            F ph, pl, gh, gl;
            split_frag<T>(sp, c2, ph, pl);
            split_frag<T>(dp, c2, gh, gl);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                F dof, qtf;
                if constexpr (kTr<T>) {
                    dof = tile_frag_tr<RROWB>(rb + L::RT, c0 + 16 * c2, 32 * db);
                    qtf = tile_frag_tr<RROWB>(rb, c0 + 16 * c2, 32 * db);
                } else {
                    dof = tile_frag<T, CROWB>(cb + L::CT, 32 * db + col, c0 + 16 * c2 + 8 * h);
                    qtf = tile_frag<T, CROWB>(cb, 32 * db + col, c0 + 16 * c2 + 8 * h);
                }
                mma_k16(dv[db], dof, ph);
                mma_k16(dk[db], qtf, gh);
                if (kSplitP<T>) {
                    mma_k16(dv[db], dof, pl);
                    mma_k16(dk[db], qtf, gl);
                }
            }
        }
    };
    // Step v's mask: key after query (steps up to the diagonal) or query >= S.
    auto needs_mask = [&](int v) { return v <= u_first || 32 * (int64_t)v + 31 >= S; };
    auto mask = [&](floatx16& sp, int v) {
        const int kl = (int)(k_base - 32 * (int64_t)v) + col - 4 * h;   // rows below kl precede the key
        const int64_t sl64 = S - 32 * (int64_t)v - 4 * h;                 // rows from sl on are past S
        const int sl = (int)(sl64 < 64 ? sl64 : 64);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (c_row0(j) < kl || c_row0(j) >= sl) sp[j] = -INFINITY;
    };

    // prologue: rows of the first two tiles, columns of the first
    if (t0 < ntiles) {
        stage_rows(t0);
        stage_cols(t0);
    }
    if (t0 + 1 < ntiles) stage_rows(t0 + 1);
    wait_tiles_and_sync();

    // Every wave runs every step of the block from the first tile on: steps
    // before its diagonal are fully masked (they add zeros), which keeps one
    // uniform instruction stream per step.  Step u's products live in sp[u & 1].
    floatx16 sp[2], dp[2];
    const int u0 = t0 * NSTEP;
    if (t0 < ntiles) {
        scores(rbuf(t0), 0, sp[0], dp[0]);
        mask(sp[0], u0);
    }
    // one step: the next step's score products, this step's gradients, then
    // (rarely) the next step's mask
    auto step = [&](int t, int qs, floatx16& sp_c, floatx16& dp_c, floatx16& sp_n, floatx16& dp_n) {
        const int u = t * NSTEP + qs;
        const bool last_in_tile = qs + 1 == NSTEP;
        scores(last_in_tile ? rbuf(t + 1) : rbuf(t), last_in_tile ? 0 : 32 * (qs + 1), sp_n, dp_n);
        grads(rbuf(t), cbuf(t), 32 * qs, sp_c, dp_c);
        if (needs_mask(u + 1)) {
            keep_branch();
            mask(sp_n, u + 1);
        }
    };
    if constexpr (NSTEP == 2) {
        for (int t = t0; t < ntiles; ++t) {
            if (t + 2 < ntiles) stage_rows(t + 2);
            if (t + 1 < ntiles) stage_cols(t + 1);
            step(t, 0, sp[0], dp[0], sp[1], dp[1]);
            step(t, 1, sp[1], dp[1], sp[0], dp[0]);
            wait_tiles_and_sync();
        }
    } else {
        for (int t = t0; t < ntiles; t += 2) {
            if (t + 2 < ntiles) stage_rows(t + 2);
            if (t + 1 < ntiles) stage_cols(t + 1);
            step(t, 0, sp[0], dp[0], sp[1], dp[1]);
            wait_tiles_and_sync();
            if (t + 1 < ntiles) {
                if (t + 3 < ntiles) stage_rows(t + 3);
                if (t + 2 < ntiles) stage_cols(t + 2);
                step(t + 1, 0, sp[1], dp[1], sp[0], dp[0]);
                wait_tiles_and_sync();
            }
        }
    }

    const int64_t key = k_base + col;
    if (key < S) {
        OutT* rk = dK + (bh * S + key) * D;
        OutT* rv = dV + (bh * S + key) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    rk[32 * db + 8 * m + 4 * h + i] = static_cast<OutT>(dk[db][4 * m + i] * a.scale);
                    rv[32 * db + 8 * m + 4 * h + i] = static_cast<OutT>(dv[db][4 * m + i]);
                }
    }
}

template <typename T, int D>
size_t fwd_lds() { return 2 * 2 * kBN * D * sizeof(T); }
template <typename T, int D>
size_t dq_lds() { return 2 * dq_buf_bytes<T, D>(); }

AttnK make_k(const AttnArgs& a) {
    AttnK k{};
    k.BH = a.BH; k.S = a.S; k.S_pad = a.S_pad; k.scale = a.scale; k.scale_log2 = a.scale * kLog2e;
    k.nblk = (int)((a.S + kBlockRows - 1) / kBlockRows);
    return k;
}

template <typename T, int D>
hipError_t fwd_t(const AttnArgs& a, const void* Q, const void* K, const void* Vop, float* O32, void* Ot, float* lse,
                 hipStream_t st) {
    const AttnK k = make_k(a);
    const size_t sh = fwd_lds<T, D>();
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)attn_fwd_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    (void)attr;
    attn_fwd_kernel<T, D><<<dim3((unsigned)(k.nblk * a.BH)), kThreads, sh, st>>>(
        (const T*)Q, (const T*)K, (const T*)Vop, O32, (T*)Ot, lse, k);
    return hipGetLastError();
}

template <typename T, int D, typename OutT>
hipError_t dkdv_t(const AttnArgs& a, const void* Q, const void* K, const void* V, const void* QT, const void* dO,
                  const void* dOT, const float* nl, const float* nd, void* dK, void* dV, hipStream_t st) {
    // 64-query tiles, except f32 at 256-byte rows, whose three row and two
    // column buffers would not fit: 32 there (bf16 has no column buffers)
    constexpr int TQ = (kTr<T> || D * sizeof(T) <= 128) ? 64 : 32;
    typedef DkdvLds<T, D, TQ> L;
    static_assert(L::BYTES <= 160 * 1024, "dK/dV LDS budget");
    // d = 128 keeps twice the key and accumulator registers: one wave per SIMD
    constexpr int NW = D == 128 ? 4 : kDkdvNW;
    AttnK k = make_k(a);
    constexpr int BK = 32 * NW;
    k.nblk = (int)((a.S + BK - 1) / BK);
    auto kern = attn_dkdv_kernel<T, D, OutT, NW, TQ>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    (void)attr;
    kern<<<dim3((unsigned)(k.nblk * a.BH)), 64 * NW, L::BYTES, st>>>((const T*)Q, (const T*)K, (const T*)V,
                                                                         (const T*)QT, (const T*)dO, (const T*)dOT,
                                                                         nl, nd, (OutT*)dK, (OutT*)dV, k);
    return hipGetLastError();
}

template <typename T, int D, typename OutT>
hipError_t dq_t(const AttnArgs& a, const void* Q, const void* K, const void* V, const void* KT, const void* dO,
                const float* nl, const float* nd, void* dQ, hipStream_t st) {
    const AttnK k = make_k(a);
    const size_t sh = dq_lds<T, D>();
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_dq_kernel<T, D, OutT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    (void)attr;
    attn_dq_kernel<T, D, OutT><<<dim3((unsigned)(k.nblk * a.BH)), kThreads, sh, st>>>(
        (const T*)Q, (const T*)K, (const T*)V, (const T*)KT, (const T*)dO, nl, nd, (OutT*)dQ, k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, int dtype, const void* Q, const void* K, const void* Vop, float* O32,
                           void* Ot, float* lse, hipStream_t st) {
    if (dtype == LH_BF16)
        return a.d == 64 ? fwd_t<bf16, 64>(a, Q, K, Vop, O32, Ot, lse, st)
                         : fwd_t<bf16, 128>(a, Q, K, Vop, O32, Ot, lse, st);
    return fwd_t<float, 64>(a, Q, K, Vop, O32, Ot, lse, st);   // f32 is built for d = 64 only
}

hipError_t launch_attn_dkdv(const AttnArgs& a, int dtype, bool out_f32, const void* Q, const void* K, const void* V,
                            const void* QT, const void* dO, const void* dOT, const float* nl, const float* nd,
                            void* dK, void* dV, hipStream_t st) {
#define LH_DKDV(T, D, O) dkdv_t<T, D, O>(a, Q, K, V, QT, dO, dOT, nl, nd, dK, dV, st)
    if (dtype == LH_BF16) {
        if (a.d == 64) return out_f32 ? LH_DKDV(bf16, 64, float) : LH_DKDV(bf16, 64, bf16);
        return out_f32 ? LH_DKDV(bf16, 128, float) : LH_DKDV(bf16, 128, bf16);
    }
    return LH_DKDV(float, 64, float);   // f32 is built for d = 64 only
#undef LH_DKDV
}

hipError_t launch_attn_dq(const AttnArgs& a, int dtype, bool out_f32, const void* Q, const void* K, const void* V,
                          const void* KT, const void* dO, const float* nl, const float* nd, void* dQ,
                          hipStream_t st) {
#define LH_DQ(T, D, O) dq_t<T, D, O>(a, Q, K, V, KT, dO, nl, nd, dQ, st)
    if (dtype == LH_BF16) {
        if (a.d == 64) return out_f32 ? LH_DQ(bf16, 64, float) : LH_DQ(bf16, 64, bf16);
        return out_f32 ? LH_DQ(bf16, 128, float) : LH_DQ(bf16, 128, bf16);
    }
    return LH_DQ(float, 64, float);
#undef LH_DQ
}
