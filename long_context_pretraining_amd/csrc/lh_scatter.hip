// Data movement around the sub-sequence attention of Lighthouse Attention on
// gfx950: gather of the selected triples (page "skillsmp.com ...
// lighthouse-attention", Stage 3; gist.science Methodology 2C), scatter-back
// over R(l, i) (skill card, Stage 4), and the backward of both (skill card,
// gradient flow).  All HBM-bound: 16-byte coalesced rows, LDS-staged
// transposes, and pull formulations (each output row reads its <= L sources)
// so no atomics and bit-reproducible results.
#include "lh_device.h"
#include "lh_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;   // rows (slots or tokens) per block
constexpr int kGatherTasks = 4;   // 16-byte gather tasks per thread: 64 rows of up to 256 bytes

struct MapGeo {
    int64_t BH, N, d, S, S_pad, Mu, M_total;
    int p, L;
    int64_t off[LH_MAX_LEVELS + 1];
    int64_t pw[LH_MAX_LEVELS];
    // n / p^l for 32-bit n as (umulhi(n, dmul) + n) >> dsh (round-up reciprocal,
    // exact for n < 2^31), and 1 / p^l in f32
    uint32_t dmul[LH_MAX_LEVELS], dsh[LH_MAX_LEVELS];
    float inv[LH_MAX_LEVELS];
};

MapGeo make_geo(const LhGeom& g) {
    MapGeo m{};
    m.BH = g.BH; m.N = g.N; m.d = g.d; m.S = g.S; m.S_pad = g.S_pad; m.Mu = g.Mu; m.M_total = g.M_total;
    m.p = g.p; m.L = g.L;
    for (int l = 0; l <= g.L; ++l) m.off[l] = g.off[l];
    for (int l = 0; l < g.L; ++l) {
        const uint64_t dv = (uint64_t)g.pw[l];
        uint32_t sh = 0;
        while ((1ull << sh) < dv) ++sh;
        m.pw[l] = g.pw[l];
        m.dsh[l] = sh;
        m.dmul[l] = (uint32_t)((((uint64_t)1 << 32) * ((1ull << sh) - dv)) / dv + 1);
        m.inv[l] = (float)(1.0 / (double)dv);
    }
    return m;
}

__device__ __forceinline__ uint32_t div_pw(const MapGeo& G, int l, uint32_t n) {
    return (__umulhi(n, G.dmul[l]) + n) >> G.dsh[l];
}

__device__ __forceinline__ int level_of(const MapGeo& G, int64_t flat) {
    int l = 0;
    while (flat >= G.off[l + 1]) ++l;
    return l;
}

// Write the [kRows x d] tile held in LDS (row stride d + pad) as columns
// s0 .. s0+63 of the transposed array xT [d][S_pad].  Within every aligned
// group of 16 columns the order is 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the
// column swapped): that is the k order in which the attention kernels feed a
// C tile back into the matrix cores, so each lane reads its 8 keys as one
// contiguous 16-byte run.
__device__ __forceinline__ int key_perm16(int p) { return (p & ~12) | ((p >> 1) & 4) | ((p << 1) & 8); }

template <typename T>
__device__ __forceinline__ void store_transposed(const T* tile, int ld, int64_t d, T* xT, int64_t S_pad,
                                                 int64_t s0) {
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const int per_row = kRows / VEC;
    for (int task = threadIdx.x; task < d * per_row; task += kThreads) {
        const int dim = task / per_row, cv = task - dim * per_row;
        VT out;
#pragma unroll
        for (int i = 0; i < VEC; ++i) out[i] = tile[key_perm16(cv * VEC + i) * ld + dim];
        *reinterpret_cast<VT*>(xT + dim * S_pad + s0 + cv * VEC) = out;
    }
}

// ---------------------------------------------------------------------------
// Gather: rows of the selected entries in slot order, row-major [S][d] and,
// when c0..c2 are given (the f32 attention kernels take them), transposed
// [d][S_pad] (columns past S are zero).  Level 0 rows come from the input,
// coarser ones from the pyramid (pyramid row = flat id - N).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, const T* __restrict__ pyr,
                                                          const int32_t* __restrict__ gidx, T* r0, T* r1, T* r2,
                                                          T* c0, T* c1, T* c2, MapGeo G) {
    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const int z = blockIdx.z;
    const T* src0 = z == 0 ? q : (z == 1 ? k : v);
    const T* srcp = pyr + (int64_t)z * G.BH * G.Mu * G.d;
    T* rows = z == 0 ? r0 : (z == 1 ? r1 : r2);
    T* cols = z == 0 ? c0 : (z == 1 ? c1 : c2);
    const bool transposed = cols != nullptr;   // uniform over the grid
    const int64_t bh = blockIdx.y, s0 = (int64_t)blockIdx.x * kRows;
    const int ld = (int)G.d + VEC;
    const int nvec = (int)(G.d / VEC);
    const int ntask = kRows * nvec;
    // A thread's tasks (at most kGatherTasks for the built row widths) go
    // through in three passes -- every slot's map entry, every row, every
    // store -- so no load is issued after a store (a wait for it would also
    // wait for the store).
    for (int first = threadIdx.x; first < ntask; first += kGatherTasks * kThreads) {
        int64_t flat[kGatherTasks];
#pragma unroll
        for (int u = 0; u < kGatherTasks; ++u) {
            const int task = first + u * kThreads;
            const int64_t s = s0 + task / nvec;
            flat[u] = task < ntask && s < G.S ? gidx[bh * G.S + s] : -1;
        }
        VT val[kGatherTasks];
#pragma unroll
        for (int u = 0; u < kGatherTasks; ++u) {
            const int task = first + u * kThreads;
            const int sl = task / nvec, vv = task - sl * nvec;
            val[u] = VT{};
            if (flat[u] >= 0 && flat[u] < G.M_total) {   // a map entry outside the pyramid gathers zeros
                const T* src = flat[u] < G.N ? src0 + (bh * G.N + flat[u]) * G.d
                                             : srcp + (bh * G.Mu + flat[u] - G.N) * G.d;
                val[u] = *reinterpret_cast<const VT*>(src + vv * VEC);
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherTasks; ++u) {
            const int task = first + u * kThreads;
            const int sl = task / nvec, vv = task - sl * nvec;
            const int64_t s = s0 + sl;
            if (task < ntask && s < G.S) *reinterpret_cast<VT*>(rows + (bh * G.S + s) * G.d + vv * VEC) = val[u];
            if (transposed && task < ntask)
#pragma unroll
                for (int i = 0; i < VEC; ++i) tile[sl * ld + vv * VEC + i] = val[u][i];
        }
    }
    if (!transposed) return;
    __syncthreads();
    store_transposed(tile, ld, G.d, cols + bh * G.d * G.S_pad, G.S_pad, s0);
}

// ---------------------------------------------------------------------------
// Pull kernels (scatter forward, gather + pool backward) over a block of R
// tokens (a power of two chosen at launch so the staged rows fit in LDS).
// Output token t reads the row of entry i_l(t) = floor((t + SHIFT) / p^l) -
// SHIFT of every level l.  Coarse rows are shared by p^l consecutive tokens,
// so the block stages them once: it loads the slot of every entry its tokens
// read into LDS, then the f32 rows of the entries of levels >= 1 (zeros where
// the entry is not selected).  Each token then reads its own level-0 row from
// global memory (only if selected) and the coarser ones from LDS, and sums the
// levels in ascending order.  L and the row width D are template parameters.
// ---------------------------------------------------------------------------
struct PullLds {
    int R;          // tokens per block
    int slot_cap;   // slots of all levels over R tokens
    int row_cap;    // staged rows (levels >= 1)
};

inline PullLds pull_lds(int p, int L, int64_t d) {
    PullLds P{};
    for (int R = 256;; R /= 2) {
        int slots = 0, rows = 0, q = 1;
        for (int l = 0; l < L; ++l, q *= p) {
            const int n = R / q + 2;
            slots += n;
            if (l > 0) rows += n;
        }
        P.R = R;
        P.slot_cap = slots;
        P.row_cap = rows;
        if ((size_t)rows * d * 4 + (size_t)slots * 4 <= 40 * 1024 || R <= 16) return P;
    }
}

template <int L, int D, int SHIFT>
__device__ __forceinline__ void stage_block_rows(const MapGeo& G, const int32_t* gp, const float* rows_g, int64_t t0,
                                                 int64_t t1, int32_t* slot, float* rows, int64_t* lo, int* base) {
    int n[L];
    int acc = 0;
#pragma unroll
    for (int l = 0; l < L; ++l) {
        lo[l] = (int64_t)div_pw(G, l, (uint32_t)(t0 + SHIFT)) - SHIFT;
        const int64_t hi = (int64_t)div_pw(G, l, (uint32_t)(t1 + SHIFT)) - SHIFT;
        base[l] = acc;
        n[l] = (int)(hi - lo[l] + 1);
        acc += n[l];
    }
    // slots of every level (-1 outside [0, M_l))
#pragma unroll
    for (int l = 0; l < L; ++l) {
        const int64_t M = G.off[l + 1] - G.off[l];
        for (int j = threadIdx.x; j < n[l]; j += kThreads) {
            const int64_t i = lo[l] + j;
            slot[base[l] + j] = (i >= 0 && i < M) ? gp[G.off[l] + i] : -1;
        }
    }
    __syncthreads();
    // rows of levels >= 1: staged entry e is slot n_0 + e
    constexpr int CH = D / 4;   // 16-byte chunks per row
    const int ne = acc - n[0];
    constexpr int BATCH = 8;   // loads in flight per thread
    for (int t0_ = threadIdx.x; t0_ < ne * CH; t0_ += BATCH * kThreads) {
        floatx4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int task = t0_ + u * kThreads;
            const int e = task / CH, c = task - e * CH;
            const int32_t g = task < ne * CH ? slot[n[0] + e] : -1;
            v[u] = floatx4{};
            if (g >= 0 && g < G.S) v[u] = *reinterpret_cast<const floatx4*>(rows_g + (int64_t)g * D + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int task = t0_ + u * kThreads;
            if (task < ne * CH) *reinterpret_cast<floatx4*>(rows + task * 4) = v[u];
        }
    }
    __syncthreads();
}

// Token loop of the pull kernels.  A task is the 8-element chunk vv of token
// t (consecutive lanes on consecutive chunks, so a wave stores 1 KB runs);
// emit(t, vv, x) gets x[l] = elements vv*8 .. vv*8+7 of token t's level-l row
// (zeros where the entry is not selected).  A thread takes its tasks in pairs
// and requests both level-0 rows (global memory, only where selected) before
// it stores either result: stores and loads share one in-order completion
// counter, so a wait for a load issued after a store also waits for that
// store.  (Larger groups cost more registers than the waits they save:
// these kernels live on occupancy.)
template <int L, int D, int SHIFT, class Emit>
__device__ __forceinline__ void pull_tokens(const MapGeo& G, const float* rows_g, const int32_t* slot,
                                            const float* rows, const int64_t* lo, const int* base, int64_t t0,
                                            int64_t t1, Emit&& emit) {
    constexpr int NVEC = D / 8, C = 2;
    const int ntask = (int)(t1 - t0 + 1) * NVEC;
    const int s0 = (int)(t0 - lo[0]);
    for (int first = threadIdx.x; first < ntask; first += C * kThreads) {
        floatx8 x0[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int task = first + c * kThreads;
            x0[c] = floatx8{};
            if (task < ntask) {
                const int tl = task / NVEC, vv = task - tl * NVEC;
                const int32_t g0 = slot[s0 + tl];   // level 0: i_0(t) = t
                if (g0 >= 0 && g0 < G.S)
                    x0[c] = *reinterpret_cast<const floatx8*>(rows_g + (int64_t)g0 * D + vv * 8);
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int task = first + c * kThreads;
            if (task < ntask) {
                const int tl = task / NVEC, vv = task - tl * NVEC;
                const int64_t t = t0 + tl;
                floatx8 x[L];
                x[0] = x0[c];
#pragma unroll
                for (int l = 1; l < L; ++l) {
                    const int e =
                        base[l] - base[1] + (int)((int64_t)div_pw(G, l, (uint32_t)(t + SHIFT)) - SHIFT - lo[l]);
                    x[l] = *reinterpret_cast<const floatx8*>(rows + e * D + vv * 8);
                }
                emit(t, vv, x);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Scatter forward (pull): o[t] = sum_l Og[gpos(l, floor((t+1)/p^l) - 1)],
// levels ascending, in f32 from the f32 sub-sequence output, one rounding to
// T; 0 where no selected entry covers t.
// ---------------------------------------------------------------------------
template <typename T, int L, int D>
__global__ __launch_bounds__(kThreads) void scatter_fwd_kernel(const float* __restrict__ og,
                                                               const int32_t* __restrict__ gpos,
                                                               T* __restrict__ o, MapGeo G, PullLds P) {
    typedef typename Frag<T>::type OV;
    extern __shared__ __align__(16) unsigned char smem[];
    float* rows = reinterpret_cast<float*>(smem);
    int32_t* slot = reinterpret_cast<int32_t*>(smem + (size_t)P.row_cap * D * 4);
    const int64_t bh = blockIdx.y, t0 = (int64_t)blockIdx.x * P.R;
    const int64_t t1 = (t0 + P.R < G.N ? t0 + P.R : G.N) - 1;
    const float* ogh = og + bh * G.S * D;
    int64_t lo[L];
    int base[L];
    stage_block_rows<L, D, 1>(G, gpos + bh * G.M_total, ogh, t0, t1, slot, rows, lo, base);
    pull_tokens<L, D, 1>(G, ogh, slot, rows, lo, base, t0, t1, [&](int64_t t, int vv, const floatx8* x) {
        floatx8 acc = x[0];
#pragma unroll
        for (int l = 1; l < L; ++l) acc += x[l];
        OV out;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = static_cast<T>(acc[e]);
        // the layer output is not read again by this layer: a non-temporal store
        // keeps it from displacing cached inputs (measured 0.03-0.04 ms per step)
        __builtin_nontemporal_store(out, reinterpret_cast<OV*>(o + (bh * G.N + t) * D + vv * 8));
    });
}

// ---------------------------------------------------------------------------
// Scatter backward: dOg[g] = sum of dout over R(l, i) (clipped at N-1) for
// the entry in slot g, summed in token order in f32 and stored in T; also its
// transpose and D[g] = dOg[g] . Og[g] (f32), which the attention backward
// needs.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void scatter_bwd_kernel(const T* __restrict__ dout,
                                                               const float* __restrict__ og,
                                                               const int32_t* __restrict__ gidx,
                                                               const float* __restrict__ lse, float inv_scale,
                                                               T* dog, T* dogT, float* __restrict__ nd,
                                                               float* __restrict__ nl, MapGeo G) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const int ld = (int)G.d + VEC;
    const int nvec = (int)(G.d / VEC);
    T* tile = reinterpret_cast<T*>(smem);
    float* dpart = reinterpret_cast<float*>(smem + sizeof(T) * kRows * ld);
    __shared__ int64_t s_lo[kRows];
    __shared__ int s_len[kRows], s_order[kRows];
    const int64_t bh = blockIdx.y, s0 = (int64_t)blockIdx.x * kRows;
    // Token range of each slot, then the slots ranked by range length (longest
    // first, ties by slot), so the lanes of a wave sum ranges of similar length.
    if (threadIdx.x < kRows) {
        const int64_t s = s0 + threadIdx.x;
        const int64_t flat = s < G.S ? gidx[bh * G.S + s] : -1;
        int64_t lo = 0;
        int len = 0;
        if (flat >= 0 && flat < G.M_total) {
            const int l = level_of(G, flat);
            lo = (flat - G.off[l] + 1) * G.pw[l] - 1;
            const int64_t hi = (lo + G.pw[l] - 1) < (G.N - 1) ? (lo + G.pw[l] - 1) : (G.N - 1);
            len = (int)(hi - lo + 1);
        }
        s_lo[threadIdx.x] = lo;
        s_len[threadIdx.x] = len;
    }
    __syncthreads();
    if (threadIdx.x < kRows) {
        const int me = threadIdx.x, len = s_len[me];
        int rank = 0;
        for (int j = 0; j < kRows; ++j) rank += (s_len[j] > len) || (s_len[j] == len && j < me);
        s_order[rank] = me;
    }
    __syncthreads();
    for (int task = threadIdx.x; task < kRows * nvec; task += kThreads) {
        const int rk = task / nvec, vv = task - rk * nvec;
        const int sl = s_order[rk];
        const int64_t s = s0 + sl;
        VT r = {};
        float dp = 0.f;
        const int len = s_len[sl];
        if (len > 0) {
            const T* src = dout + (bh * G.N + s_lo[sl]) * G.d + vv * VEC;
            float acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
            int t = 0;
            // eight independent loads per step (a 64-row range is 8 round trips, not 16),
            // summed in token order
            for (; t + 8 <= len; t += 8) {
                VT x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const VT*>(src + (int64_t)(t + u) * G.d);
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] += to_f(x[u][e]);
            }
            for (; t < len; ++t) {
                const VT x = *reinterpret_cast<const VT*>(src + (int64_t)t * G.d);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] += to_f(x[e]);
            }
            const float* ov = og + (bh * G.S + s) * G.d + vv * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                r[e] = static_cast<T>(acc[e]);
                dp += to_f(r[e]) * ov[e];
            }
        }
        if (s < G.S) *reinterpret_cast<VT*>(dog + (bh * G.S + s) * G.d + vv * VEC) = r;
        if (dogT)
#pragma unroll
            for (int e = 0; e < VEC; ++e) tile[sl * ld + vv * VEC + e] = r[e];
        dpart[sl * nvec + vv] = dp;
    }
    __syncthreads();
    for (int sl = threadIdx.x; sl < kRows; sl += kThreads) {
        const int64_t s = s0 + sl;
        if (s < G.S) {
            float acc = 0.f;
            for (int vv = 0; vv < nvec; ++vv) acc += dpart[sl * nvec + vv];
            nd[bh * G.S + s] = -acc;
            nl[bh * G.S + s] = -lse[bh * G.S + s] * inv_scale;
        }
    }
    if (dogT) store_transposed(tile, ld, G.d, dogT + bh * G.d * G.S_pad, G.S_pad, s0);
}

// ---------------------------------------------------------------------------
// Gather + pooling backward (pull): dX[t] = sum_l dXg[gpos(l, floor(t/p^l))] / p^l
// over selected entries, levels ascending, f32, stored in T.
// ---------------------------------------------------------------------------
template <typename T, int L, int D>
__global__ __launch_bounds__(kThreads) void gpool_bwd_kernel(const float* __restrict__ g0,
                                                             const float* __restrict__ g1,
                                                             const float* __restrict__ g2,
                                                             const int32_t* __restrict__ gpos, T* o0, T* o1, T* o2,
                                                             MapGeo G, PullLds P) {
    typedef typename Frag<T>::type OV;
    extern __shared__ __align__(16) unsigned char smem[];
    float* rows = reinterpret_cast<float*>(smem);
    int32_t* slot = reinterpret_cast<int32_t*>(smem + (size_t)P.row_cap * D * 4);
    const int z = blockIdx.z;
    const float* dxg = (z == 0 ? g0 : (z == 1 ? g1 : g2)) + (int64_t)blockIdx.y * G.S * D;
    T* out = z == 0 ? o0 : (z == 1 ? o1 : o2);
    const int64_t bh = blockIdx.y, t0 = (int64_t)blockIdx.x * P.R;
    const int64_t t1 = (t0 + P.R < G.N ? t0 + P.R : G.N) - 1;
    int64_t lo[L];
    int base[L];
    stage_block_rows<L, D, 0>(G, gpos + bh * G.M_total, dxg, t0, t1, slot, rows, lo, base);
    pull_tokens<L, D, 0>(G, dxg, slot, rows, lo, base, t0, t1, [&](int64_t t, int vv, const floatx8* x) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int l = 0; l < L; ++l)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(x[l][e], G.inv[l], acc[e]);
        OV r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = static_cast<T>(acc[e]);
        __builtin_nontemporal_store(r, reinterpret_cast<OV*>(out + (bh * G.N + t) * D + vv * 8));   // final gradient, as above
    });
}

// ---------------------------------------------------------------------------
// Dense-baseline helpers: transpose x [S][d] -> xT [d][S_pad] (zero columns
// past S), and the backward prologue (transposed dO and D = rowsum(dO * O)).
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Scatter backward as a pyramid (the form used when the chunk's coarse levels
// fit the LDS).  With t' = t + 1, the range R(l, i) = [(i+1) p^l - 1,
// (i+2) p^l - 2] is the aligned block i+1 of level l of the shifted sequence
// dout'[t'] = dout[t'-1] (dout'[0] = 0, and tokens past N - 1 are 0, which is
// the clipping), so every range sum is an entry of the plain sum pyramid of
// dout': children summed in index order in f32, level by level.  dout is read
// once.  A block owns one aligned chunk of t' (a multiple of p^(L-1) and of
// p^2); each group of VEC-element lanes owns p^2 consecutive rows of it: it
// issues all p^2 row loads at once and forms levels 0, 1 and 2 in registers.
// Levels 3 .. L-1 are summed from the level-2 rows kept in LDS.  Every entry
// whose slot is selected is stored as dOg (one rounding to T); level-0 slots
// and level-1 slots of the chunk are staged in LDS, loaded before the rows.
// D and -LSE/scale follow in slot order (slot_dot_kernel).
// ---------------------------------------------------------------------------
struct TreeP {
    int chunk;     // t' positions per block
    int s1_off;    // LDS: level-0 slots at 0 (chunk ints), level-1 slots at s1_off (chunk / p ints)
    int rows_off;  // LDS byte offset of the f32 rows of levels 2 .. L-2
};

template <typename T, int D, int P>
__global__ __launch_bounds__(1024) void scatter_bwd_tree_kernel(const T* __restrict__ dout,
                                                                const int32_t* __restrict__ gpos,
                                                                T* __restrict__ dog, MapGeo G, TreeP TP) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int VEC = V16<T>::N, NVEC = D / VEC, U = P * P;
    typedef typename V16<T>::type VT;
    int32_t* s0l = reinterpret_cast<int32_t*>(smem);
    int32_t* s1l = s0l + TP.s1_off;
    float* lrow = reinterpret_cast<float*>(smem + TP.rows_off);
    const int C = TP.chunk, nthr = blockDim.x, tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * C;   // first t' of the chunk
    const T* dh = dout + bh * G.N * D;
    T* dgh = dog + bh * G.S * D;
    const int32_t* gp = gpos + bh * G.M_total;

    // entry (l, k) of the shifted pyramid is range entry i = k - 1
    auto slot_of = [&](int l, int64_t k) {
        const int64_t i = k - 1;
        return i >= 0 && i < G.off[l + 1] - G.off[l] ? gp[G.off[l] + i] : -1;
    };
    auto store = [&](int32_t slot, int vv, const float* acc) {
        VT r;
#pragma unroll
        for (int e = 0; e < VEC; ++e) r[e] = static_cast<T>(acc[e]);
        *reinterpret_cast<VT*>(dgh + (int64_t)slot * D + vv * VEC) = r;
    };

    // Slots of the chunk's level-0 and level-1 entries, requested first, then
    // the rows.  All these loads are unconditional (clamped indices, results
    // masked afterwards), so the wait for the slots leaves the rows in flight.
    const int n1 = C / P;
    const int64_t M0 = G.off[1] - G.off[0], M1 = G.L > 1 ? G.off[2] - G.off[1] : 0;
    int32_t sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = tid + j * nthr;
        const bool lv0 = i < C;
        const int64_t e = lv0 ? c0 + i - 1 : c0 / P + (i - C) - 1;   // range entry i = k - 1
        const int64_t m = lv0 ? M0 : M1;
        const bool ok = i < C + n1 && e >= 0 && e < m;
        const int64_t idx = (lv0 ? G.off[0] : G.off[1]) + (ok ? e : 0);
        const int32_t v = gp[idx];
        sv[j] = ok ? v : -1;
    }
    // lane group u (the launch has at least C / U groups) owns rows u U .. u U + U - 1
    const int units = C / U;
    const int vv = tid % NVEC, u = tid / NVEC;
    VT x[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int64_t tp = c0 + (int64_t)u * U + j;
        const bool ok = u < units && tp >= 1 && tp <= G.N;
        const int64_t row = ok ? tp - 1 : 0;
        const VT v = __builtin_nontemporal_load(reinterpret_cast<const VT*>(dh + row * D + vv * VEC));
        x[j] = ok ? v : VT{};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = tid + j * nthr;
        if (i < C) s0l[i] = sv[j];
        else if (i < C + n1) s1l[i - C] = sv[j];
    }
    __syncthreads();
    if (u < units) {
        float a2[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) a2[e] = 0.f;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            float a1[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) a1[e] = 0.f;
#pragma unroll
            for (int c = 0; c < P; ++c) {
                const int j = i * P + c;
#pragma unroll
                for (int e = 0; e < VEC; ++e) a1[e] += to_f(x[j][e]);
                const int32_t s0 = s0l[u * U + j];
                if (s0 >= 0) *reinterpret_cast<VT*>(dgh + (int64_t)s0 * D + vv * VEC) = x[j];
            }
            if (G.L > 1) {
                const int32_t s1 = s1l[u * P + i];
                if (s1 >= 0) store(s1, vv, a1);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) a2[e] += a1[e];
        }
        if (G.L > 2) {
            const int32_t s2 = slot_of(2, c0 / U + u);
            if (s2 >= 0) store(s2, vv, a2);
            if (G.L > 3)
#pragma unroll
                for (int e = 0; e < VEC; ++e) lrow[u * D + vv * VEC + e] = a2[e];
        }
    }
    // levels 3 .. L-1 from the level below, kept in LDS
    int prev = 0, cur = units * D, n_prev = units;
    for (int l = 3; l < G.L; ++l) {
        __syncthreads();
        const int n = n_prev / P;
        const int64_t kl = c0 / G.pw[l];
        for (int task = tid; task < n * NVEC; task += nthr) {
            const int e = task / NVEC, w = task % NVEC;
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
#pragma unroll
            for (int c = 0; c < P; ++c)
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += lrow[prev + (e * P + c) * D + w * VEC + i];
            if (l + 1 < G.L)
#pragma unroll
                for (int i = 0; i < VEC; ++i) lrow[cur + e * D + w * VEC + i] = acc[i];
            const int32_t sl = slot_of(l, kl + e);
            if (sl >= 0) store(sl, w, acc);
        }
        prev = cur;
        cur += n * D;
        n_prev = n;
    }
}

// D[g] = dOg[g] . Og[g] (f32; per lane VEC products in order, then the lanes
// of the row in order -- the order of the dense path) and -LSE/scale, per slot.
template <typename T>
__global__ __launch_bounds__(kThreads) void slot_dot_kernel(const T* __restrict__ dog, const float* __restrict__ og,
                                                            const float* __restrict__ lse, float inv_scale,
                                                            float* __restrict__ nd, float* __restrict__ nl,
                                                            int64_t S, int64_t d) {
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    __shared__ float dpart[kRows * 32];
    const int nvec = (int)(d / VEC);
    const int64_t bh = blockIdx.y, s0 = (int64_t)blockIdx.x * kRows;
    for (int task = threadIdx.x; task < kRows * nvec; task += kThreads) {
        const int sl = task / nvec, vv = task - sl * nvec;
        float dp = 0.f;
        if (s0 + sl < S) {
            const int64_t row = (bh * S + s0 + sl) * d + vv * VEC;
            const VT v = __builtin_nontemporal_load(reinterpret_cast<const VT*>(dog + row));
            float ov[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const floatx4 o4 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(og + row + e));
                ov[e] = o4[0]; ov[e + 1] = o4[1]; ov[e + 2] = o4[2]; ov[e + 3] = o4[3];
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) dp += to_f(v[e]) * ov[e];
        }
        dpart[sl * nvec + vv] = dp;
    }
    __syncthreads();
    for (int sl = threadIdx.x; sl < kRows; sl += kThreads) {
        const int64_t s = s0 + sl;
        if (s < S) {
            float acc = 0.f;
            for (int vv = 0; vv < nvec; ++vv) acc += dpart[sl * nvec + vv];
            nd[bh * S + s] = -acc;
            nl[bh * S + s] = -lse[bh * S + s] * inv_scale;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const T* __restrict__ x, T* xT, int64_t S,
                                                             int64_t S_pad, int64_t d) {
    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const int ld = (int)d + VEC, nvec = (int)(d / VEC);
    const int64_t bh = blockIdx.y, s0 = (int64_t)blockIdx.x * kRows;
    for (int task = threadIdx.x; task < kRows * nvec; task += kThreads) {
        const int sl = task / nvec, vv = task - sl * nvec;
        VT val = {};
        if (s0 + sl < S) val = *reinterpret_cast<const VT*>(x + (bh * S + s0 + sl) * d + vv * VEC);
#pragma unroll
        for (int i = 0; i < VEC; ++i) tile[sl * ld + vv * VEC + i] = val[i];
    }
    __syncthreads();
    store_transposed(tile, ld, d, xT + bh * d * S_pad, S_pad, s0);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dense_prep_kernel(const T* __restrict__ dout, const float* __restrict__ o,
                                                              const float* __restrict__ lse, float inv_scale,
                                                              T* doT, float* __restrict__ nd,
                                                              float* __restrict__ nl, int64_t S, int64_t S_pad,
                                                              int64_t d) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const int ld = (int)d + VEC, nvec = (int)(d / VEC);
    T* tile = reinterpret_cast<T*>(smem);
    float* dpart = reinterpret_cast<float*>(smem + sizeof(T) * kRows * ld);
    const int64_t bh = blockIdx.y, s0 = (int64_t)blockIdx.x * kRows;
    for (int task = threadIdx.x; task < kRows * nvec; task += kThreads) {
        const int sl = task / nvec, vv = task - sl * nvec;
        VT val = {};
        float dp = 0.f;
        if (s0 + sl < S) {
            val = *reinterpret_cast<const VT*>(dout + (bh * S + s0 + sl) * d + vv * VEC);
            const float* ov = o + (bh * S + s0 + sl) * d + vv * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) dp += to_f(val[e]) * ov[e];
        }
        if (doT)
#pragma unroll
            for (int i = 0; i < VEC; ++i) tile[sl * ld + vv * VEC + i] = val[i];
        dpart[sl * nvec + vv] = dp;
    }
    __syncthreads();
    for (int sl = threadIdx.x; sl < kRows; sl += kThreads) {
        if (s0 + sl < S) {
            float acc = 0.f;
            for (int vv = 0; vv < nvec; ++vv) acc += dpart[sl * nvec + vv];
            nd[bh * S + s0 + sl] = -acc;
            nl[bh * S + s0 + sl] = -lse[bh * S + s0 + sl] * inv_scale;
        }
    }
    if (doT) store_transposed(tile, ld, d, doT + bh * d * S_pad, S_pad, s0);
}

template <typename T> size_t tile_bytes(int64_t d) { return sizeof(T) * kRows * (d + V16<T>::N); }

}  // namespace

hipError_t launch_gather(const LhGeom& g, int dtype, const void* q, const void* k, const void* v, const void* pyr,
                         const int32_t* gidx, void* const rows[3], void* const cols[3], hipStream_t st) {
    const MapGeo G = make_geo(g);
    dim3 grid((unsigned)(g.S_pad / kRows), (unsigned)g.BH, 3);
    if (dtype == LH_BF16)
        gather_kernel<bf16><<<grid, kThreads, tile_bytes<bf16>(g.d), st>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)pyr, gidx, (bf16*)rows[0], (bf16*)rows[1],
            (bf16*)rows[2], (bf16*)cols[0], (bf16*)cols[1], (bf16*)cols[2], G);
    else
        gather_kernel<float><<<grid, kThreads, tile_bytes<float>(g.d), st>>>(
            (const float*)q, (const float*)k, (const float*)v, (const float*)pyr, gidx, (float*)rows[0],
            (float*)rows[1], (float*)rows[2], (float*)cols[0], (float*)cols[1], (float*)cols[2], G);
    return hipGetLastError();
}

// Calls f.template operator()<L, D>() for the runtime level count and row width.
template <class F>
hipError_t with_levels(int L, int64_t d, F&& f) {
    if (d != 64 && d != 128) return hipErrorInvalidValue;
#define LH_LD(l)                                                                       \
    case l:                                                                            \
        return d == 64 ? f.template operator()<l, 64>() : f.template operator()<l, 128>();
    switch (L) {
        LH_LD(1) LH_LD(2) LH_LD(3) LH_LD(4) LH_LD(5) LH_LD(6) LH_LD(7) LH_LD(8)
        default: return hipErrorInvalidValue;
    }
#undef LH_LD
}

hipError_t launch_scatter_fwd(const LhGeom& g, int dtype, const float* og, const int32_t* gpos, void* o,
                              hipStream_t st) {
    const MapGeo G = make_geo(g);
    const PullLds P = pull_lds(g.p, g.L, g.d);
    dim3 grid((unsigned)((g.N + P.R - 1) / P.R), (unsigned)g.BH);
    const size_t sh = (size_t)P.row_cap * g.d * 4 + (size_t)P.slot_cap * 4;
    return with_levels(g.L, g.d, [&]<int L, int D>() {
        if (dtype == LH_BF16)
            scatter_fwd_kernel<bf16, L, D><<<grid, kThreads, sh, st>>>(og, gpos, (bf16*)o, G, P);
        else
            scatter_fwd_kernel<float, L, D><<<grid, kThreads, sh, st>>>(og, gpos, (float*)o, G, P);
        return hipGetLastError();
    });
}

namespace {
constexpr int kTreeLds = 48 * 1024;

// Block shape of the pyramid form: one lane group of NVEC lanes per p^2 rows
// of the chunk, 256 threads where p^(L-1) allows, otherwise the chunk rounded
// up to a multiple of p^(L-1) and up to 1024 threads; chunk = 0 (slot-centric
// form) when p, d, that thread count or the LDS rule it out.
struct TreeLaunch {
    TreeP P;
    int threads;
    size_t lds;
};
TreeLaunch tree_plan(const LhGeom& g, int dtype) {
    TreeLaunch t{};
    if (g.L < 2 || g.p < 2 || g.p > 4 || (g.d != 64 && g.d != 128)) return t;
    const int64_t nvec = g.d / (dtype == LH_BF16 ? 8 : 4), U = (int64_t)g.p * g.p;
    const int64_t m = g.pw[g.L - 1] > U ? g.pw[g.L - 1] : U;
    int64_t C = (256 / nvec) * U;
    C = (C + m - 1) / m * m;
    int64_t threads = C / U * nvec;   // one lane group per p^2 rows, all in one pass
    if (threads > 1024) return t;
    threads = (threads + 63) / 64 * 64;
    const int64_t n1 = C / g.p;
    if (C + n1 > 4 * threads) return t;   // the kernel stages the slots in four loads per thread
    const int64_t s1_off = C, rows_off = ((C + n1) * 4 + 15) & ~(int64_t)15;
    int64_t rows = 0;
    for (int l = 2; l + 1 < g.L; ++l) rows += C / g.pw[l];
    const int64_t lds = rows_off + rows * g.d * 4;
    if (lds > kTreeLds) return t;
    t.P = TreeP{(int)C, (int)s1_off, (int)rows_off};
    t.threads = (int)threads;
    t.lds = (size_t)lds;
    return t;
}

template <typename T>
hipError_t launch_tree(const LhGeom& g, const TreeLaunch& t, const void* dout, const int32_t* gpos, void* dog,
                       const MapGeo& G, hipStream_t st) {
    dim3 grid((unsigned)(g.N / t.P.chunk + 1), (unsigned)g.BH);
    auto go = [&](auto kern) {
        kern<<<grid, t.threads, t.lds, st>>>((const T*)dout, gpos, (T*)dog, G, t.P);
        return hipGetLastError();
    };
    if (g.d == 64)
        return g.p == 2 ? go(scatter_bwd_tree_kernel<T, 64, 2>)
             : g.p == 3 ? go(scatter_bwd_tree_kernel<T, 64, 3>) : go(scatter_bwd_tree_kernel<T, 64, 4>);
    return g.p == 2 ? go(scatter_bwd_tree_kernel<T, 128, 2>)
         : g.p == 3 ? go(scatter_bwd_tree_kernel<T, 128, 3>) : go(scatter_bwd_tree_kernel<T, 128, 4>);
}
}  // namespace

hipError_t launch_scatter_bwd(const LhGeom& g, int dtype, const void* dout, const float* og, const int32_t* gidx,
                              const int32_t* gpos, const float* lse, float scale, void* dog, void* dogT, float* nd,
                              float* nl, hipStream_t st) {
    const MapGeo G = make_geo(g);
    const TreeLaunch TL = tree_plan(g, dtype);
    if (TL.P.chunk > 0) {
        // pyramid form: every t' in [0, N] lies in one of the chunks
        hipError_t e = dtype == LH_BF16 ? launch_tree<bf16>(g, TL, dout, gpos, dog, G, st)
                                        : launch_tree<float>(g, TL, dout, gpos, dog, G, st);
        if (e != hipSuccess) return e;
        dim3 sg((unsigned)(g.S_pad / kRows), (unsigned)g.BH);
        if (dtype == LH_BF16)
            slot_dot_kernel<bf16><<<sg, kThreads, 0, st>>>((const bf16*)dog, og, lse, 1.f / scale, nd, nl, g.S, g.d);
        else
            slot_dot_kernel<float><<<sg, kThreads, 0, st>>>((const float*)dog, og, lse, 1.f / scale, nd, nl, g.S,
                                                            g.d);
        e = hipGetLastError();
        if (e == hipSuccess && dogT) {   // f32 attention kernels take dOg transposed
            dim3 tg((unsigned)(g.S_pad / kRows), (unsigned)g.BH);
            transpose_kernel<float><<<tg, kThreads, tile_bytes<float>(g.d), st>>>((const float*)dog, (float*)dogT,
                                                                                   g.S, g.S_pad, g.d);
            e = hipGetLastError();
        }
        return e;
    }
    dim3 grid((unsigned)(g.S_pad / kRows), (unsigned)g.BH);
    if (dtype == LH_BF16) {
        const size_t sh = tile_bytes<bf16>(g.d) + 4 * kRows * (g.d / 8);
        scatter_bwd_kernel<bf16><<<grid, kThreads, sh, st>>>((const bf16*)dout, og, gidx, lse, 1.f / scale,
                                                              (bf16*)dog, (bf16*)dogT, nd, nl, G);
    } else {
        const size_t sh = tile_bytes<float>(g.d) + 4 * kRows * (g.d / 4);
        scatter_bwd_kernel<float><<<grid, kThreads, sh, st>>>((const float*)dout, og, gidx, lse, 1.f / scale,
                                                               (float*)dog, (float*)dogT, nd, nl, G);
    }
    return hipGetLastError();
}

hipError_t launch_gather_pool_bwd(const LhGeom& g, int dtype, const float* const dx_g[3], const int32_t* gpos,
                                  void* const dx[3], hipStream_t st) {
    const MapGeo G = make_geo(g);
    const PullLds P = pull_lds(g.p, g.L, g.d);
    dim3 grid((unsigned)((g.N + P.R - 1) / P.R), (unsigned)g.BH, 3);
    const size_t sh = (size_t)P.row_cap * g.d * 4 + (size_t)P.slot_cap * 4;
    return with_levels(g.L, g.d, [&]<int L, int D>() {
        if (dtype == LH_BF16)
            gpool_bwd_kernel<bf16, L, D><<<grid, kThreads, sh, st>>>(dx_g[0], dx_g[1], dx_g[2], gpos, (bf16*)dx[0],
                                                                     (bf16*)dx[1], (bf16*)dx[2], G, P);
        else
            gpool_bwd_kernel<float, L, D><<<grid, kThreads, sh, st>>>(dx_g[0], dx_g[1], dx_g[2], gpos,
                                                                      (float*)dx[0], (float*)dx[1], (float*)dx[2], G,
                                                                      P);
        return hipGetLastError();
    });
}

hipError_t launch_transpose(int dtype, int64_t BH, int64_t S, int64_t S_pad, int64_t d, const void* x, void* xT,
                            hipStream_t st) {
    dim3 grid((unsigned)(S_pad / kRows), (unsigned)BH);
    if (dtype == LH_BF16)
        transpose_kernel<bf16><<<grid, kThreads, tile_bytes<bf16>(d), st>>>((const bf16*)x, (bf16*)xT, S, S_pad, d);
    else
        transpose_kernel<float><<<grid, kThreads, tile_bytes<float>(d), st>>>((const float*)x, (float*)xT, S, S_pad,
                                                                              d);
    return hipGetLastError();
}

hipError_t launch_dense_bwd_prep(int dtype, int64_t BH, int64_t S, int64_t S_pad, int64_t d, const void* dout,
                                 const float* o, const float* lse, float scale, void* doT, float* nd, float* nl,
                                 hipStream_t st) {
    dim3 grid((unsigned)(S_pad / kRows), (unsigned)BH);
    if (dtype == LH_BF16) {
        const size_t sh = tile_bytes<bf16>(d) + 4 * kRows * (d / 8);
        dense_prep_kernel<bf16><<<grid, kThreads, sh, st>>>((const bf16*)dout, o, lse, 1.f / scale, (bf16*)doT,
                                                             nd, nl, S, S_pad, d);
    } else {
        const size_t sh = tile_bytes<float>(d) + 4 * kRows * (d / 4);
        dense_prep_kernel<float><<<grid, kThreads, sh, st>>>((const float*)dout, o, lse, 1.f / scale,
                                                              (float*)doT, nd, nl, S, S_pad, d);
    }
    return hipGetLastError();
}
