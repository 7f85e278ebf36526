// Stage 1 and 2 of Lighthouse Attention on gfx950: the mean pyramid, the
// l2-norm token scores with max-pool inheritance, the exact per-level top-K,
// and the gather map (page "skillsmp.com ... lighthouse-attention", Stage 1-3;
// gist.science technical summary, Methodology 2A-2C).
//
// All of these are bandwidth- or latency-bound; nothing here is a dense
// contraction, so no matrix cores: coalesced 16-byte loads, LDS staging of the
// coarser levels, and wave shuffles for the per-token reductions.
#include <type_traits>

#include "lh_device.h"
#include "lh_internal.h"

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Pyramid: level l entry i = (sum of the p children of level l-1, index
// order, f32) / p; the recursion keeps f32 values, each stored level is one
// rounding to T.  One block = a chunk of tokens (a multiple of p^(L-1)) times
// a slice of DS dimensions; the f32 levels of the chunk stay in LDS.
// ---------------------------------------------------------------------------
// A load of data that the kernel streams through once: marked non-temporal
// so it does not displace cached lines.  Measured per kernel: the l2-norm
// score pass over q and k ran 1.4x and the level-1 pooling pass 1.2x faster
// with it (in the gather of scattered pyramid rows and the dO segment sums of
// the scatter backward it was slower, so those keep ordinary loads).
template <class V>
__device__ __forceinline__ V load_stream(const V* p) { return __builtin_nontemporal_load(p); }
// The pooled levels are stored non-temporally as well: left in the caches as
// dirty lines, they were written back during the next kernels (at 512K tokens
// the score pass ran 35 -> 25 us and the gather 78 -> 56 us without them).

// One lane's chunk of CW elements (as CW / VEC 16-byte vectors): squares
// rounded to f32 and added left to right.
template <typename T, int CW>
__device__ __forceinline__ float sumsq_chunk(const typename V16<T>::type* v) {
#pragma clang fp contract(off)
    constexpr int VEC = V16<T>::N;
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < CW / VEC; ++j)
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float x = to_f(v[j][i]);
            const float sq = x * x;
            a = a + sq;
        }
    return a;
}

__device__ __forceinline__ float tree8(float a) {
#pragma clang fp contract(off)
    const float t = a + __shfl_xor(a, 4, 64);
    const float u = t + __shfl_xor(t, 2, 64);
    return u + __shfl_xor(u, 1, 64);
}

struct PoolP {
    int64_t N, d, BH, Mu;
    int p, L, chunk, DS, nslices, nv_log2;   // DS / VEC = 1 << nv_log2 vectors per row slice
    int sub;                      // tokens per level-1 pass: chunk, or a power of p >= p^2 dividing it
    int64_t offu[LH_MAX_LEVELS];  // row of level l inside a head's pyramid block
    int epc[LH_MAX_LEVELS];       // entries of level l per chunk (chunk / p^l)
    // Token norms ||q_t||, ||k_t|| ([2][BH][N] f32), written by the q and k
    // blocks when their lanes hold whole rows in the norm order's chunks (8
    // lanes of d / 8 elements, or 16 of d / 16), else null (norm_kernel).
    // part_off: LDS float offset of the pass's per-lane partial sums of squares.
    float* norms;
    int part_off;
};

// PAIRS: the token norms' chunks span two lanes (16 lanes per row).
template <typename T, bool PAIRS>
__global__ __launch_bounds__(kThreads) void pool_kernel(const T* __restrict__ x0, const T* __restrict__ x1,
                                                        const T* __restrict__ x2, T* __restrict__ pyr, PoolP P) {
#pragma clang fp contract(off)   // the squares of the norm partials are rounded before the add
    extern __shared__ float lds[];
    constexpr int VEC = V16<T>::N;
    typedef typename V16<T>::type VT;
    const T* x = blockIdx.z == 0 ? x0 : (blockIdx.z == 1 ? x1 : x2);
    const int slice = blockIdx.x % P.nslices;
    const int cidx = blockIdx.x / P.nslices;
    const int64_t c0 = (int64_t)cidx * P.chunk;
    const int len = (int)((P.N - c0) < P.chunk ? (P.N - c0) : P.chunk);
    const int64_t bh = blockIdx.y;
    const int dim0 = slice * P.DS;
    const int nvm = (1 << P.nv_log2) - 1;
    const T* xh = x + bh * P.N * P.d;
    T* ph = pyr + ((int64_t)blockIdx.z * P.BH + bh) * P.Mu * P.d;

    // The chunk is taken in passes of P.sub tokens: level 1 of the pass from
    // the input into a scratch region of LDS, then (L > 2) its level-2
    // entries into the chunk's level-2 array; levels 3 .. L-1 follow from
    // that array.  (With P.sub = chunk this is one pass; smaller passes let
    // whole rows fit the LDS when p^(L-1) is large.)
    const int n1s = P.sub / P.p, n2 = len / (P.p * P.p);
    float* l2 = lds + n1s * P.DS;   // level-2 array of the chunk
    for (int sc = 0; sc < len; sc += P.sub) {
        // Level 1 from the input: two entries per step, every child load issued
        // before any is summed (children summed in index order, then / p).
        const int n1 = (len - sc < P.sub ? len - sc : P.sub) / P.p;
        const int e1 = sc / P.p;   // first level-1 entry of the pass
        const int nt = n1 << P.nv_log2;
        for (int ta = threadIdx.x; ta < nt; ta += 2 * kThreads) {
            int task[2] = {ta, ta + kThreads};
            float acc[2][VEC];
            const T* src[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tk = task[j] < nt ? task[j] : ta;
                src[j] = xh + (c0 + sc + (int64_t)(tk >> P.nv_log2) * P.p) * P.d + dim0 + (tk & nvm) * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[j][i] = 0.f;
            }
            for (int cb = 0; cb < P.p; cb += 4) {
                VT v[2][4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        v[j][u] = VT{};
                        if (cb + u < P.p)
                            v[j][u] = load_stream(reinterpret_cast<const VT*>(src[j] + (int64_t)(cb + u) * P.d));
                    }
                // With the norms, lane vv also sums the squares of its VEC elements of
                // each child row, left to right (norm order).  A norm chunk (d / 8
                // elements) is one lane's VEC or, with 16 lanes per row, two lanes':
                // the odd lane then continues from the even lane's sum.
                const bool nrm = P.norms && blockIdx.z < 2;   // uniform
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (cb + u < P.p)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            float ss = 0.f;
#pragma unroll
                            for (int i = 0; i < VEC; ++i) {
                                const float xv = to_f(v[j][u][i]);
                                acc[j][i] += xv;
                                const float sq = xv * xv;
                                ss = ss + sq;
                            }
                            if (!nrm) continue;
                            int r = task[j] & nvm;
                            if constexpr (PAIRS) {
                                const float even = __shfl_xor(ss, 1, 64);
                                if (r & 1) {
                                    ss = even;
#pragma unroll
                                    for (int i = 0; i < VEC; ++i) {
                                        const float xv = to_f(v[j][u][i]);
                                        const float sq = xv * xv;
                                        ss = ss + sq;
                                    }
                                }
                                r = (r & 1) ? r >> 1 : -1;   // the odd lane holds the chunk's sum
                            }
                            if (r >= 0 && task[j] < nt)
                                lds[P.part_off + ((task[j] >> P.nv_log2) * P.p + cb + u) * 8 + r] = ss;
                        }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (task[j] >= nt) continue;
                const int e = task[j] >> P.nv_log2, vv = task[j] & nvm;
                VT out;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    acc[j][i] = acc[j][i] / (float)P.p;
                    out[i] = static_cast<T>(acc[j][i]);
                }
                if (P.L > 2) {
                    float* dst = lds + e * P.DS + vv * VEC;
#pragma unroll
                    for (int i = 0; i < VEC; ++i) dst[i] = acc[j][i];
                }
                __builtin_nontemporal_store(out, reinterpret_cast<VT*>(ph + (P.offu[1] + (int64_t)cidx * P.epc[1] + e1 + e) * P.d + dim0 + vv * VEC));
            }
        }
        if (P.norms && blockIdx.z < 2) {
            // ||x_t|| of the pass's tokens from the 8 partial sums (the tree of the
            // norm order: (a_r + a_{r+4}), (t_r + t_{r+2}), (u_0 + u_1)), stored contiguously
            __syncthreads();
            const float* part = lds + P.part_off;
            float* nout = P.norms + ((int64_t)blockIdx.z * P.BH + bh) * P.N + c0 + sc;
            for (int t = threadIdx.x; t < n1 * P.p; t += kThreads) {
                const float* a = part + t * 8;
                const float t0 = a[0] + a[4], t1 = a[1] + a[5], t2 = a[2] + a[6], t3 = a[3] + a[7];
                nout[t] = sqrtf((t0 + t2) + (t1 + t3));
            }
            __syncthreads();   // the partials are reused by the next pass
        }
        if (P.L <= 2) continue;
        __syncthreads();
        // Level 2 of the pass from its level 1 in the scratch region.
        const int e2 = sc / (P.p * P.p);
        for (int task = threadIdx.x; task < ((n1 / P.p) << P.nv_log2); task += kThreads) {
            const int e = task >> P.nv_log2, vv = task & nvm;
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
            for (int c = 0; c < P.p; ++c) {
                const float* src = lds + (e * P.p + c) * P.DS + vv * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += src[i];
            }
            VT out;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                acc[i] = acc[i] / (float)P.p;
                out[i] = static_cast<T>(acc[i]);
            }
            if (P.L > 3) {
                float* dst = l2 + (e2 + e) * P.DS + vv * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) dst[i] = acc[i];
            }
            __builtin_nontemporal_store(out, reinterpret_cast<VT*>(ph + (P.offu[2] + (int64_t)cidx * P.epc[2] + e2 + e) * P.d + dim0 + vv * VEC));
        }
        __syncthreads();   // the scratch region is reused by the next pass
    }
    // Levels 3 .. L-1 from the f32 level below, kept in LDS.
    int prev_off = n1s * P.DS, cur_off = prev_off + n2 * P.DS, n_prev = n2;
    for (int l = 3; l < P.L; ++l) {
        const int n = n_prev / P.p;
        for (int task = threadIdx.x; task < (n << P.nv_log2); task += kThreads) {
            const int e = task >> P.nv_log2, vv = task & nvm;
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
            for (int c = 0; c < P.p; ++c) {
                const float* src = lds + prev_off + (e * P.p + c) * P.DS + vv * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += src[i];
            }
            VT out;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                acc[i] = acc[i] / (float)P.p;
                out[i] = static_cast<T>(acc[i]);
            }
            if (l + 1 < P.L) {
                float* dst = lds + cur_off + e * P.DS + vv * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) dst[i] = acc[i];
            }
            __builtin_nontemporal_store(out, reinterpret_cast<VT*>(ph + (P.offu[l] + (int64_t)cidx * P.epc[l] + e) * P.d + dim0 + vv * VEC));
        }
        __syncthreads();
        prev_off = cur_off;
        cur_off += n * P.DS;
        n_prev = n;
    }
}

// ---------------------------------------------------------------------------
// Scores: s_t = ||q_t|| + ||k_t||, f32, with ||x|| = sqrt(SS(x)): eight lanes
// per token; lane r sums the squares of elements [r*d/8, (r+1)*d/8) left to
// right (the product is rounded before the add: no contraction), then the
// xor-4, xor-2, xor-1 butterflies give (a_r + a_{r+4}), (t_r + t_{r+2}),
// (u_0 + u_1).  The norms come from the pooling pass, which streams every q
// and k row anyway (pool_kernel where its lanes hold rows that way,
// norm_kernel otherwise); levels >= 1 take the max over their children (exact).
// ---------------------------------------------------------------------------
struct ScoreP {
    int64_t N, d, BH, Mu;
    int p, L, chunk;
    int64_t offu[LH_MAX_LEVELS];
    int epc[LH_MAX_LEVELS];   // entries of level l per chunk (chunk / p^l)
};

// ||x_t|| of one chunk of tokens of q (blockIdx.z = 0) or k (1), 8 lanes per
// token; every lane first loads its chunks of kScoreU tokens (tok, tok + 32,
// ...) so that kScoreU 16-byte loads per lane are in flight.
constexpr int kScoreU = 4;
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void norm_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        float* __restrict__ norms, ScoreP P) {
#pragma clang fp contract(off)
    typedef typename V16<T>::type VT;
    const int64_t bh = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * P.chunk;
    const int len = (int)((P.N - c0) < P.chunk ? (P.N - c0) : P.chunk);
    constexpr int CW = D / 8, NV = CW / V16<T>::N, STEP = kThreads / 8;
    const int r = threadIdx.x & 7;
    const T* xb = (blockIdx.z == 0 ? q : k) + (bh * P.N + c0) * D + r * CW;
    float* nb = norms + ((int64_t)blockIdx.z * P.BH + bh) * P.N + c0;
    for (int tok0 = threadIdx.x >> 3; tok0 < len; tok0 += kScoreU * STEP) {
        VT xv[kScoreU][NV];
#pragma unroll
        for (int u = 0; u < kScoreU; ++u) {
            const int tok = tok0 + u * STEP < len ? tok0 + u * STEP : tok0;   // tail: repeat a valid token
#pragma unroll
            for (int j = 0; j < NV; ++j) xv[u][j] = load_stream(reinterpret_cast<const VT*>(xb + (int64_t)tok * D) + j);
        }
#pragma unroll
        for (int u = 0; u < kScoreU; ++u) {
            const float ss = tree8(sumsq_chunk<T, CW>(xv[u]));
            if (r == 0 && tok0 + u * STEP < len) nb[tok0 + u * STEP] = sqrtf(ss);
        }
    }
}

__global__ __launch_bounds__(kThreads) void score_kernel(const float* __restrict__ norms,
                                                         float* __restrict__ sigma, ScoreP P) {
#pragma clang fp contract(off)
    extern __shared__ float lds[];
    const int64_t bh = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * P.chunk;
    const int len = (int)((P.N - c0) < P.chunk ? (P.N - c0) : P.chunk);
    const float* nq = norms + bh * P.N + c0;
    const float* nk = norms + (P.BH + bh) * P.N + c0;
    for (int t = threadIdx.x; t < len; t += kThreads) lds[t] = nq[t] + nk[t];
    __syncthreads();
    int prev_off = 0, cur_off = len;
    int n_prev = len;
    float* sg = sigma + bh * P.Mu;
    for (int l = 1; l < P.L; ++l) {
        const int n = n_prev / P.p;
        const int64_t e0 = (int64_t)blockIdx.x * P.epc[l];
        for (int e = threadIdx.x; e < n; e += kThreads) {
            float m = lds[prev_off + e * P.p];
            for (int c = 1; c < P.p; ++c) m = fmaxf(m, lds[prev_off + e * P.p + c]);
            lds[cur_off + e] = m;
            sg[P.offu[l] + e0 + e] = m;
        }
        __syncthreads();
        prev_off = cur_off;
        cur_off += n;
        n_prev = n;
    }
}

// ---------------------------------------------------------------------------
// Exact top-K of one level of one head: one block of 1024 threads.
// Scores are non-negative floats, so their bit patterns order like the
// values.  An MSB-first radix select (12, 12 and 8 bits) finds the k-th
// largest value tau and how many entries equal to tau must be taken; those
// are the lowest-index ones (ties go to the lower index).  The result is a
// bitmap of the level plus the exclusive popcount prefix of each word.
// ---------------------------------------------------------------------------
struct TopkP {
    int64_t BH, Mu, words_total;
    int L;
    int64_t M[LH_MAX_LEVELS], k_eff[LH_MAX_LEVELS], offu[LH_MAX_LEVELS], woff[LH_MAX_LEVELS];
};

constexpr int kTopkThreads = 1024;

// Exclusive scan over the 1024 threads of a block; *total = sum of all.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    if (wid == 0) {
        uint32_t t = lane < 16 ? wsum[lane] : 0u;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const uint32_t y = __shfl_up(t, o, 64);
            if (lane >= o) t += y;
        }
        if (lane < 16) wsum[16 + lane] = t;
    }
    __syncthreads();
    const uint32_t base = wid > 0 ? wsum[16 + wid - 1] : 0u;
    *total = wsum[31];
    const uint32_t res = base + x - v;
    __syncthreads();
    return res;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += (uint32_t)__shfl_xor((int)x, o, 64);
    return x;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ sigma,
                                                            uint32_t* __restrict__ words,
                                                            int32_t* __restrict__ prefix, TopkP P) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t wsum[32];
    __shared__ uint32_t s_bin, s_above;
    const int l = blockIdx.x + 1;
    const int64_t bh = blockIdx.y;
    const int64_t M = P.M[l];
    const uint32_t kk = (uint32_t)P.k_eff[l];
    const uint32_t* sg = reinterpret_cast<const uint32_t*>(sigma + bh * P.Mu + P.offu[l]);
    uint32_t* W = words + bh * P.words_total + P.woff[l];
    int32_t* PC = prefix + bh * P.words_total + P.woff[l];
    const int64_t nw = (M + 31) / 32;
    const int tid = threadIdx.x;
    const bool all = (int64_t)kk >= M;
    constexpr int kB = 8;   // loads in flight per thread (per lane of a wave in the bitmap pass)

    uint32_t tau = 0, take = 0;
    if (!all) {
        uint32_t pre = 0, pmask = 0, remaining = kk;
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
            const uint32_t dmask = pass == 2 ? 0xFFu : 0xFFFu;
            for (int b = tid; b < 4096; b += kTopkThreads) hist[b] = 0;
            __syncthreads();
            for (int64_t i0 = tid; i0 < M; i0 += (int64_t)kTopkThreads * kB) {   // kB loads in flight
                uint32_t uu[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int64_t i = i0 + (int64_t)j * kTopkThreads;
                    uu[j] = i < M ? sg[i] : 0u;
                }
#pragma unroll
                for (int j = 0; j < kB; ++j)
                    if (i0 + (int64_t)j * kTopkThreads < M && (uu[j] & pmask) == pre)
                        atomicAdd(&hist[(uu[j] >> shift) & dmask], 1u);
            }
            __syncthreads();
            const int g = kTopkThreads - 1 - tid;     // descending bins
            uint32_t hb[4];
            uint32_t gs = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hb[j] = hist[4 * g + j];
                gs += hb[j];
            }
            uint32_t tot;
            uint32_t above = block_excl_scan(gs, wsum, &tot);
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (above < remaining && remaining <= above + hb[j]) {
                    s_bin = 4 * g + j;
                    s_above = above;
                }
                above += hb[j];
            }
            __syncthreads();
            const uint32_t b = s_bin;
            remaining -= s_above;
            pre |= b << shift;
            pmask |= dmask << shift;
            __syncthreads();
        }
        tau = pre;
        take = remaining;
    }

    // Bitmap and word prefixes.  Wave j owns the entries [j per, (j+1) per) of
    // the level (per a multiple of 64, so two whole words per 64 entries):
    // it counts its entries above tau and equal to tau, one exchange gives every
    // wave the ties and selected entries before its range, and it then walks
    // its range 64 entries at a time -- coalesced reads, ballots for the bits,
    // the ties taken in index order -- with running counts of its own.
    const int lane = tid & 63, wid = tid >> 6;
    constexpr int kWaves = kTopkThreads / 64;
    const int64_t per = (M + 64 * kWaves - 1) / (64 * kWaves) * 64;
    const int64_t c0 = wid * per, c1 = c0 + per < M ? c0 + per : M;
    uint32_t n_gt = 0, n_eq = 0;
    for (int64_t g0 = c0; g0 < c1; g0 += 64 * kB) {
        uint32_t uu[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t i = g0 + 64 * j + lane;
            uu[j] = i < c1 ? sg[i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const bool in = g0 + 64 * j + lane < c1;
            n_gt += (in && (all || uu[j] > tau)) ? 1u : 0u;
            n_eq += (in && !all && uu[j] == tau) ? 1u : 0u;
        }
    }
    n_gt = wave_sum(n_gt);
    n_eq = wave_sum(n_eq);
    if (lane == 0) {
        hist[wid] = n_gt;
        hist[kWaves + wid] = n_eq;
    }
    __syncthreads();
    uint32_t carry_tie = 0, carry_pc = 0;   // ties and selected entries before this wave's range
    for (int j = 0; j < wid; ++j) {
        const uint32_t e = hist[kWaves + j];
        const uint32_t e_sel = take > carry_tie ? (take - carry_tie < e ? take - carry_tie : e) : 0u;
        carry_pc += hist[j] + e_sel;
        carry_tie += e;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t g0 = c0; g0 < c1; g0 += 64 * kB) {
        uint32_t uu[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t i = g0 + 64 * j + lane;
            uu[j] = i < c1 ? sg[i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t i0 = g0 + 64 * j;
            if (i0 >= c1) break;
            const bool in = i0 + lane < c1;
            const bool gt = in && (all || uu[j] > tau);
            const bool eq = in && !all && uu[j] == tau;
            const uint64_t eqm = __ballot(eq);
            const bool sel = gt || (eq && carry_tie + (uint32_t)__popcll(eqm & below) < take);
            const uint64_t selm = __ballot(sel);
            if (lane == 0) {
                const int64_t w = i0 / 32;
                W[w] = (uint32_t)selm;
                PC[w] = (int32_t)carry_pc;
                if (w + 1 < nw) {
                    W[w + 1] = (uint32_t)(selm >> 32);
                    PC[w + 1] = (int32_t)(carry_pc + (uint32_t)__popc((uint32_t)selm));
                }
            }
            carry_tie += (uint32_t)__popcll(eqm);
            carry_pc += (uint32_t)__popcll(selm);
        }
    }
}

// ---------------------------------------------------------------------------
// Gather map: each pyramid entry finds whether it is selected and, if so, its
// slot = number of selected entries ordered before it by (span end, level).
// With P_l[x] = selected level-l entries among [0, x):
//   slot(l, i) = P_l[i] + sum_{l'<l} P_l'[(i+1) p^(l-l')]
//                       + sum_{l'>l} P_l'[ceil((i+1)/p^(l'-l)) - 1].
// Level l-1 entries are selected exactly when their parent is in T_l, so
// P_{l-1}[x] = p * #T_l[0, x/p) + (x mod p) * [x/p in T_l]; the coarsest
// level is whole, P_{L-1}[x] = x.
// ---------------------------------------------------------------------------
struct MapP {
    int64_t BH, M_total, S, words_total;
    int p, L;
    int64_t M[LH_MAX_LEVELS], k_eff[LH_MAX_LEVELS], off[LH_MAX_LEVELS + 1], pw[LH_MAX_LEVELS],
        woff[LH_MAX_LEVELS];
};

// Entries per head stay below 2^31 (the plan refuses more), so the map works
// in 32-bit indices; (i + 1) p^(l - l') < 2N fits as well.
__device__ __forceinline__ bool t_bit(const uint32_t* W, uint32_t y) { return (W[y >> 5] >> (y & 31)) & 1u; }

__device__ __forceinline__ uint32_t sel_before(const MapP& P, const uint32_t* Wh, const int32_t* PCh, int lp,
                                               uint32_t x) {
    if (lp == P.L - 1) return x;
    const uint32_t p = (uint32_t)P.p;
    const uint32_t y = x / p, r = x - y * p;
    const uint32_t* W = Wh + P.woff[lp + 1];
    const int32_t* PC = PCh + P.woff[lp + 1];
    uint32_t c;
    if (y >= (uint32_t)P.M[lp + 1]) {
        c = (uint32_t)P.k_eff[lp + 1];
    } else {
        const uint32_t m = (1u << (y & 31)) - 1u;
        c = (uint32_t)PC[y >> 5] + (uint32_t)__popc(W[y >> 5] & m);
    }
    c *= p;
    if (r && y < (uint32_t)P.M[lp + 1] && t_bit(W, y)) c += r;
    return c;
}

constexpr int kMapEnt = 4;   // pyramid entries per thread, kThreads apart (coalesced stores)

__global__ __launch_bounds__(kThreads) void map_kernel(const uint32_t* __restrict__ words,
                                                       const int32_t* __restrict__ prefix,
                                                       int32_t* __restrict__ gidx, int32_t* __restrict__ gpos,
                                                       MapP P) {
    const int64_t bh = blockIdx.y;
    const uint32_t* Wh = words + bh * P.words_total;
    const int32_t* PCh = prefix + bh * P.words_total;
    const uint32_t first = blockIdx.x * (uint32_t)(kThreads * kMapEnt) + threadIdx.x;
    // every entry's level and selection bit first (their loads in flight together) ...
    uint32_t ii[kMapEnt];
    int lv[kMapEnt];
    bool sel[kMapEnt];
#pragma unroll
    for (int e = 0; e < kMapEnt; ++e) {
        const uint32_t id = first + e * kThreads;
        int l = 0;
        while (l < P.L - 1 && (int64_t)id >= P.off[l + 1]) ++l;
        lv[e] = l;
        ii[e] = id - (uint32_t)P.off[l];
        sel[e] = (int64_t)id < P.M_total &&
                 (l == P.L - 1 || t_bit(Wh + P.woff[l + 1], ii[e] / (uint32_t)P.p));
    }
    // ... then the slots of the selected ones
#pragma unroll
    for (int e = 0; e < kMapEnt; ++e) {
        const uint32_t id = first + e * kThreads;
        if ((int64_t)id >= P.M_total) continue;
        int64_t pos = -1;
        if (sel[e]) {
            const int l = lv[e];
            const uint32_t i = ii[e];
            uint32_t q = sel_before(P, Wh, PCh, l, i);
            for (int lp = 0; lp < l; ++lp) q += sel_before(P, Wh, PCh, lp, (i + 1) * (uint32_t)P.pw[l - lp]);
            for (int lp = l + 1; lp < P.L; ++lp) {
                const uint32_t n = (uint32_t)P.pw[lp - l];
                q += sel_before(P, Wh, PCh, lp, (i + n) / n - 1);
            }
            pos = q < (uint32_t)P.S ? (int64_t)q : -1;   // always in range for a consistent bitmap
        }
        gpos[bh * P.M_total + id] = (int32_t)pos;
        if (pos >= 0) gidx[bh * P.S + pos] = (int32_t)id;
    }
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ---------------------------------------------------------------------------
namespace {
// Score geometry: chunks of a multiple of p^(L-1) tokens (at least 1024 where N allows).
ScoreP score_params(const LhGeom& g) {
    ScoreP P{};
    P.N = g.N; P.d = g.d; P.BH = g.BH; P.Mu = g.Mu; P.p = g.p; P.L = g.L;
    for (int l = 0; l < g.L; ++l) P.offu[l] = l ? g.off[l] - g.N : 0;
    int64_t chunk = g.pw[g.L - 1];
    while (chunk < 1024 && chunk * 2 <= g.N) chunk *= 2;
    P.chunk = (int)chunk;
    for (int l = 0; l < g.L; ++l) P.epc[l] = (int)(chunk / g.pw[l]);
    return P;
}

// Pooling geometry: a chunk of tokens (a multiple of p^(L-1)), taken in
// passes of `sub` tokens, over row slices of DS elements, so that the f32
// levels fit the LDS.  False where no such split fits.
struct PoolShape {
    int64_t chunk, sub, lds;
    int DS;
};
constexpr int64_t kPoolLds = 48 * 1024;   // a few blocks per CU
bool pool_shape(const LhGeom& g, int dtype, PoolShape* out) {
    const int VEC = dtype == LH_BF16 ? 8 : 4;
    int64_t chunk = g.pw[g.L - 1];
    while (chunk < 256 && chunk * 2 <= g.N) chunk *= 2;
    // chunk must stay a multiple of p^(L-1): it is p^(L-1) * 2^j
    int DS = (int)g.d;
    // f32 LDS: one pass's level 1 (sub / p entries) plus the chunk's levels 2 .. L-1
    auto lds_bytes = [&](int64_t ch, int64_t sub, int ds) {
        int64_t ent = sub / g.p;
        for (int l = 2; l < g.L; ++l) ent += ch / g.pw[l];
        return ent * ds * 4;
    };
    while (lds_bytes(chunk, chunk, DS) > kPoolLds && chunk > g.pw[g.L - 1]) chunk /= 2;
    // whole rows in passes of p^j tokens (j >= 2, dividing p^(L-1) and so the
    // chunk); where no pass fits whole rows, slice the rows of one pass over the
    // chunk, or, where even the narrowest slice of that does not fit, of the
    // smallest pass
    int64_t sub = chunk;
    for (int j = g.L - 2; j >= 2 && lds_bytes(chunk, sub, DS) > kPoolLds; --j) sub = g.pw[j];
    if (lds_bytes(chunk, sub, DS) > kPoolLds && lds_bytes(chunk, chunk, VEC) <= kPoolLds) sub = chunk;
    while (lds_bytes(chunk, sub, DS) > kPoolLds && DS > VEC) DS /= 2;
    const int64_t lds = lds_bytes(chunk, sub, DS);
    if (lds > 64 * 1024 || chunk > INT32_MAX) return false;
    *out = PoolShape{chunk, sub, lds, DS};
    return true;
}

// The score pass keeps one chunk's levels in LDS (f32).
constexpr int64_t kScoreMaxChunk = 16384;
}  // namespace

bool pool_fits(const LhGeom& g, int dtype) {
    PoolShape s;
    return g.L < 2 || pool_shape(g, dtype, &s);
}
bool scores_fit(const LhGeom& g) { return g.L < 2 || score_params(g).chunk <= kScoreMaxChunk; }

// Token norms of q and k by their own pass (shapes the pooling pass does not
// cover, and scoring straight from q and k).
hipError_t launch_norms(const LhGeom& g, int dtype, const void* q, const void* k, float* norms, hipStream_t st) {
    if (g.L < 2) return hipSuccess;
    const ScoreP P = score_params(g);
    dim3 grid((unsigned)ceil_div(g.N, P.chunk), (unsigned)g.BH, 2);
    if (g.d != 64 && g.d != 128) return hipErrorInvalidValue;
    if (dtype == LH_BF16) {
        if (g.d == 64) norm_kernel<bf16, 64><<<grid, kThreads, 0, st>>>((const bf16*)q, (const bf16*)k, norms, P);
        else norm_kernel<bf16, 128><<<grid, kThreads, 0, st>>>((const bf16*)q, (const bf16*)k, norms, P);
    } else {
        if (g.d == 64) norm_kernel<float, 64><<<grid, kThreads, 0, st>>>((const float*)q, (const float*)k, norms, P);
        else norm_kernel<float, 128><<<grid, kThreads, 0, st>>>((const float*)q, (const float*)k, norms, P);
    }
    return hipGetLastError();
}

hipError_t launch_pool(const LhGeom& g, int dtype, const void* q, const void* k, const void* v, void* pyr,
                       float* norms, hipStream_t st) {
    if (g.L < 2) return hipSuccess;
    PoolP P{};
    P.N = g.N; P.d = g.d; P.BH = g.BH; P.Mu = g.Mu; P.p = g.p; P.L = g.L;
    for (int l = 0; l < g.L; ++l) P.offu[l] = l ? g.off[l] - g.N : 0;
    const int VEC = dtype == LH_BF16 ? 8 : 4;
    PoolShape ps;
    if (!pool_shape(g, dtype, &ps)) return hipErrorInvalidValue;
    const int64_t chunk = ps.chunk, sub = ps.sub;
    const int DS = ps.DS;
    P.chunk = (int)chunk; P.sub = (int)sub; P.DS = DS; P.nslices = (int)(g.d / DS);
    while ((VEC << P.nv_log2) < DS) ++P.nv_log2;
    if ((VEC << P.nv_log2) != DS) return hipErrorInvalidValue;
    for (int l = 0; l < g.L; ++l) P.epc[l] = (int)(chunk / g.pw[l]);
    // the q and k blocks give the token norms when whole rows are held by 8 lanes of d / 8 elements or
    // 16 lanes of d / 16 (8 partial sums per token of a pass in LDS)
    size_t sh = (size_t)ps.lds;
    const bool fused = P.nslices == 1 && (DS == 8 * VEC || DS == 16 * VEC) && sh + (size_t)sub * 32 <= 64 * 1024;
    P.norms = fused ? norms : nullptr;
    P.part_off = (int)(sh / 4);
    if (fused) sh += (size_t)sub * 32;
    dim3 grid((unsigned)(ceil_div(g.N, chunk) * P.nslices), (unsigned)g.BH, 3);
    auto launch = [&](auto kern, auto* x) {
        typedef std::remove_const_t<std::remove_pointer_t<decltype(x)>> T;
        kern<<<grid, kThreads, sh, st>>>((const T*)q, (const T*)k, (const T*)v, (T*)pyr, P);
    };
    const bool pairs = fused && DS == 16 * VEC;
    if (dtype == LH_BF16) {
        if (pairs) launch(pool_kernel<bf16, true>, (const bf16*)q);
        else launch(pool_kernel<bf16, false>, (const bf16*)q);
    } else {
        if (pairs) launch(pool_kernel<float, true>, (const float*)q);
        else launch(pool_kernel<float, false>, (const float*)q);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fused) return e;
    return launch_norms(g, dtype, q, k, norms, st);
}

hipError_t launch_scores(const LhGeom& g, const float* norms, float* sigma, hipStream_t st) {
    if (g.L < 2) return hipSuccess;
    const ScoreP P = score_params(g);
    if (P.chunk > kScoreMaxChunk) return hipErrorInvalidValue;   // the chunk's levels in LDS
    int64_t ent = P.chunk;
    for (int l = 1; l < g.L; ++l) ent += P.chunk / g.pw[l];
    dim3 grid((unsigned)ceil_div(g.N, P.chunk), (unsigned)g.BH);
    score_kernel<<<grid, kThreads, ent * 4, st>>>(norms, sigma, P);
    return hipGetLastError();
}

hipError_t launch_topk(const LhGeom& g, const float* sigma, uint32_t* words, int32_t* prefix, hipStream_t st) {
    if (g.L < 2) return hipSuccess;
    TopkP P{};
    P.BH = g.BH; P.Mu = g.Mu; P.words_total = g.words_total; P.L = g.L;
    for (int l = 0; l < g.L; ++l) {
        P.M[l] = g.M[l]; P.k_eff[l] = g.k_eff[l];
        P.offu[l] = l ? g.off[l] - g.N : 0;
        P.woff[l] = g.words_off[l];
    }
    dim3 grid((unsigned)(g.L - 1), (unsigned)g.BH);
    topk_kernel<<<grid, kTopkThreads, 0, st>>>(sigma, words, prefix, P);
    return hipGetLastError();
}

hipError_t launch_map(const LhGeom& g, const uint32_t* words, const int32_t* prefix, int32_t* gidx, int32_t* gpos,
                      hipStream_t st) {
    MapP P{};
    P.BH = g.BH; P.M_total = g.M_total; P.S = g.S; P.words_total = g.words_total; P.p = g.p; P.L = g.L;
    for (int l = 0; l < g.L; ++l) {
        P.M[l] = g.M[l]; P.k_eff[l] = g.k_eff[l]; P.pw[l] = g.pw[l]; P.woff[l] = g.words_off[l];
    }
    for (int l = 0; l <= g.L; ++l) P.off[l] = g.off[l];
    dim3 grid((unsigned)ceil_div(g.M_total, (int64_t)kThreads * kMapEnt), (unsigned)g.BH);
    map_kernel<<<grid, kThreads, 0, st>>>(words, prefix, gidx, gpos, P);
    return hipGetLastError();
}
