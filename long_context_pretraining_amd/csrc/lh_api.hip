// C ABI of the Lighthouse Attention library (declared in include/lighthouse.h):
// host-side validation and sizing, then asynchronous launches on the caller's
// stream.  No allocation and no synchronisation.  State: the per-thread
// measurement probe (lh_set_probe, lh_set_probe_flush), which the data path
// only reads to record events, and the per-device address of the static
// selection workspace of lh_score_topk_noalloc, looked up once under a lock.
#include <math.h>
#include <string.h>

#include <mutex>

#include "lh_device.h"
#include "lh_internal.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }
inline size_t esize(int dtype) { return dtype == LH_BF16 ? 2 : 4; }
// One transposed [B,H,d,N_pad] array of the dense path (f32 only: the bf16
// attention kernels read row-major tiles across their rows), rounded for alignment.
inline size_t dense_transposed_bytes(const lh_desc* d) {
    if (d->dtype != LH_F32) return 0;
    return align_up((size_t)d->B * d->H * d->d * round64(d->N) * esize(d->dtype));
}

bool aligned(const void* p) { return p && ((uintptr_t)p % 16) == 0; }

// Bytes of the pooled levels in the lh_pyramid buffer; the token norms follow.
size_t pyr_levels_bytes(int64_t BH, int64_t Mu, const lh_desc* d) {
    return (size_t)3 * BH * Mu * d->d * esize(d->dtype);
}

// One head's padded sequence of rows fits 32-bit byte offsets (the attention
// kernels' tile loads address a head's rows that way).
bool rows_fit_u32(int64_t rows, const lh_desc* d) {
    return round64(rows) * d->d * (int64_t)esize(d->dtype) < ((int64_t)1 << 32);
}

lh_status plan_impl(const lh_desc* d, lh_plan* out, LhGeom* g) {
    if (!d || !out) return LH_E_ARG;
    if (d->B < 1 || d->H < 1 || d->N < 1 || d->d < 1 || d->p < 2 || d->L < 1 || d->L > LH_MAX_LEVELS || d->k < 1)
        return LH_E_ARG;
    if (d->dtype != LH_F32 && d->dtype != LH_BF16) return LH_E_ARG;
    if (d->d % 8) return LH_E_ARG;
    int64_t pw[LH_MAX_LEVELS];
    pw[0] = 1;
    for (int l = 1; l < d->L; ++l) {
        if (pw[l - 1] > d->N / d->p) return LH_E_ARG;   // p^l would exceed N
        pw[l] = pw[l - 1] * d->p;
    }
    if (d->N % pw[d->L - 1]) return LH_E_ARG;
    if (d->dtype == LH_BF16 && d->d != 64 && d->d != 128) return LH_E_UNSUPPORTED;
    if (d->dtype == LH_F32 && d->d != 64) return LH_E_UNSUPPORTED;

    lh_plan P;
    memset(&P, 0, sizeof(P));
    LhGeom G;
    memset(&G, 0, sizeof(G));
    int64_t off = 0, S = 0, words = 0;
    for (int l = 0; l < d->L; ++l) {
        P.M[l] = d->N / pw[l];
        P.level_off[l] = off;
        off += P.M[l];
        P.k_eff[l] = l ? (d->k < P.M[l] ? d->k : P.M[l]) : 0;
        S += l ? d->p * P.k_eff[l] : 0;
        G.words_off[l] = words;
        if (l) words += (P.M[l] + 31) / 32;
        G.pw[l] = pw[l];
    }
    P.level_off[d->L] = off;
    G.words_off[d->L] = words;
    P.M_total = off;
    P.S = S + P.M[d->L - 1];
    P.S_formula = d->N / pw[d->L - 1] + (int64_t)(d->L - 1) * d->p * d->k;
    P.S_pad = round64(P.S);
    if (P.M_total >= ((int64_t)1 << 31)) return LH_E_UNSUPPORTED;
    // the attention kernels address the S rows of one head with 32-bit byte offsets
    if (!rows_fit_u32(P.S, d)) return LH_E_UNSUPPORTED;

    const int64_t BH = d->B * d->H, Mu = P.M_total - d->N;
    const size_t e = esize(d->dtype);
    const size_t row = (size_t)BH * P.S * d->d * e;          // [BH,S,d] dtype
    // [BH,d,S_pad] dtype: transposed copies, taken by the f32 attention kernels only
    const size_t colT = d->dtype == LH_F32 ? (size_t)BH * d->d * P.S_pad * e : 0;
    const size_t rowf = (size_t)BH * P.S * d->d * 4;         // [BH,S,d] f32
    const size_t vec = (size_t)BH * P.S * 4;                 // [BH,S] f32

    // pooled levels of q, k, v, then (L > 1) the token norms ||q_t||, ||k_t|| that the scores start from
    P.pyr_bytes = pyr_levels_bytes(BH, Mu, d) + (d->L > 1 ? (size_t)2 * BH * d->N * 4 : 0);
    // level scores, top-K bitmaps and their prefixes, then (L > 1) room for the token norms when they
    // are computed from q and k rather than taken from the pyramid buffer
    P.sel_ws_bytes = align_up((size_t)BH * Mu * 4) + 2 * align_up((size_t)BH * words * 4) +
                     (d->L > 1 ? align_up((size_t)2 * BH * d->N * 4) : 0);
    size_t o = 0;
    const size_t fwd_sizes[8] = {row, row, row, colT, colT, colT, rowf, vec};
    for (int i = 0; i < 8; ++i) { P.fwd_off[i] = o; o += align_up(fwd_sizes[i]); }
    P.fwd_ws_bytes = o;
    o = 0;
    const size_t bwd_sizes[7] = {row, colT, vec, rowf, rowf, rowf, vec};
    for (int i = 0; i < 7; ++i) { P.bwd_off[i] = o; o += align_up(bwd_sizes[i]); }
    P.bwd_ws_bytes = o;
    const size_t dT = dense_transposed_bytes(d);
    P.dense_fwd_ws_bytes = dT + align_up((size_t)BH * d->N * d->d * 4);
    P.dense_bwd_ws_bytes = 3 * dT + 2 * align_up((size_t)BH * d->N * 4);

    G.BH = BH; G.N = d->N; G.d = d->d; G.S = P.S; G.S_pad = P.S_pad; G.M_total = P.M_total; G.Mu = Mu;
    G.p = d->p; G.L = d->L;
    for (int l = 0; l < d->L; ++l) { G.M[l] = P.M[l]; G.k_eff[l] = P.k_eff[l]; }
    for (int l = 0; l <= d->L; ++l) G.off[l] = P.level_off[l];
    G.words_total = words;
    // the pooling and score passes keep a chunk's levels in LDS: refuse shapes without a layout that fits
    if (!pool_fits(G, d->dtype) || !scores_fit(G)) return LH_E_UNSUPPORTED;
    *out = P;
    if (g) *g = G;
    return LH_OK;
}

inline lh_status dev(hipError_t e) { return e == hipSuccess ? LH_OK : LH_E_DEVICE; }
inline unsigned char* at(void* base, size_t off) { return static_cast<unsigned char*>(base) + off; }
inline const unsigned char* at(const void* base, size_t off) { return static_cast<const unsigned char*>(base) + off; }

float softmax_scale(const lh_desc* d) { return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->d); }

// Measurement hook (lh_set_probe): events recorded around one kernel's
// launches.  The setting belongs to the thread that made it, so calls from
// other threads never see it.
thread_local int g_probe_kernel = -1;
thread_local hipEvent_t g_probe_start = nullptr, g_probe_stop = nullptr;
thread_local void* g_probe_flush = nullptr;   // optional: buffer written just before the probed kernel
thread_local size_t g_probe_flush_bytes = 0;

// Reads `n16` 16-byte words of p: clean lines that take the place of whatever
// L2 and the Infinity Cache held, so the next kernel finds none of its inputs
// cached and has no dirty lines to write back.  The (data-dependent, never
// taken in practice) store keeps the reads from being dropped.
__global__ __launch_bounds__(256) void flush_kernel(const uint4* __restrict__ p, size_t n16, uint4* sink) {
    uint4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
        const uint4 v = p[i];
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u) sink[0] = acc;
}

// Measurement microbenchmarks (lh_peak_hbm, lh_peak_mfma): plain streams of
// 16-byte accesses, and a loop of independent bf16 matrix products: two
// waves per SIMD (eight per block, one block per CU) each issue four
// independent 32x32x16 products per iteration -- one wave alone cannot issue
// them back to back, two keep the matrix core busy.
// Streams n16 16-byte words, 8 per thread per round (all loads issued before
// any store) over a grid-stride of 16384 blocks: MODE 0 copies src to dst, 1
// only reads src (an improbable, data-dependent store keeps the loads), 2 only
// writes dst.  Loads and stores are non-temporal: over 2 GiB (beyond the
// Infinity Cache) non-temporal stores write ~8% faster than plain ones and
// copy ~14% faster.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(256) void hbm_kernel(u32x4_t* __restrict__ dst, const u32x4_t* __restrict__ src,
                                                  size_t n16) {
    constexpr int U = 8;
    const size_t stride = (size_t)gridDim.x * 256;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n16; i0 += U * stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + u * stride;
            v[u] = u32x4_t{(uint32_t)i, 1u, 2u, 3u};
            if (MODE != 2 && i < n16) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + u * stride;
            if (MODE == 1) acc ^= v[u];
            else if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
    if (MODE == 1 && acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
        dst[0] = acc;
}
constexpr int kPeakBlocks = 256;
__global__ __launch_bounds__(512, 1) void mfma_loop_kernel(float* out, int iters) {
    floatx16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = floatx16{};
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (bf16)(0.001f * (float)((threadIdx.x + e) & 63));
        b[e] = (bf16)(0.002f * (float)e);
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;   // out holds kPeakBlocks * 512 floats
}

template <class F>
hipError_t probed(int id, hipStream_t st, F&& launch) {
    const bool on = id == g_probe_kernel && g_probe_start && g_probe_stop;
    if (on) {
        if (g_probe_flush && g_probe_flush_bytes >= 16) {
            flush_kernel<<<2048, 256, 0, st>>>((const uint4*)g_probe_flush, g_probe_flush_bytes / 16,
                                               (uint4*)g_probe_flush);
            const hipError_t f = hipGetLastError();
            if (f != hipSuccess) return f;
        }
        const hipError_t r = hipEventRecord(g_probe_start, st);
        if (r != hipSuccess) return r;
    }
    const hipError_t e = launch();
    if (on && e == hipSuccess) return hipEventRecord(g_probe_stop, st);
    return e;
}

}  // namespace

extern "C" {

lh_status lh_make_plan(const lh_desc* desc, lh_plan* out) { return plan_impl(desc, out, nullptr); }

const char* lh_status_string(int s) {
    switch (s) {
        case LH_OK: return "ok";
        case LH_E_ARG: return "invalid argument (pointer, shape or parameter)";
        case LH_E_UNSUPPORTED: return "unsupported configuration (dtype/d/size not built)";
        case LH_E_WORKSPACE: return "workspace smaller than lh_make_plan reports";
        case LH_E_DEVICE: return "HIP launch failed";
        default: return "unknown status";
    }
}

lh_status lh_pyramid(const lh_desc* desc, const void* q, const void* k, const void* v, void* pyr, size_t pyr_bytes,
                     void* stream) {
    lh_plan P;
    LhGeom g;
    lh_status s = plan_impl(desc, &P, &g);
    if (s != LH_OK) return s;
    if (!aligned(q) || !aligned(k) || !aligned(v)) return LH_E_ARG;
    if (P.pyr_bytes == 0) return LH_OK;
    if (!aligned(pyr)) return LH_E_ARG;
    if (pyr_bytes < P.pyr_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    float* norms = (float*)at(pyr, pyr_levels_bytes(g.BH, g.Mu, desc));
    return dev(probed(LH_KERNEL_POOL, st, [&] { return launch_pool(g, desc->dtype, q, k, v, pyr, norms, st); }));
}

namespace {
// Scores, top-K and the gather map into the selection workspace ws (laid out
// as lh_make_plan sizes it).  The token norms come from pyr when it is given,
// else from q and k by their own pass into the end of ws.
hipError_t score_topk_impl(const LhGeom& g, const lh_desc* desc, const lh_plan& P, const void* q, const void* k,
                           const void* pyr, int32_t* gidx, int32_t* gpos, void* ws, hipStream_t st) {
    float* sigma = (float*)ws;
    const size_t sz_sigma = align_up((size_t)g.BH * g.Mu * 4), sz_w = align_up((size_t)g.BH * g.words_total * 4);
    uint32_t* words = (uint32_t*)at(ws, sz_sigma);
    int32_t* prefix = (int32_t*)at(ws, sz_sigma + sz_w);
    hipError_t e = hipSuccess;
    const float* norms = nullptr;
    if (g.L > 1) {
        if (pyr) {
            norms = (const float*)at(pyr, pyr_levels_bytes(g.BH, g.Mu, desc));
        } else {
            float* own = (float*)at(ws, sz_sigma + 2 * sz_w);
            e = probed(LH_KERNEL_NORM, st, [&] { return launch_norms(g, desc->dtype, q, k, own, st); });
            norms = own;
        }
    }
    if (e == hipSuccess) e = probed(LH_KERNEL_SCORE, st, [&] { return launch_scores(g, norms, sigma, st); });
    if (e == hipSuccess) e = probed(LH_KERNEL_TOPK, st, [&] { return launch_topk(g, sigma, words, prefix, st); });
    if (e == hipSuccess)
        e = probed(LH_KERNEL_MAP, st, [&] { return launch_map(g, words, prefix, gidx, gpos, st); });
    (void)P;
    return e;
}
}  // namespace

// Selection workspace of lh_score_topk_noalloc: one array per GPU, loaded with
// the library's code object and held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address hipGetSymbolAddress gives for the
// current device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[LH_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Bytes of the selection workspace a call uses: the level scores, the top-K
// bitmaps and their prefixes, and the token norms unless they come from pyr.
size_t sel_ws_used(const LhGeom& g, bool norms_from_pyr) {
    const size_t sz_sigma = align_up((size_t)g.BH * g.Mu * 4), sz_w = align_up((size_t)g.BH * g.words_total * 4);
    const size_t norms = (g.L > 1 && !norms_from_pyr) ? align_up((size_t)2 * g.BH * g.N * 4) : 0;
    return sz_sigma + 2 * sz_w + norms;
}
}  // namespace

lh_status lh_score_topk_noalloc(const lh_desc* desc, const void* q, const void* k, const void* pyr, int32_t* gidx,
                                int32_t* gpos, void* stream) {
    lh_plan P;
    LhGeom g;
    lh_status s = plan_impl(desc, &P, &g);
    if (s != LH_OK) return s;
    if (!aligned(q) || !aligned(k) || !aligned(gidx) || !aligned(gpos)) return LH_E_ARG;
    if (pyr && !aligned(pyr)) return LH_E_ARG;
    if (sel_ws_used(g, pyr != nullptr) > (size_t)LH_STATIC_SCRATCH_BYTES) return LH_E_WORKSPACE;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return LH_E_DEVICE;
    return dev(score_topk_impl(g, desc, P, q, k, pyr, gidx, gpos, ws, (hipStream_t)stream));
}

lh_status lh_score_topk(const lh_desc* desc, const void* q, const void* k, const void* pyr, int32_t* gidx,
                        int32_t* gpos, void* ws, size_t ws_bytes, void* stream) {
    lh_plan P;
    LhGeom g;
    lh_status s = plan_impl(desc, &P, &g);
    if (s != LH_OK) return s;
    if (!aligned(q) || !aligned(k) || !aligned(gidx) || !aligned(gpos)) return LH_E_ARG;
    if (pyr && !aligned(pyr)) return LH_E_ARG;
    if (P.sel_ws_bytes && !aligned(ws)) return LH_E_ARG;
    if (ws_bytes < P.sel_ws_bytes) return LH_E_WORKSPACE;
    return dev(score_topk_impl(g, desc, P, q, k, pyr, gidx, gpos, ws, (hipStream_t)stream));
}

lh_status lh_forward(const lh_desc* desc, const void* q, const void* k, const void* v, const void* pyr,
                     const int32_t* gidx, const int32_t* gpos, void* o, void* fwd_ws, size_t fwd_ws_bytes,
                     void* stream) {
    lh_plan P;
    LhGeom g;
    lh_status s = plan_impl(desc, &P, &g);
    if (s != LH_OK) return s;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(gidx) || !aligned(gpos) || !aligned(o) ||
        !aligned(fwd_ws))
        return LH_E_ARG;
    if (P.pyr_bytes && !aligned(pyr)) return LH_E_ARG;
    if (fwd_ws_bytes < P.fwd_ws_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    void* rows[3] = {at(fwd_ws, P.fwd_off[LH_FWD_QG]), at(fwd_ws, P.fwd_off[LH_FWD_KG]), at(fwd_ws, P.fwd_off[LH_FWD_VG])};
    // transposed copies only for the f32 attention kernels (bf16 reads the row-major rows transposed in LDS)
    const bool f32 = desc->dtype == LH_F32;
    void* cols[3] = {nullptr, nullptr, nullptr};
    if (f32) {
        cols[0] = at(fwd_ws, P.fwd_off[LH_FWD_QT]);
        cols[1] = at(fwd_ws, P.fwd_off[LH_FWD_KT]);
        cols[2] = at(fwd_ws, P.fwd_off[LH_FWD_VT]);
    }
    float* og = (float*)at(fwd_ws, P.fwd_off[LH_FWD_O]);
    float* lse = (float*)at(fwd_ws, P.fwd_off[LH_FWD_LSE]);
    hipError_t e = probed(LH_KERNEL_GATHER, st,
                          [&] { return launch_gather(g, desc->dtype, q, k, v, pyr, gidx, rows, cols, st); });
    if (e == hipSuccess) {
        AttnArgs a{g.BH, g.S, g.S_pad, g.d, softmax_scale(desc)};
        e = probed(LH_KERNEL_ATTN_FWD, st, [&] {
            return launch_attn_fwd(a, desc->dtype, rows[0], rows[1], f32 ? cols[2] : rows[2], og, nullptr, lse, st);
        });
    }
    if (e == hipSuccess)
        e = probed(LH_KERNEL_SCATTER_FWD, st, [&] { return launch_scatter_fwd(g, desc->dtype, og, gpos, o, st); });
    return dev(e);
}

lh_status lh_backward(const lh_desc* desc, const int32_t* gidx, const int32_t* gpos, const void* fwd_ws,
                      const void* dout, void* dq, void* dk, void* dv, void* bwd_ws, size_t bwd_ws_bytes,
                      void* stream) {
    lh_plan P;
    LhGeom g;
    lh_status s = plan_impl(desc, &P, &g);
    if (s != LH_OK) return s;
    if (!aligned(gidx) || !aligned(gpos) || !aligned(fwd_ws) || !aligned(dout) || !aligned(dq) || !aligned(dk) ||
        !aligned(dv) || !aligned(bwd_ws))
        return LH_E_ARG;
    if (bwd_ws_bytes < P.bwd_ws_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const float* og = (const float*)at(fwd_ws, P.fwd_off[LH_FWD_O]);
    const float* lse = (const float*)at(fwd_ws, P.fwd_off[LH_FWD_LSE]);
    const bool f32 = desc->dtype == LH_F32;   // only the f32 kernels take transposed copies
    void* dog = at(bwd_ws, P.bwd_off[LH_BWD_DO]);
    void* dogT = f32 ? at(bwd_ws, P.bwd_off[LH_BWD_DOT]) : nullptr;
    float* nd = (float*)at(bwd_ws, P.bwd_off[LH_BWD_NEG_D]);
    float* nl = (float*)at(bwd_ws, P.bwd_off[LH_BWD_NEG_LSE]);
    float* dxg[3] = {(float*)at(bwd_ws, P.bwd_off[LH_BWD_DQ]), (float*)at(bwd_ws, P.bwd_off[LH_BWD_DK]),
                     (float*)at(bwd_ws, P.bwd_off[LH_BWD_DV])};
    hipError_t e = probed(LH_KERNEL_SCATTER_BWD, st, [&] {
        return launch_scatter_bwd(g, desc->dtype, dout, og, gidx, gpos, lse, softmax_scale(desc), dog, dogT, nd, nl,
                                  st);
    });
    const void* Qg = at(fwd_ws, P.fwd_off[LH_FWD_QG]);
    const void* Kg = at(fwd_ws, P.fwd_off[LH_FWD_KG]);
    const void* Vg = at(fwd_ws, P.fwd_off[LH_FWD_VG]);
    AttnArgs a{g.BH, g.S, g.S_pad, g.d, softmax_scale(desc)};
    if (e == hipSuccess)
        e = probed(LH_KERNEL_ATTN_DKDV, st, [&] {
            return launch_attn_dkdv(a, desc->dtype, true, Qg, Kg, Vg, f32 ? at(fwd_ws, P.fwd_off[LH_FWD_QT]) : nullptr,
                                    dog, dogT, nl, nd, dxg[1], dxg[2], st);
        });
    if (e == hipSuccess)
        e = probed(LH_KERNEL_ATTN_DQ, st, [&] {
            return launch_attn_dq(a, desc->dtype, true, Qg, Kg, Vg, f32 ? at(fwd_ws, P.fwd_off[LH_FWD_KT]) : nullptr,
                                  dog, nl, nd, dxg[0], st);
        });
    if (e == hipSuccess) {
        const float* cg[3] = {dxg[0], dxg[1], dxg[2]};
        void* outs[3] = {dq, dk, dv};
        e = probed(LH_KERNEL_GATHER_POOL_BWD, st,
                   [&] { return launch_gather_pool_bwd(g, desc->dtype, cg, gpos, outs, st); });
    }
    return dev(e);
}

lh_status dense_causal_attn(const lh_desc* desc, const void* q, const void* k, const void* v, void* o, float* lse,
                            void* ws, size_t ws_bytes, void* stream) {
    lh_plan P;
    lh_status s = plan_impl(desc, &P, nullptr);
    if (s != LH_OK) return s;
    if (!rows_fit_u32(desc->N, desc)) return LH_E_UNSUPPORTED;   // the dense path attends over all N rows
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(lse) || !aligned(ws)) return LH_E_ARG;
    if (ws_bytes < P.dense_fwd_ws_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int64_t BH = desc->B * desc->H, N = desc->N, N_pad = round64(N);
    const size_t dT = dense_transposed_bytes(desc);
    float* o32 = (float*)at(ws, dT);
    const bool f32 = desc->dtype == LH_F32;   // only the f32 kernels take V^T
    hipError_t e = f32 ? probed(LH_KERNEL_TRANSPOSE, st,
                                [&] { return launch_transpose(desc->dtype, BH, N, N_pad, desc->d, v, ws, st); })
                       : hipSuccess;
    if (e == hipSuccess) {
        AttnArgs a{BH, N, N_pad, desc->d, softmax_scale(desc)};
        e = probed(LH_KERNEL_ATTN_FWD, st,
                   [&] { return launch_attn_fwd(a, desc->dtype, q, k, f32 ? ws : v, o32, o, lse, st); });
    }
    return dev(e);
}

lh_status dense_causal_attn_backward(const lh_desc* desc, const void* q, const void* k, const void* v,
                                     const float* lse, const void* fwd_ws, const void* dout, void* dq, void* dk,
                                     void* dv, void* ws, size_t ws_bytes, void* stream) {
    lh_plan P;
    lh_status s = plan_impl(desc, &P, nullptr);
    if (s != LH_OK) return s;
    if (!rows_fit_u32(desc->N, desc)) return LH_E_UNSUPPORTED;   // the dense path attends over all N rows
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(fwd_ws) || !aligned(lse) || !aligned(dout) ||
        !aligned(dq) || !aligned(dk) || !aligned(dv) || !aligned(ws))
        return LH_E_ARG;
    if (ws_bytes < P.dense_bwd_ws_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int64_t BH = desc->B * desc->H, N = desc->N, N_pad = round64(N);
    const size_t dT = dense_transposed_bytes(desc);
    const bool f32 = desc->dtype == LH_F32;   // only the f32 kernels take Q^T, K^T, dO^T
    void* qT = f32 ? ws : nullptr;
    void* kT = f32 ? at(ws, dT) : nullptr;
    void* doT = f32 ? at(ws, 2 * dT) : nullptr;
    float* nd = (float*)at(ws, 3 * dT);
    float* nl = (float*)at(ws, 3 * dT + align_up((size_t)BH * N * 4));
    const float* o32 = (const float*)at(fwd_ws, dT);
    hipError_t e = f32 ? launch_transpose(desc->dtype, BH, N, N_pad, desc->d, q, qT, st) : hipSuccess;
    if (e == hipSuccess && f32) e = launch_transpose(desc->dtype, BH, N, N_pad, desc->d, k, kT, st);
    if (e == hipSuccess)
        e = probed(LH_KERNEL_DENSE_PREP, st, [&] {
            return launch_dense_bwd_prep(desc->dtype, BH, N, N_pad, desc->d, dout, o32, lse, softmax_scale(desc),
                                         doT, nd, nl, st);
        });
    AttnArgs a{BH, N, N_pad, desc->d, softmax_scale(desc)};
    if (e == hipSuccess)
        e = probed(LH_KERNEL_ATTN_DKDV, st, [&] {
            return launch_attn_dkdv(a, desc->dtype, f32, q, k, v, qT, dout, doT, nl, nd, dk, dv, st);
        });
    if (e == hipSuccess)
        e = probed(LH_KERNEL_ATTN_DQ, st,
                   [&] { return launch_attn_dq(a, desc->dtype, f32, q, k, v, kT, dout, nl, nd, dq, st); });
    return dev(e);
}

namespace {
// The dW product has few 256 x 256 output tiles (3Hd x Dm) and a long k (every
// token): its k is split so that tiles x splits comes close to one block per CU
// (256 CUs), at most 16 ways and never below one 64-token k-block per split.
int proj_splits(int64_t Nc, int64_t Dm, int64_t M) {
    const int64_t tiles = ((Nc + 255) / 256) * ((Dm + 255) / 256);
    int64_t s = 256 / tiles;
    if (s > 16) s = 16;
    if (s > M / 64) s = M / 64;
    return s < 1 ? 1 : (int)s;
}

lh_status proj_geom(const lh_proj_desc* d, ProjGeom* g) {
    if (!d || !g) return LH_E_ARG;
    if (d->B < 1 || d->N < 1 || d->Dm < 1 || d->H < 1 || d->d < 1) return LH_E_ARG;
    if (d->Dm % 64 || d->N % 64 || (d->d != 64 && d->d != 128)) return LH_E_UNSUPPORTED;
    const int64_t Nc = 3 * d->H * d->d, M = d->B * d->N;
    if (Nc * M >= (int64_t(1) << 31) || M * d->Dm >= (int64_t(1) << 31) || Nc * d->Dm >= (int64_t(1) << 31))
        return LH_E_UNSUPPORTED;
    ProjGeom G{};
    G.B = d->B; G.N = d->N; G.Dm = d->Dm; G.H = d->H; G.d = d->d;
    G.splits = proj_splits(Nc, d->Dm, M);
    size_t off = 0;
    G.ws_wT = off; off += align_up((size_t)d->Dm * Nc * 2);
    G.ws_part = off; off += align_up((size_t)G.splits * Nc * d->Dm * 4);
    G.ws_bytes = off;
    *g = G;
    return LH_OK;
}
}  // namespace

lh_status lh_qkv_plan(const lh_proj_desc* desc, size_t* bwd_ws_bytes) {
    ProjGeom g;
    if (!bwd_ws_bytes) return LH_E_ARG;
    const lh_status s = proj_geom(desc, &g);
    if (s == LH_OK) *bwd_ws_bytes = g.ws_bytes;
    return s;
}

lh_status lh_qkv_forward(const lh_proj_desc* desc, const void* x, const void* w, void* q, void* k, void* v,
                         void* stream) {
    ProjGeom g;
    const lh_status s = proj_geom(desc, &g);
    if (s != LH_OK) return s;
    if (!aligned(x) || !aligned(w) || !aligned(q) || !aligned(k) || !aligned(v)) return LH_E_ARG;
    hipStream_t st = (hipStream_t)stream;
    return dev(probed(LH_KERNEL_QKV_FWD, st, [&] { return launch_qkv_forward(g, x, w, q, k, v, st); }));
}

lh_status lh_qkv_backward(const lh_proj_desc* desc, const void* x, const void* w, const void* dq, const void* dk,
                          const void* dv, void* dx, float* dw, void* ws, size_t ws_bytes, void* stream) {
    ProjGeom g;
    const lh_status s = proj_geom(desc, &g);
    if (s != LH_OK) return s;
    if (!aligned(x) || !aligned(w) || !aligned(dq) || !aligned(dk) || !aligned(dv) || !aligned(dx) ||
        !aligned(dw) || !aligned(ws))
        return LH_E_ARG;
    if (ws_bytes < g.ws_bytes) return LH_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    return dev(probed(LH_KERNEL_QKV_BWD, st,
                      [&] { return launch_qkv_backward(g, x, w, dq, dk, dv, dx, dw, ws, st); }));
}

lh_status lh_set_probe(int kernel, void* start_event, void* stop_event) {
    if (kernel < -1 || kernel >= LH_KERNEL_COUNT) return LH_E_ARG;
    g_probe_kernel = (start_event && stop_event) ? kernel : -1;
    g_probe_start = (hipEvent_t)start_event;
    g_probe_stop = (hipEvent_t)stop_event;
    return LH_OK;
}

lh_status lh_peak_hbm(int mode, void* dst, const void* src, size_t bytes, void* stream) {
    if (mode < 0 || mode > 2 || !aligned(dst) || (mode != 2 && !aligned(src)) || bytes % 16 || !bytes)
        return LH_E_ARG;
    hipStream_t st = (hipStream_t)stream;
    const size_t n16 = bytes / 16;
    u32x4_t* d = (u32x4_t*)dst;
    const u32x4_t* s = (const u32x4_t*)src;
    if (mode == 0) hbm_kernel<0><<<16384, 256, 0, st>>>(d, s, n16);
    if (mode == 1) hbm_kernel<1><<<16384, 256, 0, st>>>(d, s, n16);
    if (mode == 2) hbm_kernel<2><<<16384, 256, 0, st>>>(d, s, n16);
    return dev(hipGetLastError());
}

lh_status lh_peak_mfma(float* out, int iters, void* stream) {
    if (!aligned(out) || iters < 1) return LH_E_ARG;
    mfma_loop_kernel<<<kPeakBlocks, 512, 0, (hipStream_t)stream>>>(out, iters);
    return dev(hipGetLastError());
}

lh_status lh_set_probe_flush(void* buffer, size_t bytes) {
    if (bytes && !aligned(buffer)) return LH_E_ARG;
    g_probe_flush = bytes ? buffer : nullptr;
    g_probe_flush_bytes = bytes;
    return LH_OK;
}

}  // extern "C"
