// Internal launch interface between the C-ABI layer (lh_api.hip) and the
// kernel translation units.  Every launcher only enqueues on `st`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lighthouse.h"

struct LhGeom {
    int64_t BH, N, d, S, S_pad, M_total, Mu;   // Mu = M_total - N (rows above level 0)
    int p, L;
    int64_t M[LH_MAX_LEVELS];
    int64_t k_eff[LH_MAX_LEVELS];
    int64_t off[LH_MAX_LEVELS + 1];           // level offsets (flat ids)
    int64_t pw[LH_MAX_LEVELS];                // p^l
    int64_t words_off[LH_MAX_LEVELS + 1];     // bitmap word offset of level l (l >= 1)
    int64_t words_total;                      // per head
};

// selection-side kernels (lh_select.hip)
// Pyramid levels 1 .. L-1 of q, k, v into pyr, and the token norms ||q_t||,
// ||k_t|| ([2][BH][N] f32) into norms.
hipError_t launch_pool(const LhGeom& g, int dtype, const void* q, const void* k, const void* v, void* pyr,
                       float* norms, hipStream_t st);
// Token norms ||q_t||, ||k_t|| ([2][BH][N] f32) straight from q and k.
hipError_t launch_norms(const LhGeom& g, int dtype, const void* q, const void* k, float* norms, hipStream_t st);
// Whether the pooling and score passes have an LDS layout for this shape
// (checked on the host before any launch).
bool pool_fits(const LhGeom& g, int dtype);
bool scores_fit(const LhGeom& g);
// Scores of levels >= 1 (max-pooled ||q|| + ||k||) from the token norms.
hipError_t launch_scores(const LhGeom& g, const float* norms, float* sigma, hipStream_t st);
hipError_t launch_topk(const LhGeom& g, const float* sigma, uint32_t* words, int32_t* prefix, hipStream_t st);
hipError_t launch_map(const LhGeom& g, const uint32_t* words, const int32_t* prefix, int32_t* gidx,
                      int32_t* gpos, hipStream_t st);

// data movement (lh_scatter.hip)
hipError_t launch_gather(const LhGeom& g, int dtype, const void* q, const void* k, const void* v,
                         const void* pyr, const int32_t* gidx, void* const rows[3], void* const cols[3],
                         hipStream_t st);
// og: the sub-sequence output, kept in f32 [BH,S,d]
hipError_t launch_scatter_fwd(const LhGeom& g, int dtype, const float* og, const int32_t* gpos, void* o,
                              hipStream_t st);
// also writes nd = -rowsum(dOg * Og) and nl = -lse / scale, the backward's
// per-row offsets of dP and of the raw scores
// (dogT: the transposed copy, f32 only, else null)
hipError_t launch_scatter_bwd(const LhGeom& g, int dtype, const void* dout, const float* og,
                              const int32_t* gidx, const int32_t* gpos, const float* lse, float scale, void* dog,
                              void* dogT, float* nd, float* nl, hipStream_t st);
hipError_t launch_gather_pool_bwd(const LhGeom& g, int dtype, const float* const dx_g[3], const int32_t* gpos,
                                  void* const dx[3], hipStream_t st);
hipError_t launch_transpose(int dtype, int64_t BH, int64_t S, int64_t S_pad, int64_t d, const void* x,
                            void* xT, hipStream_t st);
hipError_t launch_dense_bwd_prep(int dtype, int64_t BH, int64_t S, int64_t S_pad, int64_t d, const void* dout,
                                 const float* o32, const float* lse, float scale, void* doT, float* nd,
                                 float* nl, hipStream_t st);

// attention (lh_attention.hip)
struct AttnArgs {
    int64_t BH, S, S_pad, d;
    float scale;
};
// O32: f32 output [BH,S,d] (always); Ot: optional copy in the input dtype (may be null).
// Vop: V row-major [BH,S,d] for bf16, V^T [BH,d,S_pad] (store_transposed order) for f32.
hipError_t launch_attn_fwd(const AttnArgs& a, int dtype, const void* Q, const void* K, const void* Vop, float* O32,
                           void* Ot, float* lse, hipStream_t st);
// out_f32: dq/dk/dv are f32 (true) or the input dtype (false); nl = -LSE/scale, nd = -D per row.
// QT, dOT, KT: transposed copies, read by the f32 kernels only (null for bf16).
hipError_t launch_attn_dkdv(const AttnArgs& a, int dtype, bool out_f32, const void* Q, const void* K,
                            const void* V, const void* QT, const void* dO, const void* dOT, const float* nl,
                            const float* nd, void* dK, void* dV, hipStream_t st);
hipError_t launch_attn_dq(const AttnArgs& a, int dtype, bool out_f32, const void* Q, const void* K, const void* V,
                          const void* KT, const void* dO, const float* nl, const float* nd, void* dQ,
                          hipStream_t st);

// projections (lh_proj.hip)
struct ProjGeom {
    int64_t B, N, Dm, H, d;
    int splits;                                  // k-splits of the dW product
    size_t ws_wT, ws_part, ws_bytes;             // backward workspace layout (byte offsets)
};
hipError_t launch_qkv_forward(const ProjGeom& g, const void* x, const void* w, void* q, void* k, void* v,
                              hipStream_t st);
hipError_t launch_qkv_backward(const ProjGeom& g, const void* x, const void* w, const void* dq, const void* dk,
                               const void* dv, void* dx, float* dw, void* ws, hipStream_t st);
