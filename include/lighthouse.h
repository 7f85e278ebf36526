/*
 * lighthouse.h -- C ABI of the Lighthouse Attention layer for MI355X (gfx950).
 *
 * The layer replaces causal attention over N tokens by attention over a short
 * sub-sequence of S pooled and selected entries (arXiv 2605.06554, "Long
 * Context Pre-Training with Lighthouse Attention"; the pages cited below are
 * the skill card at skillsmp.com, "lighthouse-attention", and the technical
 * summary at gist.science/paper/2605.06554):
 *
 *   lh_pyramid     Stage 1: mean-pool Q, K and V into L levels, factor p.
 *   lh_score_topk  Stage 2: l2-norm scores of Q and K, max-pool inheritance,
 *                  per-level top-K, and the gather map.
 *   lh_forward     Stage 3 and 4: gather, dense causal attention on the S
 *                  entries, scatter-back over the ranges R(l, i).
 *   lh_backward    Gradient flow back through scatter, attention, gather and
 *                  pooling to dQ, dK, dV (no gradient through selection).
 *   dense_causal_attn[_backward]  the dense baseline the layer is measured
 *                  against (the same attention kernels at S = N).
 *
 * Conventions shared by every call:
 *  - Tensors are DEVICE pointers, contiguous, row-major, 16-byte aligned.
 *    Q, K, V, O, dO, dQ, dK, dV have shape [B, H, N, d] in the descriptor's
 *    dtype (bf16 = IEEE binary32 upper half, round-to-nearest-even).
 *  - The caller owns all memory and the stream.  The library never allocates,
 *    frees or synchronises; lh_make_plan reports every buffer size and the
 *    calls check the sizes they are given.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream and returns.
 *  - Every argument check runs on the host before any launch; a call that
 *    returns an error has enqueued nothing and written nothing.
 *    LH_E_DEVICE reports a launch failure (hipGetLastError); faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Results are deterministic: no atomics feed any output.
 *  - Supported on the GPU: dtype bf16 with d in {64, 128}, or f32 with
 *    d = 64; p >= 2; 1 <= L <= 8; k >= 1; N a multiple of p^(L-1);
 *    M_total < 2^31 (the maps are int32); p^(L-1) at most 16384 (the
 *    pooling and score passes keep one chunk of that many tokens in LDS;
 *    lh_make_plan returns LH_E_UNSUPPORTED above it).
 */
#ifndef LIGHTHOUSE_H
#define LIGHTHOUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LH_MAX_LEVELS 8

typedef enum { LH_F32 = 0, LH_BF16 = 1 } lh_dtype;

typedef enum {
    LH_OK = 0,
    LH_E_ARG = -1,         /* null/misaligned pointer, bad shape or parameter */
    LH_E_UNSUPPORTED = -2, /* valid for the method, not built here (e.g. d = 96) */
    LH_E_WORKSPACE = -3,   /* a workspace smaller than lh_make_plan reports */
    LH_E_DEVICE = -4       /* a HIP launch failed */
} lh_status;

/* Problem statement (skill card, Stage 1-3): Q, K, V of shape [B,H,N,d],
 * pooling factor p, L levels, budget k per level.  scale <= 0 selects the
 * softmax scale 1/sqrt(d). */
typedef struct {
    int64_t B, H, N, d;
    int32_t p, L, k;
    int32_t dtype;         /* lh_dtype */
    float scale;
} lh_desc;

/* Sizes derived from a descriptor.
 *  M[l]         entries of level l = N / p^l (l = 0..L-1); their total
 *               M_total is at most N p/(p-1) (skill card, Stage 1).
 *  k_eff[l]     entries of level l (l >= 1) whose p children are selected:
 *               min(k, M[l]); k_eff[0] = 0.
 *  level_off[l] flat id of entry (l, i) is level_off[l] + i.
 *  S            gathered entries = M[L-1] + p * sum_{l>=1} k_eff[l];
 *  S_formula    the skill card's N/p^(L-1) + (L-1) p k (Stage 3); the two
 *               differ only when k exceeds the coarsest level, where a
 *               level's budget is clamped to its size.
 *  *_bytes      buffer sizes for the calls below (see each call). */
typedef struct {
    int64_t M[LH_MAX_LEVELS];
    int64_t k_eff[LH_MAX_LEVELS];
    int64_t level_off[LH_MAX_LEVELS + 1];
    int64_t M_total, S, S_formula;
    int64_t S_pad;          /* row length of the transposed arrays: S rounded up to 64 */
    size_t pyr_bytes;       /* lh_pyramid output */
    size_t sel_ws_bytes;    /* lh_score_topk workspace */
    size_t fwd_ws_bytes;    /* lh_forward state, read again by lh_backward */
    size_t bwd_ws_bytes;    /* lh_backward workspace */
    size_t dense_fwd_ws_bytes;
    size_t dense_bwd_ws_bytes;
    /* Byte offsets inside the forward state (each array [B*H] heads, head-major):
     *   FWD_QG, FWD_KG, FWD_VG  gathered Q~, K~, V~   [B,H,S,d] dtype
     *   FWD_QT, FWD_KT, FWD_VT  the same, transposed   [B,H,d,S_pad] dtype (zero past S;
     *                           within each aligned group of 16 slots the order is
     *                           0-3, 8-11, 4-7, 12-15) -- f32 only; for bf16 these
     *                           arrays have size 0 (the kernels read Q~, K~, V~
     *                           transposed out of LDS)
     *   FWD_O                   sub-sequence output O~ [B,H,S,d] f32 (an
     *                           intermediate: kept unrounded for the scatter and
     *                           for D = rowsum(dO~ * O~) in the backward)
     *   FWD_LSE                 row log-sum-exp (natural log) [B,H,S] f32 */
    size_t fwd_off[8];
    /* Inside the backward workspace:
     *   BWD_DO, BWD_DOT  dO~ [B,H,S,d] and transposed [B,H,d,S_pad] (same slot order), dtype;
     *                    the transposed copy only for f32 (size 0 for bf16)
     *   BWD_NEG_D        -rowsum(dO~ * O~) [B,H,S] f32
     *   BWD_DQ, BWD_DK, BWD_DV  dQ~, dK~, dV~ [B,H,S,d] f32
     *   BWD_NEG_LSE      -(row log-sum-exp) / scale [B,H,S] f32: the offset of
     *                    the unscaled scores q.k that P = exp(scale (q.k) - LSE) needs */
    size_t bwd_off[7];
} lh_plan;

enum { LH_FWD_QG = 0, LH_FWD_KG, LH_FWD_VG, LH_FWD_QT, LH_FWD_KT, LH_FWD_VT, LH_FWD_O, LH_FWD_LSE };
enum { LH_BWD_DO = 0, LH_BWD_DOT, LH_BWD_NEG_D, LH_BWD_DQ, LH_BWD_DK, LH_BWD_DV, LH_BWD_NEG_LSE };

/* Host only; validates the descriptor and fills `out`.  No device work.
 * LH_E_UNSUPPORTED also where one head's S rows (padded to 64) of d elements
 * reach 2^32 bytes: the attention kernels address a head's rows with 32-bit
 * byte offsets. */
lh_status lh_make_plan(const lh_desc* desc, lh_plan* out);

/* Stage 1, symmetric pyramid (skill card Stage 1; gist.science 2A).
 * Level l entry i = mean of the p entries p*i .. p*i+p-1 of level l-1 (so the
 * mean of p^l consecutive tokens), computed in f32 with the children summed
 * in index order, stored once rounded to the dtype.
 * pyr: out, [3][B,H,M_total-N,d] dtype (tensor Q, K, V; levels 1..L-1
 * concatenated, level l of a head at row level_off[l]-N), followed (L > 1)
 * by the token norms ||q_t||, ||k_t|| as [2][B,H,N] f32 (the order below,
 * under lh_score_topk), which lh_score_topk may take instead of re-reading
 * Q and K: the pass that pools Q and K reads every row once for both.
 * pyr_bytes given (0 at L = 1: then nothing is written). */
lh_status lh_pyramid(const lh_desc* desc, const void* q, const void* k, const void* v,
                     void* pyr, size_t pyr_bytes, void* stream);

/* Stage 2 and the gather map (skill card Stage 2-3; gist.science 2B-2C).
 * Token score s_t = ||q_t|| + ||k_t|| in f32 (squared norm: 8 contiguous
 * chunks of d/8 summed left to right with the product rounded before the
 * add, then (a_r + a_{r+4}), (t_r + t_{r+2}), (u_0 + u_1); correctly rounded
 * sqrt).  Level l >= 1 scores are the max over the span.  For l = 1..L-1 the
 * k_eff[l] entries first under (score descending, index ascending) are
 * selected and their p children at level l-1 are gathered; the coarsest level
 * is gathered whole.  Gathered order: ascending (last token of the span,
 * level).
 * q, k: in [B,H,N,d] dtype, the layer's queries and keys.
 * pyr:  optional (may be NULL).  NULL: the token norms are computed from q and
 *       k (one more pass over both, into the end of ws).  Non-NULL: the buffer
 *       lh_pyramid filled from these same q and k, earlier on this stream; its
 *       token norms are used instead (bit-identical, and q and k are not read).
 *       The library cannot tell a stale buffer from a current one: a pyramid
 *       of other q, k gives the selection of those.
 * gidx: out [B,H,S] int32, flat id of the entry in each slot.
 * gpos: out [B,H,M_total] int32, slot of each entry or -1.
 * ws:   scratch of sel_ws_bytes; nothing in it needs clearing.  Inputs must
 *       be finite. */
lh_status lh_score_topk(const lh_desc* desc, const void* q, const void* k, const void* pyr,
                        int32_t* gidx, int32_t* gpos, void* ws, size_t ws_bytes, void* stream);

/* lh_score_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without the ws argument.  Its workspace is
 * one array of LH_STATIC_SCRATCH_BYTES per GPU, loaded with the library and
 * held until the process ends; the first call on a device looks up that
 * device's address (hipGetSymbolAddress, with the calling thread's current
 * device, which must be the stream's).  The call allocates nothing.
 * Returns LH_E_WORKSPACE, before any launch, when the selection needs more than
 * that: the level scores and top-K bitmaps, plus the token norms unless pyr is
 * given -- e.g. B*H = 16 at N = 98304 needs 15 MB from q and k; at N = 524288,
 * 78 MB from q and k (refused) or 11 MB with pyr.  Every byte of the array a
 * call reads is written earlier in that same call, so nothing is cleared;
 * calls that overlap on one GPU (other streams, other threads) share the array
 * and race. */
#define LH_STATIC_SCRATCH_BYTES (32u << 20)
lh_status lh_score_topk_noalloc(const lh_desc* desc, const void* q, const void* k, const void* pyr,
                                int32_t* gidx, int32_t* gpos, void* stream);

/* Stage 3 and 4 (skill card Stage 3-4; gist.science 2C).
 * Gathers the S selected triples (level 0 rows from q/k/v, coarser ones from
 * pyr), runs causal softmax attention over them (scale, causal mask with the
 * diagonal; bf16 MFMA with f32 accumulation, or f32 MFMA for f32), then
 * o[t] = sum over levels l of O~[gpos(l, floor((t+1)/p^l) - 1)] for the
 * selected entries, i.e. each entry (l, i) adds into R(l, i) =
 * [i p^l + p^l - 1, i p^l + 2 p^l - 2] clipped at N-1; 0 where nothing lands.
 * o: out [B,H,N,d] dtype.  fwd_ws: out, fwd_ws_bytes, layout in lh_plan;
 * keep it for lh_backward.  gidx/gpos as produced by lh_score_topk (a caller
 * may pass any valid map, e.g. to freeze a selection). */
lh_status lh_forward(const lh_desc* desc, const void* q, const void* k, const void* v,
                     const void* pyr, const int32_t* gidx, const int32_t* gpos,
                     void* o, void* fwd_ws, size_t fwd_ws_bytes, void* stream);

/* Gradient flow (skill card, gradient flow; gist.science 2B): gradient of
 * sum(o * dout) w.r.t. q, k, v with the selection held fixed.
 * dO~[g] = sum of dout over R(l,i) of the entry in slot g (stored in dtype);
 * attention backward in f32 from the forward state; then
 * dX[t] = sum_l p^-l dX~[gpos(l, floor(t/p^l))] over selected entries.
 * dq, dk, dv: out [B,H,N,d] dtype.  fwd_ws: the state lh_forward wrote for
 * the same gidx/gpos.  bwd_ws: scratch of bwd_ws_bytes, layout in lh_plan. */
lh_status lh_backward(const lh_desc* desc, const int32_t* gidx, const int32_t* gpos,
                      const void* fwd_ws, const void* dout, void* dq, void* dk, void* dv,
                      void* bwd_ws, size_t bwd_ws_bytes, void* stream);

/* Dense causal attention over all N tokens (the baseline the pages compare
 * with; equal to the layer at L = 1, skill card "selection-attention
 * decoupling").  o: out [B,H,N,d] dtype; lse: out [B,H,N] f32;
 * ws: out, dense_fwd_ws_bytes: the forward state (V transposed and the
 * output in f32), keep it for the backward.  p, L, k are not used.
 * LH_E_UNSUPPORTED where one head's N rows (padded to 64) of d elements reach
 * 2^32 bytes (32-bit row offsets in the kernels; the backward likewise). */
lh_status dense_causal_attn(const lh_desc* desc, const void* q, const void* k, const void* v,
                            void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of dense_causal_attn from its lse and forward state fwd_ws.
 * dq, dk, dv: out [B,H,N,d] dtype; ws: scratch of dense_bwd_ws_bytes. */
lh_status dense_causal_attn_backward(const lh_desc* desc, const void* q, const void* k,
                                     const void* v, const float* lse, const void* fwd_ws,
                                     const void* dout, void* dq, void* dk, void* dv,
                                     void* ws, size_t ws_bytes, void* stream);

/* Q, K, V projections either side of the layer (skill card: the pipeline
 * starts from the projections of the layer input X; the complexity table
 * lists them as a GEMM of Theta(N d_model d); the gradient flows back through
 * gather into W_Q, W_K, W_V).  bf16 only; Dm a multiple of 64; N a multiple
 * of 64; H*d*3*N*B and B*N*Dm below 2^31.  Products accumulate in f32 on the
 * matrix cores.
 *   x:  [B, N, Dm] bf16, the layer input, row-major.
 *   w:  [3*H*d, Dm] bf16 (out x in): rows 0..Hd-1 project to Q (head h at
 *       rows h*d..), rows Hd..2Hd-1 to K, rows 2Hd..3Hd-1 to V. */
typedef struct {
    int64_t B, N, Dm, H, d;
} lh_proj_desc;

/* Backward workspace size (a transposed copy of W and the split partials of
 * dW).  Host only. */
lh_status lh_qkv_plan(const lh_proj_desc* desc, size_t* bwd_ws_bytes);

/* q = x Wq^T, k = x Wk^T, v = x Wv^T, written as [B, H, N, d] bf16 (the
 * layout lh_pyramid / lh_forward take), one rounding from f32. */
lh_status lh_qkv_forward(const lh_proj_desc* desc, const void* x, const void* w,
                         void* q, void* k, void* v, void* stream);

/* Gradients of the projections given dq, dk, dv [B, H, N, d] bf16 (e.g. from
 * lh_backward): dx = dq Wq + dk Wk + dv Wv  [B, N, Dm] bf16, and
 * dw = [dq dk dv]^T x summed over all B*N tokens  [3*H*d, Dm] f32 (the
 * k-split partials are summed in a fixed order: deterministic).
 * ws: scratch of bwd_ws_bytes from lh_qkv_plan. */
lh_status lh_qkv_backward(const lh_proj_desc* desc, const void* x, const void* w,
                          const void* dq, const void* dk, const void* dv,
                          void* dx, float* dw, void* ws, size_t ws_bytes, void* stream);

/* Static string for a status code. */
const char* lh_status_string(int status);

/* Measurement hook (for benchmarks, not for the data path).  After
 * lh_set_probe(kernel, start, stop), every later call that launches kernel
 * `kernel` records hipEvent_t `start` on its stream just before that launch
 * and `stop` just after it, so hipEventElapsedTime(start, stop) is the
 * kernel's duration as the stream sees it.  kernel = -1 (or null events)
 * switches the hook off.  The setting belongs to the calling thread: calls
 * made from other threads never record the events, so concurrent callers on
 * other threads are unaffected.  The events are owned by the caller. */
enum {
    LH_KERNEL_POOL = 0, LH_KERNEL_SCORE, LH_KERNEL_TOPK, LH_KERNEL_MAP, LH_KERNEL_GATHER,
    LH_KERNEL_ATTN_FWD, LH_KERNEL_SCATTER_FWD, LH_KERNEL_SCATTER_BWD, LH_KERNEL_ATTN_DKDV,
    LH_KERNEL_ATTN_DQ, LH_KERNEL_GATHER_POOL_BWD, LH_KERNEL_TRANSPOSE, LH_KERNEL_DENSE_PREP,
    LH_KERNEL_QKV_FWD, LH_KERNEL_QKV_BWD, LH_KERNEL_NORM,
    LH_KERNEL_COUNT
};
lh_status lh_set_probe(int kernel, void* start_event, void* stop_event);

/* Measurement hook, with lh_set_probe: when `bytes` > 0, every probed launch
 * is preceded (on the same stream, before the start event) by a kernel that
 * reads `bytes` of the device buffer `buffer`, so that the probed
 * kernel starts with caches holding none of its inputs (>= 512 MB clears the
 * 256 MB Infinity Cache; the buffer is read, so no dirty lines are left for
 * the probed kernel to write back).  bytes = 0 switches it off.  Thread-local like
 * lh_set_probe; the buffer is owned by the caller. */
lh_status lh_set_probe_flush(void* buffer, size_t bytes);

/* Measurement microbenchmarks (achievable peaks of this GPU, the second
 * denominators of the benchmark's roofline figures; not part of the layer).
 * lh_peak_hbm: `bytes` (a multiple of 16) streamed with 16-byte accesses,
 * mode 0 copying src to dst (rate = 2 * bytes / time), 1 reading src only, 2
 * writing dst only (dst must hold 16 bytes in mode 1; src may be NULL in mode
 * 2).  lh_peak_mfma: 256 blocks of 8 waves, each wave
 * issuing `iters` x 4 independent v_mfma_f32_32x32x16_bf16 (32768 flops
 * each): 256 * 8 * 4 * 32768 * iters flops; out: [256 * 512] floats (device),
 * overwritten.  Both only enqueue on `stream`. */
lh_status lh_peak_hbm(int mode, void* dst, const void* src, size_t bytes, void* stream);
lh_status lh_peak_mfma(float* out, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIGHTHOUSE_H */
