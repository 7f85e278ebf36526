// The Q, K, V projections of the attention layer and their gradients, on the
// gfx950 matrix cores.  Page "skillsmp.com ... lighthouse-attention": the
// four-stage pipeline starts from the Q, K, V projections of the layer input X,
// the complexity table lists them as a GEMM of Theta(N d_model d), and the
// gradient-flow figure ends in W_Q, W_K, W_V (selection carries no gradient).
//
//   forward   [Q K V] = X W^T              X [B,N,Dm] row-major, W [3Hd, Dm] row-major
//                                          (rows: the H*d Q features, then K, then V)
//   backward  dX = [dQ dK dV] W            [B,N,Dm]
//             dW = [dQ dK dV]^T X          [3Hd, Dm], summed over all B*N tokens, f32
//
// Q, K, V and their gradients are head-major [B,H,N,d], the layout of the
// layer's inputs.  One GEMM kernel computes C = A B^T.  Its operands are
// either k-contiguous (every matrix-core fragment a 16-byte run of one
// LDS-staged row) or, for dW, whose k runs over the tokens, k-major: X and
// [dQ dK dV] are staged as they lie and read across their rows with the LDS
// transpose load.  The dX product takes W^T, made by a (6 MB) transpose.  The
// output goes through LDS so that it leaves the block as 16-byte stores.
#include "lh_device.h"
#include "lh_internal.h"

namespace {

// Block tile 256 x 256 (8 waves, each 128 rows x 64 columns of C), k in
// stages of 64 double-buffered in LDS: each stage is 32 matrix products per
// wave, enough to cover the next stage's global-to-LDS load.
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWM = 2, kWN = 4;                    // waves along m and n
constexpr int kGWaves = kWM * kWN, kGThreads = 64 * kGWaves;
constexpr int kTM = kBM / kWM, kTN = kBN / kWN;    // one wave's block of C
constexpr int kTileBytes = kBM * kBK * 2;          // one operand tile (bf16, 128-byte rows); kBM == kBN
constexpr int kCRows = 64, kCLd = kBN + 8;         // C leaves through LDS 64 rows at a time; the
                                                   // pitch puts lane halves (4 rows apart) on disjoint banks
constexpr int kGemmLds = (2 * 2 * kTileBytes > kCRows * kCLd * 4) ? 2 * 2 * kTileBytes : kCRows * kCLd * 4;
static_assert(kBM == kBN, "one tile size for both operands");

// Operands.  Each stages the k-block kb of its 256 output rows base .. base+255
// into one 32 KB LDS tile (stage) and says how the kernel reads fragments of
// it (kKMajor).  k-contiguous operands store the tile as 256 rows of 64 k
// (128-byte rows); k-major ones -- whose global rows run along k -- as four
// sub-tiles of 64 k-rows x 64 output rows, read across their rows by the
// transpose load.  Rows past the operand's end repeat its last row (or
// 64-row block); the epilogue drops them.
constexpr int kSubBytes = kBK * 64 * 2;   // one 64 x 64 bf16 sub-tile
static_assert(4 * kSubBytes == kTileBytes, "four sub-tiles per operand tile");

// k-contiguous rows: row r of k-block kb at kblock(kb) + r * row_bytes.
template <class Self>
struct KContiguous {
    static constexpr bool kKMajor = false;
    __device__ void stage(unsigned char* buf, int kb, uint32_t base) const {
        const Self& o = *static_cast<const Self*>(this);
        const uint32_t last = (uint32_t)(o.rows - 1), rb = o.row_bytes();
        stage_tile<128, kTileBytes, kGWaves>(buf, o.kblock(kb), [&](int r) {
            const uint32_t row = base + r < last ? base + r : last;
            return row * rb;
        });
    }
};
struct RowMajorOp : KContiguous<RowMajorOp> {
    const bf16* p;
    int64_t ld;      // elements between rows
    int64_t rows;    // valid rows
    RowMajorOp(const bf16* p_, int64_t ld_, int64_t rows_) : p(p_), ld(ld_), rows(rows_) {}
    __device__ uint32_t row_bytes() const { return (uint32_t)(ld * 2); }
    __device__ const unsigned char* kblock(int kb) const {
        return reinterpret_cast<const unsigned char*>(p + (int64_t)kb * kBK);
    }
};
// [dQ dK dV] of one batch as rows = tokens, k = feature (which, h, dd): k-block
// kb covers 64 features of one head.  32-bit index math: the source is picked
// by comparisons, the head and the offset inside it by shifts (d = 64 or 128).
struct HeadMajorOp : KContiguous<HeadMajorOp> {
    const bf16 *x0, *x1, *x2;        // this batch's [H, N, d] slabs
    int kb_per_src;                   // H * d / 64
    int head_shift;                   // log2(d / 64)
    uint32_t head_stride;             // N * d elements
    uint32_t rbytes;                  // d * 2
    int64_t rows;
    HeadMajorOp(const bf16* a, const bf16* b, const bf16* c, int kps, int hs, uint32_t hst, uint32_t rb, int64_t r)
        : x0(a), x1(b), x2(c), kb_per_src(kps), head_shift(hs), head_stride(hst), rbytes(rb), rows(r) {}
    __device__ uint32_t row_bytes() const { return rbytes; }
    __device__ const unsigned char* kblock(int kb) const {
        const int which = (kb >= kb_per_src) + (kb >= 2 * kb_per_src);
        const int r = kb - which * kb_per_src;
        const uint32_t h = (uint32_t)r >> head_shift, dd = ((uint32_t)r & ((1u << head_shift) - 1)) * 64;
        const bf16* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
        return reinterpret_cast<const unsigned char*>(x + (h * head_stride + dd));
    }
};
// k-major: a row-major [K x cols] array (rows run along k), output row = column.
struct KMajorOp {
    static constexpr bool kKMajor = true;
    const bf16* p;
    int64_t ld;      // elements between k-rows
    int cols;        // valid columns (a multiple of 64)
    __device__ void stage(unsigned char* buf, int kb, uint32_t base) const {
        const bf16* k0 = p + (int64_t)kb * kBK * ld;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = (int)base + 64 * j < cols ? (int)base + 64 * j : cols - 64;
            stage_tile<128, kSubBytes, kGWaves>(buf + j * kSubBytes, k0 + c0,
                                                [&](int r) { return (uint32_t)(r * ld * 2); });
        }
    }
};
// k-major [dQ dK dV]: k = tokens (all B*N of them), output row = feature
// (which, h, dd); a 64-token k-block lies in one batch (N is a multiple of 64).
struct HeadKMajorOp {
    static constexpr bool kKMajor = true;
    const bf16 *x0, *x1, *x2;   // [B, H, N, d]
    int Hd, log2d, H;
    uint32_t kb_per_batch;      // N / 64
    uint32_t N;
    __device__ void stage(unsigned char* buf, int kb, uint32_t base) const {
        const uint32_t b = (uint32_t)kb / kb_per_batch, n0 = ((uint32_t)kb - b * kb_per_batch) * kBK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f0 = (int)base + 64 * j < 3 * Hd ? (int)base + 64 * j : 3 * Hd - 64;
            const int which = (f0 >= Hd) + (f0 >= 2 * Hd);
            const uint32_t f = (uint32_t)(f0 - which * Hd), h = f >> log2d, dd = f & ((1u << log2d) - 1);
            const bf16* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
            const bf16* src = x + ((int64_t)(b * (uint32_t)H + h) * N + n0) * (1 << log2d) + dd;
            stage_tile<128, kSubBytes, kGWaves>(buf + j * kSubBytes, src,
                                                [&](int r) { return (uint32_t)r << (log2d + 1); });
        }
    }
};

// Epilogues: where 8 consecutive output columns n .. n+7 of row m go.
struct QkvOut {                 // rows = tokens b*N + t, columns = features -> q/k/v [B,H,N,d]
    bf16 *x0, *x1, *x2;
    int Hd, log2d;                // H * d, log2(d)
    uint32_t N;
    __device__ bf16* at(int64_t m, int64_t n) const {
        const int nn = (int)n;
        const int which = (nn >= Hd) + (nn >= 2 * Hd);
        const uint32_t f = (uint32_t)(nn - which * Hd);               // h * d + dd
        const uint32_t b = (uint32_t)m / N, t = (uint32_t)m - b * N;
        bf16* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
        // element offset ((b*H + h)*N + t)*d + dd < 2^31 (one of q, k, v)
        const uint32_t d = 1u << log2d, h = f >> log2d, dd = f & (d - 1);
        return x + (((b * (uint32_t)(Hd >> log2d) + h) * N + t) << log2d) + dd;
    }
};
template <typename OutT>
struct RowMajorOut {            // split z of a split-k product writes its own copy at p + z * zstride
    OutT* p;
    int64_t ld, zstride;
    __device__ OutT* at(int64_t m, int64_t n) const { return p + blockIdx.z * zstride + m * ld + n; }
};

template <typename OutT> __device__ __forceinline__ void store8(OutT* dst, const float* v);
template <> __device__ __forceinline__ void store8<bf16>(bf16* dst, const float* v) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(v[e]);
    *reinterpret_cast<bf16x8*>(dst) = r;
}
template <> __device__ __forceinline__ void store8<float>(float* dst, const float* v) {
    *reinterpret_cast<floatx4*>(dst) = floatx4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4*>(dst + 4) = floatx4{v[4], v[5], v[6], v[7]};
}

// C[M x Nc] = A[M x K] B[Nc x K]^T over the k-blocks of this block's split
// (blockIdx.z); f32 accumulation, one rounding to OutT.  Blocks are numbered
// so that each XCD (blocks are dealt to the 8 XCDs in turn) works on a
// contiguous range of C tiles.  With group_m > 0 (unsplit products whose row
// tiles divide into whole groups per XCD) the range is walked in groups of
// group_m row tiles, column by column: the ~32 blocks an XCD runs at once then
// cover group_m row tiles of A and a few column tiles of B, instead of ~3 row
// tiles and every column tile of B (W, 6 MB at d_model = 1024, more than the
// XCD's 4 MB L2).  Otherwise row tile by row tile.
template <class OpA, class OpB, class Epi, typename OutT>
__global__ __launch_bounds__(kGThreads, 1) void gemm_nt_kernel(OpA A, OpB B, Epi E, int64_t M, int64_t Nc,
                                                               int nkb, int kb_per_split, int tiles_n,
                                                               int tiles, int group_m) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 31, h = lane >> 5;
    const int wm = wave / kWN, wn = wave % kWN;
    int mt, nt;
    if (group_m > 0) {
        // each XCD takes tiles_m / 8 consecutive row tiles; inside, groups of group_m row
        // tiles are walked column-major, so the blocks running together share both operands
        const int tiles_m = tiles / tiles_n, rows_per_xcd = tiles_m / 8;
        const int xcd = (int)(blockIdx.x % 8), li = (int)(blockIdx.x / 8);
        const int g = li / (group_m * tiles_n), r = li - g * group_m * tiles_n;
        mt = xcd * rows_per_xcd + g * group_m + r % group_m;
        nt = r / group_m;
    } else {
        const int per_xcd = (tiles + 7) / 8;
        const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
        if (tile >= tiles) return;   // uniform per block
        mt = tile / tiles_n;
        nt = tile % tiles_n;
    }
    const int64_t m0 = (int64_t)mt * kBM, n0 = (int64_t)nt * kBN;
    const int kb0 = blockIdx.z * kb_per_split;
    const int kb1 = kb0 + kb_per_split < nkb ? kb0 + kb_per_split : nkb;

    static_assert(OpA::kKMajor == OpB::kKMajor, "both operands must present k in the same order");
    constexpr bool KM = OpA::kKMajor;
    auto stage = [&](int kb, unsigned char* buf) {
        A.stage(buf, kb, (uint32_t)m0);
        B.stage(buf + kTileBytes, kb, (uint32_t)n0);
    };

    constexpr int FI = kTM / 32, FJ = kTN / 32, NS = kBK / 16;
    floatx16 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = floatx16{};

    // Fragments are double-buffered in registers: the reads for k-substep s+1
    // are issued before the products of substep s, and those for substep 0 of
    // the next stage right after the barrier that makes it visible, so the
    // matrix cores never wait for a fresh LDS read at a stage boundary.
    bf16x8 fa[2][FI], fb[2][FJ];
    // fragment of tile rows r0 .. r0+31 (a multiple of 32) for k16 step s
    auto frag = [&](const unsigned char* t, int r0, int s) {
        if constexpr (KM) return tile_frag_tr<128>(t + (r0 >> 6) * kSubBytes, 16 * s, r0 & 32);
        else return tile_frag<bf16, 128>(t, r0 + col, 16 * s + 8 * h);
    };
    auto read_frags = [&](const unsigned char* t, int s, bf16x8* a, bf16x8* b) {
#pragma unroll
        for (int i = 0; i < FI; ++i) a[i] = frag(t, wm * kTM + 32 * i, s);
#pragma unroll
        for (int j = 0; j < FJ; ++j) b[j] = frag(t + kTileBytes, wn * kTN + 32 * j, s);
    };
    auto products = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) mma_k16(acc[i][j], a[i], b[j]);
    };
    auto buffer = [&](int kb) { return smem + ((kb - kb0) & 1) * 2 * kTileBytes; };
    // Scheduling pattern for one substep: one product, then the FI+FJ reads
    // for the next substep, then the remaining products.  With global-to-LDS
    // loads in flight the compiler can only wait for every outstanding LDS
    // read; that wait now falls before the first product, when the reads it
    // covers were issued a whole substep earlier.
    constexpr int READS = (KM ? 2 : 1) * (FI + FJ);   // a transpose-read fragment is two loads
    auto interleave = [] {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // matrix product
        __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);         // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, FI * FJ - 1, 0);   // matrix products
    };
    static_assert(NS % 2 == 0, "substeps alternate between the two fragment sets");

    // One k-stage.  On entry substep 0's fragments of stage kb are in flight
    // and stage kb+1 is being loaded into the other buffer.  LOAD2: stage kb+2
    // exists; NEXT: stage kb+1 exists.
    auto iteration = [&]<bool LOAD2, bool NEXT>(int kb) {
        const unsigned char* t = buffer(kb);
#pragma unroll
        for (int s = 0; s + 1 < NS; ++s) {
            read_frags(t, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            products(fa[s & 1], fb[s & 1]);
            interleave();
        }
        // stage kb+1 has landed and every wave holds its last fragments of stage kb
        wait_tiles_and_sync();
        if constexpr (LOAD2) stage(kb + 2, buffer(kb));
        if constexpr (NEXT) read_frags(buffer(kb + 1), 0, fa[0], fb[0]);
        products(fa[(NS - 1) & 1], fb[(NS - 1) & 1]);
        if constexpr (NEXT) interleave();
    };

    if (kb0 < kb1) stage(kb0, smem);
    wait_tiles_and_sync();
    if (kb0 + 1 < kb1) stage(kb0 + 1, buffer(kb0 + 1));
    if (kb0 < kb1) read_frags(smem, 0, fa[0], fb[0]);
    int kb = kb0;
    for (; kb + 2 < kb1; ++kb) iteration.template operator()<true, true>(kb);
    if (kb + 1 < kb1) iteration.template operator()<false, true>(kb++);
    if (kb < kb1) iteration.template operator()<false, false>(kb);

    // C leaves through LDS, kCRows rows at a time, as 8-column chunks
    float* ct = reinterpret_cast<float*>(smem);
    static_assert(kTM % kCRows == 0 && kCRows % 32 == 0, "whole row tiles per pass");
#pragma unroll
    for (int pass = 0; pass < kBM / kCRows; ++pass) {
        const int r0 = pass * kCRows;
        if (wm * kTM <= r0 && r0 < (wm + 1) * kTM) {   // this wave's rows
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int row_base = wm * kTM + 32 * i - r0;
                if (row_base < 0 || row_base >= kCRows) continue;
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ct[(row_base + c_row(r, h)) * kCLd + wn * kTN + 32 * j + col] = acc[i][j][r];
            }
        }
        __syncthreads();
        for (int task = threadIdx.x; task < kCRows * (kBN / 8); task += kGThreads) {
            const int r = task / (kBN / 8), c = task - r * (kBN / 8);
            const int64_t m = m0 + r0 + r, n = n0 + 8 * c;
            if (m < M && n < Nc) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = ct[r * kCLd + 8 * c + e];
                store8<OutT>(E.at(m, n), v);
            }
        }
        __syncthreads();
    }
}

// out[c][r] = in[r][c] for an R x C bf16 block of rows (row stride ld_in),
// written with row stride ld_out; blockIdx.z selects one of up to three
// sources and a slab of it (src + z_in * slab_in, dst + z_out * slab_out).
struct TransposeSlabs {
    const bf16 *s0, *s1, *s2;
    bf16* dst;
    int64_t R, C, ld_in, ld_out;
    int per_src;                        // slabs per source
    int64_t slab_in, slab_out_src, slab_out;   // element offsets
};

__global__ __launch_bounds__(256) void transpose_slabs_kernel(TransposeSlabs T) {
    __shared__ bf16 tile[64][64 + 8];
    const int src = blockIdx.z / T.per_src, slab = blockIdx.z - src * T.per_src;
    const bf16* in = (src == 0 ? T.s0 : (src == 1 ? T.s1 : T.s2)) + (int64_t)slab * T.slab_in;
    bf16* out = T.dst + (int64_t)src * T.slab_out_src + (int64_t)slab * T.slab_out;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    for (int task = threadIdx.x; task < 64 * 8; task += 256) {   // 64 rows x 8 chunks of 8
        const int r = task >> 3, ch = task & 7;
        bf16x8 v = {};
        if (r0 + r < T.R && c0 + 8 * ch < T.C) v = *reinterpret_cast<const bf16x8*>(in + (r0 + r) * T.ld_in + c0 + 8 * ch);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[r][8 * ch + e] = v[e];
    }
    __syncthreads();
    for (int task = threadIdx.x; task < 64 * 8; task += 256) {
        const int c = task >> 3, ch = task & 7;
        if (c0 + c >= T.C || r0 + 8 * ch >= T.R) continue;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[8 * ch + e][c];
        *reinterpret_cast<bf16x8*>(out + (c0 + c) * T.ld_out + r0 + 8 * ch) = v;
    }
}

// dW = sum of the split partials, in split order (deterministic).
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                            int64_t n, int splits) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    floatx4 a = *reinterpret_cast<const floatx4*>(part + i);
    for (int s = 1; s < splits; ++s) a += *reinterpret_cast<const floatx4*>(part + (int64_t)s * n + i);
    *reinterpret_cast<floatx4*>(out + i) = a;
}

template <class OpA, class OpB, class Epi, typename OutT>
hipError_t gemm_nt(const OpA& A, const OpB& B, const Epi& E, int64_t M, int64_t Nc, int64_t K, int splits,
                   hipStream_t st) {
    const int nkb = (int)(K / kBK);
    const int per = (nkb + splits - 1) / splits;
    const int tiles_n = (int)((Nc + kBN - 1) / kBN), tiles = tiles_n * (int)((M + kBM - 1) / kBM);
    auto kern = gemm_nt_kernel<OpA, OpB, Epi, OutT>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)attr;
    const int tiles_m = tiles / tiles_n;
    const int group_m = (splits == 1 && tiles_m % 64 == 0) ? 8 : 0;   // whole groups of 8 row tiles per XCD
    // (a split-k product has too few row tiles to spread over the XCDs this way)
    dim3 grid((unsigned)((tiles + 7) / 8 * 8), 1, (unsigned)splits);
    kern<<<grid, kGThreads, kGemmLds, st>>>(A, B, E, M, Nc, nkb, per, tiles_n, tiles, group_m);
    return hipGetLastError();
}

hipError_t transpose(const TransposeSlabs& T, int nz, hipStream_t st) {
    dim3 grid((unsigned)((T.C + 63) / 64), (unsigned)((T.R + 63) / 64), (unsigned)nz);
    transpose_slabs_kernel<<<grid, 256, 0, st>>>(T);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_forward(const ProjGeom& g, const void* x, const void* w, void* q, void* k, void* v,
                              hipStream_t st) {
    const int64_t M = g.B * g.N, Nc = 3 * g.H * g.d;
    RowMajorOp A{(const bf16*)x, g.Dm, M};
    RowMajorOp B{(const bf16*)w, g.Dm, Nc};
    QkvOut E{(bf16*)q, (bf16*)k, (bf16*)v, (int)(g.H * g.d), g.d == 64 ? 6 : 7, (uint32_t)g.N};
    return gemm_nt<RowMajorOp, RowMajorOp, QkvOut, bf16>(A, B, E, M, Nc, g.Dm, 1, st);
}

hipError_t launch_qkv_backward(const ProjGeom& g, const void* x, const void* w, const void* dq, const void* dk,
                               const void* dv, void* dx, float* dw, void* ws, hipStream_t st) {
    const int64_t M = g.B * g.N, Nc = 3 * g.H * g.d, Dm = g.Dm;
    unsigned char* p = (unsigned char*)ws;
    bf16* wT = (bf16*)(p + g.ws_wT);      // [Dm x Nc]
    float* part = (float*)(p + g.ws_part);   // [splits][Nc x Dm]
    hipError_t e = transpose(TransposeSlabs{(const bf16*)w, nullptr, nullptr, wT, Nc, Dm, Dm, Nc, 1, 0, 0, 0}, 1, st);
    // dX = [dQ dK dV] W, per batch (rows: the batch's tokens)
    for (int64_t b = 0; b < g.B && e == hipSuccess; ++b) {
        const int64_t boff = b * g.H * g.N * g.d;
        HeadMajorOp A{(const bf16*)dq + boff, (const bf16*)dk + boff, (const bf16*)dv + boff,
                      (int)(g.H * g.d / 64), g.d == 64 ? 0 : 1, (uint32_t)(g.N * g.d), (uint32_t)(g.d * 2), g.N};
        RowMajorOp B{wT, Nc, Dm};
        RowMajorOut<bf16> E{(bf16*)dx + b * g.N * Dm, Dm, 0};
        e = gemm_nt<HeadMajorOp, RowMajorOp, RowMajorOut<bf16>, bf16>(A, B, E, g.N, Dm, Nc, 1, st);
    }
    // dW = [dQ dK dV]^T X over all tokens: both operands are read k-major (rows
    // along the tokens), split over k, partials summed in order
    if (e == hipSuccess) {
        HeadKMajorOp A{(const bf16*)dq, (const bf16*)dk, (const bf16*)dv, (int)(g.H * g.d), g.d == 64 ? 6 : 7,
                       (int)g.H, (uint32_t)(g.N / kBK), (uint32_t)g.N};
        KMajorOp B{(const bf16*)x, Dm, (int)Dm};
        RowMajorOut<float> E{g.splits > 1 ? part : dw, Dm, Nc * Dm};
        e = gemm_nt<HeadKMajorOp, KMajorOp, RowMajorOut<float>, float>(A, B, E, Nc, Dm, M, g.splits, st);
    }
    if (e == hipSuccess && g.splits > 1) {
        const int64_t n = Nc * Dm;
        reduce_splits_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(part, dw, n, g.splits);
        e = hipGetLastError();
    }
    return e;
}
