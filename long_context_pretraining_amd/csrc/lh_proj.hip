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
// layer's inputs.  One GEMM kernel computes C = A B^T with both operands
// k-contiguous (A [M x K], B [Nc x K]), so every matrix-core fragment is a
// 16-byte run of one LDS-staged row; the backward builds the k-contiguous
// operands it needs (W^T, X^T, [dQ dK dV]^T) with transposes.  The output
// goes through LDS so that it leaves the block as 16-byte stores.
#include "lh_device.h"
#include "lh_internal.h"

namespace {

constexpr int kGThreads = 256;                 // 4 waves, each a 64 x 64 block of C
constexpr int kBM = 128, kBN = 128, kBK = 64;  // C tile, k per stage
constexpr int kTileBytes = kBM * kBK * 2;      // one operand tile (bf16, 128-byte rows)
constexpr int kCLd = kBN + 4;                  // f32 row stride of the staged C tile
constexpr int kGemmLds = (2 * 2 * kTileBytes > kBM * kCLd * 4) ? 2 * 2 * kTileBytes : kBM * kCLd * 4;

// Operand with k-contiguous rows: row r of k-block kb at kblock(kb) + r * row_bytes.
struct RowMajorOp {
    const bf16* p;
    int64_t ld;      // elements between rows
    int64_t rows;    // valid rows (later rows repeat the last one)
    __device__ const unsigned char* kblock(int kb) const {
        return reinterpret_cast<const unsigned char*>(p + (int64_t)kb * kBK);
    }
};
// [dQ dK dV] of one batch b as rows = tokens, k = feature (which, h, dd).
struct HeadMajorOp {
    const bf16 *x0, *x1, *x2;
    int64_t H, N, d, b;
    int64_t rows;
    __device__ const unsigned char* kblock(int kb) const {
        const int64_t f = (int64_t)kb * kBK;
        const int64_t which = f / (H * d), h = (f / d) % H, dd = f % d;
        const bf16* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
        return reinterpret_cast<const unsigned char*>(x + ((b * H + h) * N) * d + dd);
    }
};
template <class Op> __device__ __forceinline__ uint32_t op_row_bytes(const Op& o);
template <> __device__ __forceinline__ uint32_t op_row_bytes(const RowMajorOp& o) { return (uint32_t)(o.ld * 2); }
template <> __device__ __forceinline__ uint32_t op_row_bytes(const HeadMajorOp& o) { return (uint32_t)(o.d * 2); }

// Epilogues: where 8 consecutive output columns n .. n+7 of row m go.
struct QkvOut {                 // rows = tokens b*N + n, columns = features -> q/k/v [B,H,N,d]
    bf16 *x0, *x1, *x2;
    int64_t H, N, d;
    __device__ bf16* at(int64_t m, int64_t n) const {
        const int64_t which = n / (H * d), h = (n / d) % H, dd = n % d;
        const int64_t b = m / N, t = m - b * N;
        bf16* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
        return x + ((b * H + h) * N + t) * d + dd;
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

// C[M x Nc] (+)= A[M x K] B[Nc x K]^T for the k-blocks [kb0, kb1) of this
// block's split (blockIdx.z); f32 accumulation, one rounding to OutT.
template <class OpA, class OpB, class Epi, typename OutT>
__global__ __launch_bounds__(kGThreads, 2) void gemm_nt_kernel(OpA A, OpB B, Epi E, int64_t M, int64_t Nc,
                                                               int nkb, int kb_per_split) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 31, h = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
    const int kb0 = blockIdx.z * kb_per_split;
    const int kb1 = kb0 + kb_per_split < nkb ? kb0 + kb_per_split : nkb;

    const uint32_t a_rb = op_row_bytes(A), b_rb = op_row_bytes(B);
    const uint32_t a_last = (uint32_t)(A.rows - 1), b_last = (uint32_t)(B.rows - 1);
    auto stage = [&](int kb, unsigned char* buf) {
        stage_tile<128, kTileBytes, 4>(buf, A.kblock(kb), [&](int r) {
            const uint32_t row = (uint32_t)m0 + r < a_last ? (uint32_t)m0 + r : a_last;
            return row * a_rb;
        });
        stage_tile<128, kTileBytes, 4>(buf + kTileBytes, B.kblock(kb), [&](int r) {
            const uint32_t row = (uint32_t)n0 + r < b_last ? (uint32_t)n0 + r : b_last;
            return row * b_rb;
        });
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

    if (kb0 < kb1) stage(kb0, smem);
    wait_tiles_and_sync();
    for (int kb = kb0; kb < kb1; ++kb) {
        const int buf = (kb - kb0) & 1;
        if (kb + 1 < kb1) stage(kb + 1, smem + (buf ^ 1) * 2 * kTileBytes);
        const unsigned char* ta = smem + buf * 2 * kTileBytes;
        const unsigned char* tb = ta + kTileBytes;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) af[i] = tile_frag<bf16, 128>(ta, wm * 64 + 32 * i + col, 16 * s + 8 * h);
#pragma unroll
            for (int j = 0; j < 2; ++j) bfr[j] = tile_frag<bf16, 128>(tb, wn * 64 + 32 * j + col, 16 * s + 8 * h);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma_k16(acc[i][j], af[i], bfr[j]);
        }
        wait_tiles_and_sync();
    }

    // C tile through LDS, then 8-column chunks to global memory
    float* ct = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ct[(wm * 64 + 32 * i + c_row(r, h)) * kCLd + wn * 64 + 32 * j + col] = acc[i][j][r];
    __syncthreads();
    for (int task = threadIdx.x; task < kBM * (kBN / 8); task += kGThreads) {
        const int r = task / (kBN / 8), c = task - r * (kBN / 8);
        const int64_t m = m0 + r, n = n0 + 8 * c;
        if (m >= M || n >= Nc) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ct[r * kCLd + 8 * c + e];
        store8<OutT>(E.at(m, n), v);
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
    auto kern = gemm_nt_kernel<OpA, OpB, Epi, OutT>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)attr;
    dim3 grid((unsigned)((Nc + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM), (unsigned)splits);
    kern<<<grid, kGThreads, kGemmLds, st>>>(A, B, E, M, Nc, nkb, per);
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
    QkvOut E{(bf16*)q, (bf16*)k, (bf16*)v, g.H, g.N, g.d};
    return gemm_nt<RowMajorOp, RowMajorOp, QkvOut, bf16>(A, B, E, M, Nc, g.Dm, 1, st);
}

hipError_t launch_qkv_backward(const ProjGeom& g, const void* x, const void* w, const void* dq, const void* dk,
                               const void* dv, void* dx, float* dw, void* ws, hipStream_t st) {
    const int64_t M = g.B * g.N, Nc = 3 * g.H * g.d, Dm = g.Dm;
    unsigned char* p = (unsigned char*)ws;
    bf16* wT = (bf16*)(p + g.ws_wT);      // [Dm x Nc]
    bf16* xT = (bf16*)(p + g.ws_xT);      // [Dm x M]
    bf16* gT = (bf16*)(p + g.ws_gT);      // [Nc x M]
    float* part = (float*)(p + g.ws_part);   // [splits][Nc x Dm]
    hipError_t e = transpose(TransposeSlabs{(const bf16*)w, nullptr, nullptr, wT, Nc, Dm, Dm, Nc, 1, 0, 0, 0}, 1, st);
    // dX = [dQ dK dV] W, per batch (rows: the batch's tokens)
    for (int64_t b = 0; b < g.B && e == hipSuccess; ++b) {
        HeadMajorOp A{(const bf16*)dq, (const bf16*)dk, (const bf16*)dv, g.H, g.N, g.d, b, g.N};
        RowMajorOp B{wT, Nc, Dm};
        RowMajorOut<bf16> E{(bf16*)dx + b * g.N * Dm, Dm, 0};
        e = gemm_nt<HeadMajorOp, RowMajorOp, RowMajorOut<bf16>, bf16>(A, B, E, g.N, Dm, Nc, 1, st);
    }
    // X^T [Dm x M] and [dQ dK dV]^T [Nc x M]: every (source, b, h) slab [N x d] -> rows (src H + h) d.., cols b N..
    if (e == hipSuccess)
        e = transpose(TransposeSlabs{(const bf16*)x, nullptr, nullptr, xT, M, Dm, Dm, M, 1, 0, 0, 0}, 1, st);
    // per batch b: slab z = (source, h) is the [N x d] block of head h, which lands in rows
    // (source * H + h) * d .. and columns b * N .. of [dQ dK dV]^T
    for (int64_t b = 0; b < g.B && e == hipSuccess; ++b) {
        const int64_t off = b * g.H * g.N * g.d;
        TransposeSlabs T{(const bf16*)dq + off, (const bf16*)dk + off, (const bf16*)dv + off, gT + b * g.N,
                         g.N, g.d, g.d, M, (int)g.H, g.N * g.d, g.H * g.d * M, g.d * M};
        e = transpose(T, (int)(3 * g.H), st);
    }
    // dW = [dQ dK dV]^T X over all tokens, split over k, partials summed in order
    if (e == hipSuccess) {
        RowMajorOp A{gT, M, Nc};
        RowMajorOp B{xT, M, Dm};
        RowMajorOut<float> E{g.splits > 1 ? part : dw, Dm, Nc * Dm};
        e = gemm_nt<RowMajorOp, RowMajorOp, RowMajorOut<float>, float>(A, B, E, Nc, Dm, M, g.splits, st);
    }
    if (e == hipSuccess && g.splits > 1) {
        const int64_t n = Nc * Dm;
        reduce_splits_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(part, dw, n, g.splits);
        e = hipGetLastError();
    }
    return e;
}
