// Device-side building blocks for the Lighthouse kernels on gfx950 (CDNA4).
//
// Matrix-core conventions (checked on the device: lane layouts of
// v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32):
//   A operand (32 x 16 slice of a row-major A): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B operand (16 x 32):                        lane l holds B[8*(l/32) + e][l % 32]
//   C/D (32 x 32, 16 floats per lane):          reg j holds C[8*(j/4) + 4*(l/32) + (j%4)][l % 32]
// A "k16 step" contracts 16 k-indices: one bf16 MFMA, or eight f32 MFMAs (f32
// step j contracts the two k-indices {j, 8 + j} of the same fragments).
//
// Because the k-index order of one step is free, a C tile produced by one MFMA
// can be fed back as the B operand of the next without moving data between
// lanes: rows 16c + {4h..4h+3, 8+4h..8+4h+3} of the C tile (c = 0, 1; h = l/32)
// are exactly registers 8c..8c+7 of lane l, so the matching A operand reads
// those same k-indices (two runs of four) -- see a_frag_perm().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct Frag<float> { typedef floatx8 type; typedef floatx4 half; };

__device__ __forceinline__ void mma_k16(floatx16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k16(floatx16& acc, const floatx8& a, const floatx8& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
}

// Eight consecutive elements (16 B for bf16, 32 B for f32).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load8(const T* p) {
    return *reinterpret_cast<const typename Frag<T>::type*>(p);
}
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load8_or_zero(const T* p, bool ok) {
    typename Frag<T>::type z = {};
    return ok ? *reinterpret_cast<const typename Frag<T>::type*>(p) : z;
}
// Two runs of four consecutive elements at p and p + 8 (the permuted k order).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_4_4(const T* p) {
    typedef typename Frag<T>::half H;
    H lo = *reinterpret_cast<const H*>(p);
    H hi = *reinterpret_cast<const H*>(p + 8);
    typename Frag<T>::type r;
    r.lo = lo;
    r.hi = hi;
    return r;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Registers 8c .. 8c+7 of a C tile as a B-operand fragment of type T
// (bf16: four paired round-to-nearest-even conversions).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type c_to_frag(const floatx16& c, int cc);
template <>
__device__ __forceinline__ bf16x8 c_to_frag<bf16>(const floatx16& c, int cc) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2 h = __builtin_convertvector((floatx2){c[8 * cc + 2 * e], c[8 * cc + 2 * e + 1]}, bf16x2);
        r[2 * e] = h[0];
        r[2 * e + 1] = h[1];
    }
    return r;
}
template <>
__device__ __forceinline__ floatx8 c_to_frag<float>(const floatx16& c, int cc) {
    floatx8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = c[8 * cc + e];
    return r;
}

// Registers 8c .. 8c+7 as hi + lo bf16 fragments: hi = RNE(x), lo = RNE(x - hi).
// x - hi is exact in f32 and comes from one dot2 against (-1, 0) or (0, -1),
// so the split costs two VALU operations per element.  For f32 the fragment
// is exact and lo is unused.
template <typename T>
__device__ __forceinline__ void split_frag(const floatx16& c, int cc, typename Frag<T>::type& hi,
                                          typename Frag<T>::type& lo);
template <>
__device__ __forceinline__ void split_frag<bf16>(const floatx16& c, int cc, bf16x8& hi, bf16x8& lo) {
    // (-1, -0) rather than (-1, 0): the compiler turns the pair (-1, 0) into the
    // inline constant -1.0, which the hardware reads as the f32 bit pattern,
    // i.e. the pair (0, -1).  -0 keeps it a literal and adds nothing.
    const bf16x2 sel0 = {(bf16)-1.0f, (bf16)-0.0f}, sel1 = {(bf16)0.0f, (bf16)-1.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x0 = c[8 * cc + 2 * e], x1 = c[8 * cc + 2 * e + 1];
        const bf16x2 h = __builtin_convertvector((floatx2){x0, x1}, bf16x2);
        const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, sel0, x0, false);
        const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, sel1, x1, false);
        const bf16x2 l = __builtin_convertvector((floatx2){r0, r1}, bf16x2);
        hi[2 * e] = h[0];
        hi[2 * e + 1] = h[1];
        lo[2 * e] = l[0];
        lo[2 * e + 1] = l[1];
    }
}
template <>
__device__ __forceinline__ void split_frag<float>(const floatx16& c, int cc, floatx8& hi, floatx8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) hi[e] = c[8 * cc + e];
    lo = hi;
}

// The same split with x - hi from a shift or mask of the packed pair and a
// subtraction (bit-identical results): plain vector operations, which the
// hardware issues alongside matrix products, where the dot2 form is not.
template <typename T>
__device__ __forceinline__ void split_frag_vec(const floatx16& c, int cc, typename Frag<T>::type& hi,
                                               typename Frag<T>::type& lo) {
    split_frag<T>(c, cc, hi, lo);
}
template <>
__device__ __forceinline__ void split_frag_vec<bf16>(const floatx16& c, int cc, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x0 = c[8 * cc + 2 * e], x1 = c[8 * cc + 2 * e + 1];
        const bf16x2 h = __builtin_convertvector((floatx2){x0, x1}, bf16x2);
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float r0 = x0 - __uint_as_float(hb << 16), r1 = x1 - __uint_as_float(hb & 0xffff0000u);
        const bf16x2 l = __builtin_convertvector((floatx2){r0, r1}, bf16x2);
        hi[2 * e] = h[0];
        hi[2 * e + 1] = h[1];
        lo[2 * e] = l[0];
        lo[2 * e + 1] = l[1];
    }
}

// max over the 16 registers of a C tile (eight 3-input maxima)
__device__ __forceinline__ float max16(const floatx16& v) {
    float m = __builtin_fmaxf(v[0], v[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, v[j]), v[j + 1]);
    return m;
}

// Row (within a 32-row C tile) held by register j of lane-half h.
__device__ __forceinline__ int c_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ float to_f(T x) { return static_cast<float>(x); }

// Wave-wide helpers (wave64).  v_permlane32_swap exchanges the two 32-lane
// halves, so combining its two results gives the reduction over lanes l and
// l ^ 32 in every lane with one cross-lane instruction.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Placed first in the body of a rarely taken uniform branch: an empty volatile
// asm cannot be executed speculatively, so the compiler keeps the branch
// instead of turning its body into selects that run on every pass.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Wave index as a uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Row offset (within a 32-row C tile) of register j, without the 4*(l/32) term.
__device__ __forceinline__ constexpr int c_row0(int j) { return 8 * (j >> 2) + (j & 3); }

// Sixteen bytes of T.
template <typename T> struct V16;
template <> struct V16<bf16> { typedef bf16x8 type; enum { N = 8 }; };
template <> struct V16<float> { typedef floatx4 type; enum { N = 4 }; };

// ---------------------------------------------------------------------------
// LDS tiles.  A tile is ROWS rows of ROWB bytes, filled straight from global
// memory by global_load_lds (16 bytes per lane, 1 KB per wave instruction, no
// staging registers).  16-byte chunk c of row r sits at chunk c ^ f(r) of that
// row.  f is a bijection on every aligned group of 8 (128-byte rows) or 16
// (256-byte rows) rows, so lanes reading the same chunk of consecutive rows
// hit distinct bank groups; it also sends 4 consecutive rows (128-byte rows:
// rows r and r+2, which share banks) to disjoint sets of 4-chunk runs, so the
// transpose loads of tile_frag_tr, which read 64 bytes of each of 4
// consecutive rows, are conflict-free too:
//   128-byte rows: f(r) = perm(r & 7) ^ ((r >> 3) & 7), perm swapping bits 1, 2
//   256-byte rows: f(r) = ((r & 3) << 2) | ((r >> 2) & 3)
// The attention kernels' row tiles hold 64 (or 32) rows of a row-major
// [S][D] array (rows past S repeat row S-1; masks give them zero weight).  In
// bf16 the products that contract over the sequence read those same row tiles
// with tile_frag_tr; the f32 kernels instead take column tiles: D rows of a
// transposed [D][S_pad] array, in the slot order store_transposed writes, so
// that lane half h finds the keys of its k-step as one run.  The projection
// GEMMs stage k-contiguous row tiles of both operands the same way.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <int ROWB>
__device__ __forceinline__ int swz_key(int row) {
    static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "row tiles of 64, 128 or 256 bytes");
    if (ROWB == 64) return ((row >> 1) ^ (row >> 3)) & 3;
    if (ROWB == 128) return ((row & 1) | ((row & 2) << 1) | ((row >> 1) & 2)) ^ ((row >> 3) & 7);
    return ((row & 3) << 2) | ((row >> 2) & 3);
}
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ swz_key<ROWB>(row)) << 4); }

// Loads one tile: chunk (wave * PER + i) * 64 + lane of the tile (byte
// position pos, tile row r = pos / ROWB) receives global 16-byte chunk
// (pos % ROWB) / 16 ^ f(r) of row r, found at base + row_off(r).  row_off
// returns a 32-bit byte offset and base is uniform, so the per-lane address is
// a single 32-bit value.
template <int ROWB, int BYTES, int NW, class RowOff>
__device__ __forceinline__ void stage_tile(unsigned char* tile, const void* base, RowOff row_off) {
    static_assert(BYTES % (1024 * NW) == 0, "tile must split into 1 KB wave instructions");
    constexpr int PER_WAVE = BYTES / (1024 * NW);
    const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int dst = (wave * PER_WAVE + i) * 1024;
        const int pos = dst + 16 * lane;
        const int row = pos / ROWB;
        const uint32_t chunk = (uint32_t)(((pos % ROWB) >> 4) ^ swz_key<ROWB>(row));
        const unsigned char* g = reinterpret_cast<const unsigned char*>(base) + (row_off(row) + (chunk << 4));
        __builtin_amdgcn_global_load_lds(g, (lds_void*)(tile + dst), 16, 0, 0);
    }
}

// 8 elements of T starting at element e0 (a multiple of 8) of a tile row.
template <typename T, int ROWB>
__device__ __forceinline__ typename Frag<T>::type tile_frag(const unsigned char* tile, int row, int e0);
template <>
__device__ __forceinline__ bf16x8 tile_frag<bf16, 64>(const unsigned char* tile, int row, int e0) {
    return *reinterpret_cast<const bf16x8*>(tile + swz<64>(row, e0 >> 3));
}
template <>
__device__ __forceinline__ bf16x8 tile_frag<bf16, 128>(const unsigned char* tile, int row, int e0) {
    return *reinterpret_cast<const bf16x8*>(tile + swz<128>(row, e0 >> 3));
}
template <>
__device__ __forceinline__ bf16x8 tile_frag<bf16, 256>(const unsigned char* tile, int row, int e0) {
    return *reinterpret_cast<const bf16x8*>(tile + swz<256>(row, e0 >> 3));
}
// 8 bf16 of one column of a row-major bf16 tile read across its rows with the
// LDS transpose load: lane l gets column c0 + l % 32 of rows k0 + 4h + (0..3)
// and k0 + 8 + 4h + (0..3), h = l / 32 -- the order in which the C tile of a
// 32x32 product holds its rows, so a score tile can be the other operand of
// a product that contracts over those rows without moving data between lanes.
// (The transpose load gives lane j of each group of 16 lanes element j % 4 of
// the 4-element runs addressed by lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12 of
// its group; each lane below addresses the run its readers need.)
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
template <int ROWB>
__device__ __forceinline__ bf16x8 tile_frag_tr(const unsigned char* tile, int k0, int c0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, s = lane & 15;
    const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
    const int row = k0 + 4 * (g >> 1) + (s >> 2);
    const int within = (col & 4) * 2;   // byte offset of the 4-element run inside its 16-byte chunk
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + swz<ROWB>(row, col >> 3) + within));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + swz<ROWB>(row + 8, col >> 3) + within));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, r);
}

template <int ROWB>
__device__ __forceinline__ floatx8 tile_frag_f32(const unsigned char* tile, int row, int e0) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(tile + swz<ROWB>(row, e0 >> 2));
    const floatx4 b = *reinterpret_cast<const floatx4*>(tile + swz<ROWB>(row, (e0 >> 2) + 1));
    floatx8 r;
    r.lo = a;
    r.hi = b;
    return r;
}
template <>
__device__ __forceinline__ floatx8 tile_frag<float, 128>(const unsigned char* tile, int row, int e0) {
    return tile_frag_f32<128>(tile, row, e0);
}
template <>
__device__ __forceinline__ floatx8 tile_frag<float, 256>(const unsigned char* tile, int row, int e0) {
    return tile_frag_f32<256>(tile, row, e0);
}

__device__ __forceinline__ void wait_tiles_and_sync() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}
