// Internal declarations shared by the HIP translation units of libwoq.
// Device-side descriptor tables live in the caller's workspace; the host
// fills them, copies them in with one hipMemcpyAsync per call, and the
// kernels map their block index to a matrix by binary search over
// per-matrix unit offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "woq.h"

namespace woq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- helpers
// Loads / stores through global (address space 1) pointers: the descriptor
// tables hold generic pointers, which would otherwise become flat accesses.
template <class T>
__device__ __forceinline__ T gload(const void* p) {
    typedef const __attribute__((address_space(1))) T* gptr;
    return *(gptr)(p);
}
template <class T>
__device__ __forceinline__ void gstore(void* p, T v) {
    typedef __attribute__((address_space(1))) T* gptr;
    *(gptr)(p) = v;
}
// 16- and 8-byte vector forms (HIP's uint4 / float4 wrappers do not bind to
// address-space-qualified pointers, native vector types do).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload_u4(const void* p) {
    const u32x4 v = gload<u32x4>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 gload_f4(const void* p) {
    const f32x4 v = gload<f32x4>(p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 gload_f2(const void* p) {
    const f32x2 v = gload<f32x2>(p);
    return make_float2(v.x, v.y);
}
__device__ __forceinline__ void gstore_f4(void* p, float a, float b, float c, float d) {
    f32x4 v;
    v.x = a; v.y = b; v.z = c; v.w = d;
    gstore<f32x4>(p, v);
}

// Cross-lane exchanges on VALU (no LDS round trip): gfx950 permlane swaps
// exchange 32- and 16-lane halves; DPP handles partners within a row.
__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppMirror8 = 0x141;     // row_half_mirror: lane i <-> 7 - i in each 8
constexpr int kDppMirror16 = 0x140;    // row_mirror: lane i <-> 15 - i in each 16
constexpr int kDppXor8 = 0x128;        // row_ror:8 within 16-lane rows
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Butterfly reductions over a full wave.  Every lane ends with the same
// value (IEEE addition is commutative, so partners compute identical sums),
// and the combination order is fixed, so results are deterministic.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Largest m in [0, n) with begin[m] <= u (begin ascending, n + 1 entries,
// begin[0] <= u < begin[n]).
__device__ __forceinline__ int find_unit_owner(const int64_t* begin, int n, int64_t u) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (begin[mid] <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------ descriptors
// Entropy: one entry per matrix.  An fp32 contiguous matrix (ld == cols) is
// read in work units of `chunk` consecutive elements; a strided one in units
// of rpu whole rows.  bf16 matrices are read as 16-byte vectors shared out
// evenly over the counting pass.
struct EntMat {
    const void* data;
    int64_t n;          // rows * cols
    int64_t cols;
    int64_t ld;         // row stride (elements)
    int32_t dtype;
    int32_t slot;       // index of this matrix in the caller's h_mat
    int32_t rows;
    int32_t rpu;        // rows per work unit when strided (0: contiguous)
    int64_t chunk;      // elements per work unit when contiguous (a multiple of 8)
};

// Sinkhorn: one entry per matrix.  A matrix is cut into row strips, one
// workgroup per strip; each strip writes its column partial sums to part.
struct SinqMat {
    const void* data;
    float* s;           // caller's row scales [rows]
    float* t;           // caller's column scales [cols]
    float* u;           // workspace 1/t [cols]
    void* part;         // workspace column partials [n_strips][cols] (float2 / float4)
    int32_t rows, cols;
    int32_t ld;         // row stride of data (elements)
    int32_t dtype;
    int32_t n_strips;
    int32_t strip_rows;
    int32_t rms;        // 1: root mean square in place of the centred std
    int32_t pad;
};

// Quantise / dequantise / ternary: one entry per matrix.
struct QMat {
    const void* data;   // input weights (quant, ternary) or output (dequant)
    uint8_t* codes;
    float* scales;      // delta per group (or beta per row)
    uint8_t* zeros;
    const float* rs;    // 1/s (quant) or s (dequant), NULL = 1
    const float* ct;    // 1/t (quant) or t (dequant), NULL = 1
    int32_t rows, cols;
    int32_t ld;         // row stride of data (elements); codes stay contiguous
    int32_t dtype;
    int32_t group;      // group size for this matrix (cols for per-row groups)
    int32_t pad;
};

// Non-uniform code book (code-book grid): up to kCbMax ascending levels,
// their fp32 midpoints (+inf from the last midpoint on) and a table of
// kCbCells cells of width 2 / kCbCells over [-1, 1].  For y whose true cell
// floor((y + 1) * kCbCells / 2) is c or a neighbour, at least lo[c]
// midpoints lie below y and at most lo[c] + steps do, steps being the
// largest such spread over all cells.  One byte per cell keeps the whole
// table in 32 LDS dwords, one per bank, so random lookups do not conflict.
constexpr int kCbCells = 128;
constexpr int kCbMax = 16;
struct CbTable {
    float mid[kCbMax];
    float level[kCbMax];
    uint8_t lo[kCbCells];
};
static_assert(sizeof(CbTable) % 4 == 0, "copied as dwords");

// Lossless exponent code (DF11): one entry per matrix.
constexpr int kDf11Chunk = 8192;   // weights per encoding work unit
constexpr int kDf11MaxLen = 32;    // longest codeword (bits)
constexpr int kDf11PtrMin = 240;   // table entries >= this are sub-table pointers
constexpr int kDf11MaxSub = 16;    // sub-tables (pointer values 255 .. 240)
constexpr int kDf11BlockSegs = 256;  // decoding threads (64-bit segments) per block
struct DfMat {
    const uint16_t* src;     // encode: bf16 weights
    uint16_t* dst;           // decode: bf16 weights (written)
    uint8_t* enc;            // EncodedExponent
    uint8_t* sm;             // PackedSignMantissa
    uint8_t* gaps;           // Gaps (5 bits per segment)
    uint32_t* bpos;          // output position of each decoding block's first weight
    const uint8_t* tables;   // decode: n_tables x 256 table bytes
    const uint8_t* lens;     // decode: CodeLengths [256]
    int64_t n;               // weights
    int64_t total_bits;
    int64_t n_seg;
    int64_t n_blocks;
    int64_t enc_bytes;
    int64_t gap_bytes;
    int32_t n_tables;
    int32_t pad;
};
// Encode: the matrix's code (codewords right-aligned, lengths 0 = unused).
struct DfCode {
    uint32_t code[256];
    uint8_t len[256];
};

}  // namespace woq
