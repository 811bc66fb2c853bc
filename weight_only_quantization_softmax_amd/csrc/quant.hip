// Group-wise asymmetric round-to-nearest quantisation with LSB-first bit
// packing, its inverse, and ternary {-1, 0, +1} coding with a per-row scale.
//
// Low-bit integer storage of the balanced matrix: [SINQ] "Huawei gioi thieu
// SINQ" (asiadaily.org; 4-bit and, in some cases, 3-bit codes after the
// dual-axis scaling).  Groups are independent and need no communication:
// [BitNet] "Khung Nguon BitNet.cpp" (unite.ai), section "Luong Tu Hoa Nhom
// va Chuan Hoa".  Ternary weights: the same page, section "He Thong Trong So
// Ternary"; EWQ's 1.58-bit option for its lowest-entropy blocks.
//
// Every rounding decision is a fixed sequence of correctly rounded fp32
// operations (__fmul_rn, __fsub_rn, __fdiv_rn, rintf = round half to even),
// so codes, deltas and zero-points are reproducible bit for bit; ratios at or
// next to a half-way point are taken by a correctly rounded division, so
// exact half-way points round as the definition says (half to even).
//
// Work mapping:
//  k_quant_tile   groups of 8..512 columns (powers of two): a workgroup
//                 takes 8 rows x 2048 columns; each thread owns 8
//                 consecutive columns (one 16-byte bf16 load per row), a
//                 group is group/8 consecutive lanes reduced with DPP and
//                 permlane swaps.
//  k_quant_wave   groups of 513..4096 columns: one wave per group.
//  k_quant_big    wider groups (e.g. one group per 14336-column row): one
//                 workgroup per group, one LDS exchange.
//  k_dequant      tiles of kDTileRows rows x 2048 columns (measured on the
//                 8B stack's int4 matrices: 4 rows beat 8 and 16).
//  k_ternary_wave rows of up to 4096 columns: one wave per row, 16 rows
//                 per workgroup (the MoE experts' 1408- and 2048-column
//                 rows are 3-4 KB: a workgroup each left most of it idle).
//  k_ternary      wider rows: one workgroup per row.
//
// The tile, wave and big kernels and k_dequant also serve the code-book
// grid (template argument CB): a group is scaled by its largest |x| and each
// value takes the nearest of 2^b caller-given levels (the [SINQ] page's
// non-uniform option, same section as the low-bit codes).  The nearest level
// is the number of level midpoints below y, found from a 128-byte cell table
// in LDS and `steps` comparisons (one for the normal-quantile books).
#include "launch.h"

#include <math.h>

#include <type_traits>

namespace woq {
namespace {

constexpr int kT = 256;

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
    return fminf(fmaxf(v, lo), hi);
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* codes, uint32_t e0, const uint32_t (&c)[8]) {
    if constexpr (BITS == 8) {
        f32x2 w;  // 8 bytes as two raw 32-bit words
        w.x = __uint_as_float(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24));
        w.y = __uint_as_float(c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
        gstore<f32x2>(codes + e0, w);
    } else if constexpr (BITS == 4) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (4 * k);
        gstore<uint32_t>(codes + (e0 >> 1), w);
    } else if constexpr (BITS == 2) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (2 * k);
        gstore<uint16_t>(codes + (e0 >> 2), (uint16_t)w);
    } else {  // 3 bits: 8 codes fill exactly 3 bytes
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (3 * k);
        uint8_t* p = codes + (size_t)(e0 >> 3) * 3;
        gstore<uint8_t>(p, (uint8_t)w);
        gstore<uint8_t>(p + 1, (uint8_t)(w >> 8));
        gstore<uint8_t>(p + 2, (uint8_t)(w >> 16));
    }
}

struct GroupParams {
    float delta, inv, z, d;
    bool ok;
};

// A fast ratio v * inv (inv = 1/delta) lies within about 4 ulps of the
// exact ratio (2^b - 1) * v / d, d = hi - lo: within 6.1e-5 for |ratio| <=
// 255.  Its rounding can differ from the exact one only when it lies within
// that distance of a half-way point, so such ratios (|u - rne(u)| >
// kNearHalf, rare) are recomputed with one correctly rounded division, which
// for exact operands (inputs without scales) returns an exact half-way ratio
// as exactly k + 1/2, rounded half to even as the definition says.
constexpr float kNearHalf = 0.5f - 0x1p-13f;

__device__ __forceinline__ bool near_half(float u, float r) { return fabsf(__fsub_rn(u, r)) > kNearHalf; }

// Per group: d = hi - lo, delta = d / (2^b - 1), inv = 1 / delta, and the
// zero-point rne(-lo / delta) from the fast ratio -lo * inv, or from
// ((2^b - 1) * -lo) / d when that is near a half-way point (the same
// rounding as always dividing: away from a half-way point both round alike).
template <int BITS>
__device__ __forceinline__ GroupParams group_params(float lo, float hi) {
    constexpr float qmax = (float)((1 << BITS) - 1);
    GroupParams g;
    lo = fminf(lo, 0.f);
    hi = fmaxf(hi, 0.f);
    g.d = __fsub_rn(hi, lo);
    g.delta = __fdiv_rn(g.d, qmax);
    g.inv = __fdiv_rn(1.0f, g.delta);
    g.ok = isfinite(g.inv);
    const float uz = __fmul_rn(-lo, g.inv);
    float rz = rintf(uz);
    if (near_half(uz, rz)) rz = rintf(__fdiv_rn(__fmul_rn(-lo, qmax), g.d));
    g.z = g.ok ? clampf(rz, 0.f, qmax) : 0.f;
    return g;
}

// Codes of 8 values.  exact: element ratios near a half-way point are
// recomputed by the division (matrices without scales, whose ratios can be
// exact half-way points, and 8-bit codes, where the fast ratio's error can
// exceed the 1e-5 near-tie window).  Otherwise (2-4-bit codes of a balanced
// matrix) the fast ratio is within 4 ulps * 15 = 3.6e-6 of the exact one, so
// the two can differ only at near ties of the definition.
template <int BITS>
__device__ __forceinline__ void code8(const float (&x)[8], const GroupParams& g, bool exact,
                                      uint32_t (&c)[8]) {
    constexpr float qmax = (float)((1 << BITS) - 1);
    float r[8];
    bool near = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float u = __fmul_rn(x[k], g.inv);
        r[k] = rintf(u);
        if (exact) near |= near_half(u, r[k]);
    }
    if (near) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float u = __fmul_rn(x[k], g.inv);
            if (near_half(u, rintf(u))) r[k] = rintf(__fdiv_rn(__fmul_rn(x[k], qmax), g.d));
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = g.ok ? (uint32_t)clampf(r[k] + g.z, 0.f, qmax) : 0u;
}

// Code-book grid: a = max |x| of the group, inv = 1/a (0 when not finite,
// so y = x * inv = 0 and the code is that of level nearest 0).
struct CbParams {
    float a, inv;
};
__device__ __forceinline__ CbParams cb_params(float lo, float hi) {
    CbParams p;
    p.a = fmaxf(hi, -lo);  // max |x| from the group's min and max
    const float inv = __fdiv_rn(1.0f, p.a);
    p.inv = isfinite(inv) ? inv : 0.0f;
    return p;
}

// Copies the code book into LDS; every thread of the workgroup takes part,
// before any early exit.  Called after the workgroup's data loads are issued,
// so the table's load latency overlaps theirs.
template <bool CB>
__device__ __forceinline__ const CbTable* stage_book(const CbTable* g) {
    if constexpr (!CB) {
        return nullptr;
    } else {
        __shared__ CbTable sh;
        constexpr int kWords = sizeof(CbTable) / 4;
        static_assert(kWords <= kT, "one word per thread");
        if (threadIdx.x < kWords)
            reinterpret_cast<uint32_t*>(&sh)[threadIdx.x] =
                gload<uint32_t>(reinterpret_cast<const uint32_t*>(g) + threadIdx.x);
        __syncthreads();
        return &sh;
    }
}

// The levels alone (dequantisation), same rules as stage_book.
template <bool CB>
__device__ __forceinline__ const float* stage_levels(const CbTable* g) {
    if constexpr (!CB) {
        return nullptr;
    } else {
        __shared__ float lv[kCbMax];
        if (threadIdx.x < kCbMax) lv[threadIdx.x] = gload<float>(g->level + threadIdx.x);
        __syncthreads();
        return lv;
    }
}

// code = number of midpoints m_k with y > m_k (the nearest level; a tie
// goes to the lower one).  The cell index comes from the bits of z = y + 3
// (one rounding): z in [2, 4) has a fixed exponent, so mantissa bits 22..16
// are floor((z - 2) * 64), which is the true cell floor((y + 1) * 64) or a
// neighbour (the rounding moves it by at most 2^-17 of a cell), both of
// which the table covers.  Clamping the bits to [2, 4) handles |y| up to
// 1 + 2^-23 and keeps a NaN's index in the table, with no float-to-int
// conversion.  The cell bounds the count to [lo, lo + steps]; the midpoints
// ascend, so each comparison with mid[code] either adds one or leaves the
// code final.
__device__ __forceinline__ void code8_cb(const float (&x)[8], float inv, const CbTable* bk,
                                         int steps, uint32_t (&c)[8]) {
    static_assert(kCbCells == 128, "7 mantissa bits index the table");
    constexpr int lo_bits = 0x40000000, hi_bits = 0x407FFFFF;  // 2.0f, largest float below 4
    // Phases, so that the eight reads of each kind are in flight together.
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        y[k] = __fmul_rn(x[k], inv);
        const int zb = min(max(__float_as_int(__fadd_rn(y[k], 3.0f)), lo_bits), hi_bits);
        c[k] = bk->lo[(zb >> 16) & (kCbCells - 1)];
    }
#pragma nounroll
    for (int st = 0; st < steps; ++st) {
        float m[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = bk->mid[c[k]];
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] += y[k] > m[k] ? 1u : 0u;
    }
}

// A group's parameters on either grid: derived from the group's min / max,
// coding 8 values, storing the per-group scale (and zero-point).
template <bool CB, int BITS>
struct Grid {
    GroupParams g;
    CbParams p;
    __device__ __forceinline__ Grid(float lo, float hi) {
        if constexpr (CB) p = cb_params(lo, hi);
        else g = group_params<BITS>(lo, hi);
    }
    __device__ __forceinline__ void code(const float (&x)[8], const CbTable* bk, int steps,
                                         bool exact, uint32_t (&c)[8]) const {
        if constexpr (CB) code8_cb(x, p.inv, bk, steps, c);
        else code8<BITS>(x, g, exact, c);
    }
    __device__ __forceinline__ void store(const QMat& q, uint32_t gi) const {
        if constexpr (CB) {
            gstore<float>(q.scales + gi, p.a);
        } else {
            gstore<float>(q.scales + gi, g.delta);
            gstore<uint8_t>(q.zeros + gi, (uint8_t)g.z);
        }
    }
};

// Raw storage of 8 elements: a 16-byte bf16 vector or two float4.
template <int DT> struct Raw8;
template <> struct Raw8<WOQ_BF16> { uint4 v; };
template <> struct Raw8<WOQ_F32> { float4 a, b; };

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw(const void* base, uint32_t e) {
    Raw8<DT> r;
    if constexpr (DT == WOQ_BF16) {
        r.v = gload_u4(reinterpret_cast<const uint16_t*>(base) + e);
    } else {
        const float* p = reinterpret_cast<const float*>(base) + e;
        r.a = gload_f4(p);
        r.b = gload_f4(p + 4);
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void unpack_raw(const Raw8<DT>& r, float (&x)[8]) {
    if constexpr (DT == WOQ_BF16) {
        x[0] = bf_lo(r.v.x); x[1] = bf_hi(r.v.x); x[2] = bf_lo(r.v.y); x[3] = bf_hi(r.v.y);
        x[4] = bf_lo(r.v.z); x[5] = bf_hi(r.v.z); x[6] = bf_lo(r.v.w); x[7] = bf_hi(r.v.w);
    } else {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
}

// 1/t for 8 consecutive columns.
__device__ __forceinline__ void load_ct(const float* ct, uint32_t col, float (&c)[8]) {
    const float4 a = gload_f4(ct + col), b = gload_f4(ct + col + 4);
    c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
    c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
}

// x = (w * (1/s_i)) * (1/t_j), each product rounded once.  An absent scale
// is passed as 1.0f: multiplying by exactly 1 is the identity in IEEE
// arithmetic, so the result equals skipping the product (and there is no
// per-element select).
template <int DT>
__device__ __forceinline__ void balance(const Raw8<DT>& r, float rsv, const float (&c)[8],
                                        float (&x)[8]) {
    unpack_raw<DT>(r, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(__fmul_rn(x[k], rsv), c[k]);
}

// min / max over aligned groups of `lanes` lanes (a power of two <= 64):
// DPP within rows of 16 lanes, permlane swaps across them.
__device__ __forceinline__ void group_minmax(float& lo, float& hi, int lanes) {
    if (lanes >= 2) { lo = fminf(lo, dpp<kDppXor1>(lo)); hi = fmaxf(hi, dpp<kDppXor1>(hi)); }
    if (lanes >= 4) { lo = fminf(lo, dpp<kDppXor2>(lo)); hi = fmaxf(hi, dpp<kDppXor2>(hi)); }
    if (lanes >= 8) { lo = fminf(lo, dpp<kDppMirror8>(lo)); hi = fmaxf(hi, dpp<kDppMirror8>(hi)); }
    if (lanes >= 16) { lo = fminf(lo, dpp<kDppMirror16>(lo)); hi = fmaxf(hi, dpp<kDppMirror16>(hi)); }
    if (lanes >= 32) {
        float a = lo, b = lo, c = hi, d = hi;
        swap16(a, b);
        swap16(c, d);
        lo = fminf(a, b);
        hi = fmaxf(c, d);
    }
    if (lanes >= 64) {
        float a = lo, b = lo, c = hi, d = hi;
        swap32(a, b);
        swap32(c, d);
        lo = fminf(a, b);
        hi = fmaxf(c, d);
    }
}

// Groups of 8..512 columns (powers of two).  A workgroup takes a tile of
// kTileRows rows x kTileCols columns of one matrix; thread t owns the 8
// columns 8t.. of the tile, so its 1/t factors are loaded once and the
// tile's rows are all in flight before the first is coded.  A group is
// group/8 consecutive lanes; groups never straddle the tile's edge because
// cols is a multiple of the group size.
constexpr int kTileRows = kQTileRows;
constexpr int kTileCols = kQTileCols;
static_assert(kTileCols == 8 * kT, "one 8-column vector per thread");

// TIE: the launch may hold matrices whose ratios need the near-half
// fallback of code8 (no scales, or 8-bit codes); without it no check is made.
template <int DT, int BITS, bool CB, bool TIE>
__global__ __launch_bounds__(kT) void k_quant_tile(const QMat* __restrict__ mats,
                                                   const int64_t* __restrict__ ubeg, int nmat,
                                                   const CbTable* __restrict__ book, int steps) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int ctiles = (q.cols + kTileCols - 1) / kTileCols;
    const int tl = (int)(u - ubeg[m]);
    const int rt = tl / ctiles;
    const uint32_t col = (uint32_t)(tl - rt * ctiles) * kTileCols + 8u * threadIdx.x;
    const bool active = col < (uint32_t)q.cols;
    const int r0 = rt * kTileRows;
    const int nr = min(kTileRows, q.rows - r0);
    const int lanes = q.group >> 3;
    const bool has_rs = q.rs != nullptr, has_ct = q.ct != nullptr;
    const bool exact = TIE && ((!has_rs && !has_ct) || BITS == 8);  // near-half fallback (code8)
    float c[8];
    if (has_ct && active) load_ct(q.ct, col, c);
    else {
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = 1.0f;
    }
    Raw8<DT> raw[kTileRows];
    float rsv[kTileRows];  // every load is issued before the first use
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
        if (r < nr && active) raw[r] = load_raw<DT>(q.data, (uint32_t)(r0 + r) * (uint32_t)q.ld + col);
        rsv[r] = has_rs && r < nr ? gload<float>(q.rs + r0 + r) : 1.0f;
    }
    const CbTable* bk = stage_book<CB>(book);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
        if (r >= nr) break;
        const uint32_t row = (uint32_t)(r0 + r);
        float x[8];
        if (active) balance<DT>(raw[r], rsv[r], c, x);
        else {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = 0.f;
        }
        float lo = x[0], hi = x[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) { lo = fminf(lo, x[k]); hi = fmaxf(hi, x[k]); }
        group_minmax(lo, hi, lanes);
        const Grid<CB, BITS> g(lo, hi);
        if (active) {
            const uint32_t e0 = row * (uint32_t)q.cols + col;
            uint32_t cd[8];
            g.code(x, bk, steps, exact, cd);
            store_codes<BITS>(q.codes, e0, cd);
            if ((threadIdx.x & (lanes - 1)) == 0)
                g.store(q, e0 >> __builtin_ctz((uint32_t)q.group));  // power-of-two group
        }
    }
}

// Groups of more than 512 and at most 64 * 8 * NVL columns: one wave per
// group (four per workgroup), values kept packed in registers between the
// min / max reduction and the coding pass.
template <int DT, int BITS, int NVL, bool CB, bool TIE>
__global__ __launch_bounds__(kT) void k_quant_wave(const QMat* __restrict__ mats,
                                                   const int64_t* __restrict__ ubeg, int nmat,
                                                   const CbTable* __restrict__ book, int steps) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int lane = threadIdx.x & 63;
    const uint32_t ng = (uint32_t)q.rows * (uint32_t)q.cols / (uint32_t)q.group;
    const uint32_t gi = (uint32_t)(u - ubeg[m]) * (kT / 64) + (threadIdx.x >> 6);
    const bool live = gi < ng;  // whole wave
    const uint32_t gbase = live ? gi * (uint32_t)q.group : 0u;  // codes (contiguous)
    const uint32_t row = gbase / (uint32_t)q.cols;
    const uint32_t col0 = gbase - row * (uint32_t)q.cols;
    const uint32_t ibase = row * (uint32_t)q.ld + col0;           // weights (row stride ld)
    const int nvg = q.group >> 3;
    const bool has_rs = q.rs != nullptr, has_ct = q.ct != nullptr;
    const bool exact = TIE && ((!has_rs && !has_ct) || BITS == 8);  // near-half fallback (code8)
    const float rsv = has_rs && live ? gload<float>(q.rs + row) : 1.0f;
    Raw8<DT> raw[NVL];
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
        const int v = lane + 64 * k;
        if (live && v < nvg) raw[k] = load_raw<DT>(q.data, ibase + 8u * v);
    }
    const CbTable* bk = stage_book<CB>(book);
    if (!live) return;  // after the workgroup barrier; none below
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
        const int v = lane + 64 * k;
        if (v < nvg) {
            float c[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}, x[8];
            if (has_ct) load_ct(q.ct, col0 + 8u * v, c);
            balance<DT>(raw[k], rsv, c, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) { lo = fminf(lo, x[e]); hi = fmaxf(hi, x[e]); }
        }
    }
    group_minmax(lo, hi, 64);
    const Grid<CB, BITS> g(lo, hi);
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
        const int v = lane + 64 * k;
        if (v < nvg) {
            float c[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}, x[8];
            if (has_ct) load_ct(q.ct, col0 + 8u * v, c);
            balance<DT>(raw[k], rsv, c, x);
            uint32_t cd[8];
            g.code(x, bk, steps, exact, cd);
            store_codes<BITS>(q.codes, gbase + 8u * v, cd);
        }
    }
    if (lane == 0) g.store(q, gi);
}

// Wider groups (e.g. one group per row of 14336 columns): one workgroup per
// group, raw values kept in registers between the min / max reduction
// (waves, then one LDS exchange) and the coding pass.
template <int DT, int BITS, bool CB, bool TIE>
__global__ __launch_bounds__(kT) void k_quant_big(const QMat* __restrict__ mats,
                                                  const int64_t* __restrict__ ubeg,
                                                  int nmat, const CbTable* __restrict__ book,
                                                  int steps) {
    constexpr int MAXV = (DT == WOQ_BF16) ? 16 : 8;
    __shared__ float2 sh[kT / 64];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const uint32_t gl = (uint32_t)(u - ubeg[m]);
    const uint32_t gbase = gl * (uint32_t)q.group;               // codes (contiguous)
    const uint32_t row = gbase / (uint32_t)q.cols;
    const uint32_t col0 = gbase - row * (uint32_t)q.cols;
    const uint32_t ibase = row * (uint32_t)q.ld + col0;          // weights (row stride ld)
    const int nvg = q.group >> 3;
    const bool has_rs = q.rs != nullptr, has_ct = q.ct != nullptr;
    const bool exact = TIE && ((!has_rs && !has_ct) || BITS == 8);  // near-half fallback (code8)
    const float rsv = has_rs ? gload<float>(q.rs + row) : 1.0f;

    Raw8<DT> raw[MAXV];
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nvg) raw[k] = load_raw<DT>(q.data, ibase + 8u * v);
    }
    const CbTable* bk = stage_book<CB>(book);
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nvg) {
            float c[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}, x[8];
            if (has_ct) load_ct(q.ct, col0 + 8u * v, c);
            balance<DT>(raw[k], rsv, c, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) { lo = fminf(lo, x[e]); hi = fmaxf(hi, x[e]); }
        }
    }
    group_minmax(lo, hi, 64);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = make_float2(lo, hi);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) { lo = fminf(lo, sh[w].x); hi = fmaxf(hi, sh[w].y); }
    const Grid<CB, BITS> g(lo, hi);
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nvg) {
            float c[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}, x[8];
            if (has_ct) load_ct(q.ct, col0 + 8u * v, c);
            balance<DT>(raw[k], rsv, c, x);
            uint32_t cd[8];
            g.code(x, bk, steps, exact, cd);
            store_codes<BITS>(q.codes, gbase + 8u * v, cd);
        }
    }
    if (threadIdx.x == 0) g.store(q, gl);
}

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32,
// packed low / high into 32 bits.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Dequantisation W' = (((q - z) delta) s_i) t_j (code book: ((a l_q) s_i)
// t_j), one fp32 rounding per product, then (bf16 output) one
// round-to-nearest-even.  Same tiles as
// k_quant_tile: a workgroup takes 8 rows x 2048 columns, thread t the 8
// columns 8t..; t_j is loaded once per tile, s_i once per row.
template <int BITS>
__device__ __forceinline__ void load_codes_g(const uint8_t* codes, uint32_t e0, uint32_t (&c)[8]) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (BITS == 8) {
        const f32x2 w = gload<f32x2>(codes + e0);
        const uint32_t lo = __float_as_uint(w.x), hi = __float_as_uint(w.y);
#pragma unroll
        for (int k = 0; k < 4; ++k) { c[k] = (lo >> (8 * k)) & mask; c[k + 4] = (hi >> (8 * k)) & mask; }
    } else {
        uint32_t w;
        if constexpr (BITS == 4) w = gload<uint32_t>(codes + (e0 >> 1));
        else if constexpr (BITS == 2) w = gload<uint16_t>(codes + (e0 >> 2));
        else {
            const uint8_t* p = codes + (size_t)(e0 >> 3) * 3;
            w = (uint32_t)gload<uint8_t>(p) | ((uint32_t)gload<uint8_t>(p + 1) << 8) |
                ((uint32_t)gload<uint8_t>(p + 2) << 16);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = (w >> (BITS * k)) & mask;
    }
}

template <int BITS, int ODT, bool CB>
__global__ __launch_bounds__(kT) void k_dequant(const QMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat,
                                                int zdef, const CbTable* __restrict__ book) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int ctiles = (q.cols + kTileCols - 1) / kTileCols;
    const int tl = (int)(u - ubeg[m]);
    const int rt = tl / ctiles;
    const uint32_t col = (uint32_t)(tl - rt * ctiles) * kTileCols + 8u * threadIdx.x;
    // Lanes past the matrix's edge exit at once on the affine grid; on the
    // code-book grid they first join the workgroup barrier of the level table.
    const bool active = col < (uint32_t)q.cols;
    if constexpr (!CB) {
        if (!active) return;
    }
    const int r0 = rt * kDTileRows;
    const int nr = min(kDTileRows, q.rows - r0);
    const bool has_rs = q.rs != nullptr, has_ct = q.ct != nullptr;
    float t8[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (has_ct && active) load_ct(q.ct, col, t8);
    // Every load of the tile (codes and the per-row group parameters) is
    // issued before the first use.  The group divides the row and is a
    // multiple of 8, so a thread's 8 columns share one group, whose index is
    // row * (cols / group) + col / group.
    const uint32_t gpr = (uint32_t)q.cols / (uint32_t)q.group, gcol = col / (uint32_t)q.group;
    uint32_t cw[kDTileRows][8];
    float delta[kDTileRows], rsv[kDTileRows];
    int zr[kDTileRows];
#pragma unroll
    for (int r = 0; r < kDTileRows; ++r) {
        if (r < nr && active) {
            const uint32_t row = (uint32_t)(r0 + r), gi = row * gpr + gcol;
            load_codes_g<BITS>(q.codes, row * (uint32_t)q.cols + col, cw[r]);
            delta[r] = gload<float>(q.scales + gi);
            if constexpr (!CB) zr[r] = q.zeros ? (int)gload<uint8_t>(q.zeros + gi) : zdef;
            rsv[r] = has_rs ? gload<float>(q.rs + row) : 1.0f;
        }
    }
    const float* lv = stage_levels<CB>(book);
    if (!active) return;
#pragma unroll
    for (int r = 0; r < kDTileRows; ++r) {
        if (r >= nr) break;
        const uint32_t e0 = (uint32_t)(r0 + r) * (uint32_t)q.ld + col;  // output row stride ld
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {  // absent scales are exactly 1 (identity)
            // affine: (q - z) * delta; code book: a * level[q]
            float v;
            if constexpr (CB) v = __fmul_rn(delta[r], lv[cw[r][k]]);
            else v = __fmul_rn((float)((int)cw[r][k] - zr[r]), delta[r]);
            y[k] = __fmul_rn(__fmul_rn(v, rsv[r]), t8[k]);
        }
        if constexpr (ODT == WOQ_F32) {
            float* o = const_cast<float*>(reinterpret_cast<const float*>(q.data)) + e0;
            gstore_f4(o, y[0], y[1], y[2], y[3]);
            gstore_f4(o + 4, y[4], y[5], y[6], y[7]);
        } else {
            u32x4 w;
            w.x = f32x2_to_bf16x2(y[0], y[1]);
            w.y = f32x2_to_bf16x2(y[2], y[3]);
            w.z = f32x2_to_bf16x2(y[4], y[5]);
            w.w = f32x2_to_bf16x2(y[6], y[7]);
            gstore<u32x4>(const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(q.data)) + e0, w);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kT) void k_ternary(const QMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat) {
    constexpr int MAXV = (DT == WOQ_BF16) ? 16 : 8;
    __shared__ double shd[kT / 64];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const uint32_t row = (uint32_t)(u - ubeg[m]);
    const uint32_t rbase = row * (uint32_t)q.cols;   // codes (contiguous)
    const uint32_t ibase = row * (uint32_t)q.ld;     // weights (row stride ld)
    const int nv = q.cols >> 3;
    Raw8<DT> raw[MAXV];
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nv) raw[k] = load_raw<DT>(q.data, ibase + 8u * v);
    }
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nv) {
            float x[8];
            unpack_raw<DT>(raw[k], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (double)fabsf(x[e]);
        }
    }
    // row sum of |w| in fp64: waves, then the wave totals in wave order
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) shd[threadIdx.x >> 6] = acc;
    __syncthreads();
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) sum += shd[w];
    const float beta = (float)(sum / (double)q.cols);
    const float inv = __fdiv_rn(1.0f, beta);
    const bool ok = isfinite(inv);
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nv) {
            float x[8];
            unpack_raw<DT>(raw[k], x);
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = ok ? clampf(rintf(__fmul_rn(x[e], inv)), -1.f, 1.f) : 0.f;
                w |= (uint32_t)(int)(t + 1.0f) << (2 * e);
            }
            gstore<uint16_t>(q.codes + ((rbase + 8u * v) >> 2), (uint16_t)w);
        }
    }
    if (threadIdx.x == 0) gstore<float>(q.scales + row, beta);
}

// Ternary codes for rows of at most 64 * 8 * NVL columns: one wave per row,
// kTernRows rows per workgroup (wave w takes rows w, w + 4, ...), the next
// row's loads issued before the current row is coded.  Same arithmetic as
// k_ternary: beta = (sum |w| in fp64, lanes then the wave) / cols, rounded
// once to fp32; code q + 1 with q = clamp(rne(w * (1/beta)), -1, 1).
template <int DT, int NVL>
__global__ __launch_bounds__(kT) void k_ternary_wave(const QMat* __restrict__ mats,
                                                     const int64_t* __restrict__ ubeg, int nmat) {
    constexpr int RPW = kTernRows / 4;  // rows per wave
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int lane = threadIdx.x & 63;
    const int nv = q.cols >> 3;
    const int r0 = (int)(u - ubeg[m]) * kTernRows + (threadIdx.x >> 6);
    Raw8<DT> buf[2][NVL];
    auto load = [&](Raw8<DT> (&b)[NVL], int row) {
#pragma unroll
        for (int k = 0; k < NVL; ++k) {
            const int v = lane + 64 * k;
            if (v < nv) b[k] = load_raw<DT>(q.data, (uint32_t)row * (uint32_t)q.ld + 8u * v);
        }
    };
    if (r0 < q.rows) load(buf[0], r0);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int row = r0 + 4 * i;
        if (row >= q.rows) break;  // wave-uniform
        if (i + 1 < RPW && row + 4 < q.rows) load(buf[(i + 1) & 1], row + 4);
        Raw8<DT>(&b)[NVL] = buf[i & 1];
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < NVL; ++k) {
            if (lane + 64 * k < nv) {
                float x[8];
                unpack_raw<DT>(b[k], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += (double)fabsf(x[e]);
            }
        }
        acc = wave_sum(acc);
        const float beta = (float)(acc / (double)q.cols);
        const float inv = __fdiv_rn(1.0f, beta);
        const bool ok = isfinite(inv);
        const uint32_t rbase = (uint32_t)row * (uint32_t)q.cols;   // codes (contiguous)
#pragma unroll
        for (int k = 0; k < NVL; ++k) {
            const int v = lane + 64 * k;
            if (v < nv) {
                float x[8];
                unpack_raw<DT>(b[k], x);
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = ok ? clampf(rintf(__fmul_rn(x[e], inv)), -1.f, 1.f) : 0.f;
                    w |= (uint32_t)(int)(t + 1.0f) << (2 * e);
                }
                gstore<uint16_t>(q.codes + ((rbase + 8u * v) >> 2), (uint16_t)w);
            }
        }
        if (lane == 0) gstore<float>(q.scales + row, beta);
    }
}

__global__ __launch_bounds__(kT) void k_recip(const RecipSeg* __restrict__ segs,
                                              const int64_t* __restrict__ ubeg, int nseg) {
    const int64_t u = blockIdx.x;
    const int s = find_unit_owner(ubeg, nseg, u);
    const RecipSeg sg = segs[s];
    const int64_t i = (u - ubeg[s]) * kT + threadIdx.x;
    if (i < sg.n) gstore<float>(sg.dst + i, __fdiv_rn(1.0f, gload<float>(sg.src + i)));
}

// Calls f(Bits<b>{}) for the code width; the code-book grid has no 8-bit
// form (the API admits 2, 3 and 4 bits for it).
template <int B> struct Bits { static constexpr int value = B; };
template <bool CB, class F>
hipError_t by_bits(int bits, F&& f) {
    switch (bits) {
        case 2: f(Bits<2>{}); break;
        case 3: f(Bits<3>{}); break;
        case 4: f(Bits<4>{}); break;
        default:
            if constexpr (CB) return hipErrorInvalidValue;
            else f(Bits<8>{});
    }
    return hipGetLastError();
}

// Calls f(std::bool_constant<tie>) (the code-book grid has no fallback).
template <bool CB, class F>
void by_tie(bool tie, F&& f) {
    if constexpr (CB) f(std::false_type{});
    else if (tie) f(std::true_type{});
    else f(std::false_type{});
}

template <int DT, bool CB>
hipError_t quant_tile_g(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        int bits, const CbTable* book, int steps, bool tie, hipStream_t s) {
    return by_bits<CB>(bits, [&](auto b) {
        by_tie<CB>(tie, [&](auto t) {
            k_quant_tile<DT, decltype(b)::value, CB, decltype(t)::value>
                <<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, book, steps);
        });
    });
}

template <int DT, int NVL, bool CB>
hipError_t quant_wave_g(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        int bits, const CbTable* book, int steps, bool tie, hipStream_t s) {
    return by_bits<CB>(bits, [&](auto b) {
        by_tie<CB>(tie, [&](auto t) {
            k_quant_wave<DT, decltype(b)::value, NVL, CB, decltype(t)::value>
                <<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, book, steps);
        });
    });
}

template <int DT, bool CB>
hipError_t quant_wave_nv(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                         int bits, int nvl, const CbTable* book, int steps, bool tie, hipStream_t s) {
    switch (nvl) {
        case 1: return quant_wave_g<DT, 1, CB>(mats, ubeg, nmat, n_units, bits, book, steps, tie, s);
        case 2: return quant_wave_g<DT, 2, CB>(mats, ubeg, nmat, n_units, bits, book, steps, tie, s);
        case 4: return quant_wave_g<DT, 4, CB>(mats, ubeg, nmat, n_units, bits, book, steps, tie, s);
        default: return quant_wave_g<DT, 8, CB>(mats, ubeg, nmat, n_units, bits, book, steps, tie, s);
    }
}

template <int DT, bool CB>
hipError_t quant_big_g(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                       int bits, const CbTable* book, int steps, bool tie, hipStream_t s) {
    return by_bits<CB>(bits, [&](auto b) {
        by_tie<CB>(tie, [&](auto t) {
            k_quant_big<DT, decltype(b)::value, CB, decltype(t)::value>
                <<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, book, steps);
        });
    });
}

template <int ODT, bool CB>
hipError_t dequant_g(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     int bits, const CbTable* book, hipStream_t s) {
    const int zdef = (1 << (bits - 1)) - 1;
    return by_bits<CB>(bits, [&](auto b) {
        k_dequant<decltype(b)::value, ODT, CB>
            <<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, zdef, book);
    });
}

}  // namespace

hipError_t recip(const RecipSeg* segs, const int64_t* ubeg, int nseg, int64_t n_units,
                 hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_recip<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(segs, ubeg, nseg);
    return hipGetLastError();
}

hipError_t quant_tile(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                      int dtype, int bits, const CbTable* book, int steps, bool tie,
                      hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (book)
        return dtype == WOQ_BF16
                   ? quant_tile_g<WOQ_BF16, true>(mats, ubeg, nmat, n_units, bits, book, steps, false, s)
                   : quant_tile_g<WOQ_F32, true>(mats, ubeg, nmat, n_units, bits, book, steps, false, s);
    return dtype == WOQ_BF16
               ? quant_tile_g<WOQ_BF16, false>(mats, ubeg, nmat, n_units, bits, nullptr, 0, tie, s)
               : quant_tile_g<WOQ_F32, false>(mats, ubeg, nmat, n_units, bits, nullptr, 0, tie, s);
}

hipError_t quant_wave(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                      int dtype, int bits, int nvl, const CbTable* book, int steps, bool tie,
                      hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (book)
        return dtype == WOQ_BF16
                   ? quant_wave_nv<WOQ_BF16, true>(mats, ubeg, nmat, n_units, bits, nvl, book, steps, false, s)
                   : quant_wave_nv<WOQ_F32, true>(mats, ubeg, nmat, n_units, bits, nvl, book, steps, false, s);
    return dtype == WOQ_BF16
               ? quant_wave_nv<WOQ_BF16, false>(mats, ubeg, nmat, n_units, bits, nvl, nullptr, 0, tie, s)
               : quant_wave_nv<WOQ_F32, false>(mats, ubeg, nmat, n_units, bits, nvl, nullptr, 0, tie, s);
}

hipError_t quant_big(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     int dtype, int bits, const CbTable* book, int steps, bool tie, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (book)
        return dtype == WOQ_BF16
                   ? quant_big_g<WOQ_BF16, true>(mats, ubeg, nmat, n_units, bits, book, steps, false, s)
                   : quant_big_g<WOQ_F32, true>(mats, ubeg, nmat, n_units, bits, book, steps, false, s);
    return dtype == WOQ_BF16
               ? quant_big_g<WOQ_BF16, false>(mats, ubeg, nmat, n_units, bits, nullptr, 0, tie, s)
               : quant_big_g<WOQ_F32, false>(mats, ubeg, nmat, n_units, bits, nullptr, 0, tie, s);
}

hipError_t dequant(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                   int out_dtype, int bits, const CbTable* book, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (book)
        return out_dtype == WOQ_BF16
                   ? dequant_g<WOQ_BF16, true>(mats, ubeg, nmat, n_units, bits, book, s)
                   : dequant_g<WOQ_F32, true>(mats, ubeg, nmat, n_units, bits, book, s);
    return out_dtype == WOQ_BF16
               ? dequant_g<WOQ_BF16, false>(mats, ubeg, nmat, n_units, bits, nullptr, s)
               : dequant_g<WOQ_F32, false>(mats, ubeg, nmat, n_units, bits, nullptr, s);
}

hipError_t ternary(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units, int dtype,
                   hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (dtype == WOQ_BF16)
        k_ternary<WOQ_BF16><<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat);
    else
        k_ternary<WOQ_F32><<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat);
    return hipGetLastError();
}

template <int DT>
hipError_t ternary_wave_dt(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                           int nvl, hipStream_t s) {
    const dim3 g((unsigned)n_units), b(kT);
    switch (nvl) {
        case 1: k_ternary_wave<DT, 1><<<g, b, 0, s>>>(mats, ubeg, nmat); break;
        case 2: k_ternary_wave<DT, 2><<<g, b, 0, s>>>(mats, ubeg, nmat); break;
        case 4: k_ternary_wave<DT, 4><<<g, b, 0, s>>>(mats, ubeg, nmat); break;
        default: k_ternary_wave<DT, 8><<<g, b, 0, s>>>(mats, ubeg, nmat); break;
    }
    return hipGetLastError();
}

hipError_t ternary_wave(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        int dtype, int nvl, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    return dtype == WOQ_BF16 ? ternary_wave_dt<WOQ_BF16>(mats, ubeg, nmat, n_units, nvl, s)
                             : ternary_wave_dt<WOQ_F32>(mats, ubeg, nmat, n_units, nvl, s);
}

}  // namespace woq
