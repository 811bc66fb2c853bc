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
// so codes, deltas and zero-points are reproducible bit for bit.
//
// Work mapping:
//  k_quant_small  groups of 8..512 columns: a work unit is 2048 consecutive
//                 elements of one matrix; each thread owns 8 consecutive
//                 elements (one 16-byte bf16 load), a group is owned by
//                 group/8 consecutive lanes of one wave and reduced with
//                 shuffles.  Groups tile the row-major matrix contiguously,
//                 so group g starts at element g*group.
//  k_quant_big    larger groups (e.g. one group per row): one workgroup per
//                 group, raw values kept in registers between the min/max
//                 reduction and the coding pass.
//  k_dequant      2048-element units, 8 elements per thread.
//  k_ternary      one workgroup per row.
#include "launch.h"

#include <math.h>

namespace woq {
namespace {

constexpr int kT = 256;

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
    return fminf(fmaxf(v, lo), hi);
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* codes, uint32_t e0, const uint32_t (&c)[8]) {
    if constexpr (BITS == 8) {
        uint2 w;
        w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        *reinterpret_cast<uint2*>(codes + e0) = w;
    } else if constexpr (BITS == 4) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (4 * k);
        *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = w;
    } else if constexpr (BITS == 2) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (2 * k);
        *reinterpret_cast<uint16_t*>(codes + (e0 >> 2)) = (uint16_t)w;
    } else {  // 3 bits: 8 codes fill exactly 3 bytes
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= c[k] << (3 * k);
        uint8_t* p = codes + (size_t)(e0 >> 3) * 3;
        p[0] = (uint8_t)w;
        p[1] = (uint8_t)(w >> 8);
        p[2] = (uint8_t)(w >> 16);
    }
}

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* codes, uint32_t e0, uint32_t (&c)[8]) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (BITS == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(codes + e0);
#pragma unroll
        for (int k = 0; k < 4; ++k) { c[k] = (w.x >> (8 * k)) & mask; c[k + 4] = (w.y >> (8 * k)) & mask; }
    } else {
        uint32_t w;
        if constexpr (BITS == 4) w = *reinterpret_cast<const uint32_t*>(codes + (e0 >> 1));
        else if constexpr (BITS == 2) w = *reinterpret_cast<const uint16_t*>(codes + (e0 >> 2));
        else {
            const uint8_t* p = codes + (size_t)(e0 >> 3) * 3;
            w = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = (w >> (BITS * k)) & mask;
    }
}

// x = (w * rs_row) * ct_col, each product rounded once; absent scales skipped.
template <int DT>
__device__ __forceinline__ void balanced8(const QMat& q, uint32_t e0, float (&x)[8]) {
    load8<DT>(q.data, e0, x);
    if (q.rs || q.ct) {
        const uint32_t row = e0 / (uint32_t)q.cols;
        const uint32_t col = e0 - row * (uint32_t)q.cols;
        if (q.rs) {
            const float r = q.rs[row];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(x[k], r);
        }
        if (q.ct) {
            float c[8];
            load8f(q.ct + col, c);
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(x[k], c[k]);
        }
    }
}

struct GroupParams {
    float delta, inv, z;
    bool ok;
};

template <int BITS>
__device__ __forceinline__ GroupParams group_params(float lo, float hi) {
    constexpr float qmax = (float)((1 << BITS) - 1);
    GroupParams g;
    lo = fminf(lo, 0.f);
    hi = fmaxf(hi, 0.f);
    g.delta = __fdiv_rn(__fsub_rn(hi, lo), qmax);
    g.inv = __fdiv_rn(1.0f, g.delta);
    g.ok = isfinite(g.inv);
    g.z = g.ok ? clampf(rintf(__fmul_rn(-lo, g.inv)), 0.f, qmax) : 0.f;
    return g;
}

template <int BITS>
__device__ __forceinline__ void code8(const float (&x)[8], const GroupParams& g, uint32_t (&c)[8]) {
    constexpr float qmax = (float)((1 << BITS) - 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float t = g.ok ? clampf(rintf(__fmul_rn(x[k], g.inv)) + g.z, 0.f, qmax) : 0.f;
        c[k] = (uint32_t)t;
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(kT) void k_quant_small(const QMat* __restrict__ mats,
                                                    const int64_t* __restrict__ ubeg,
                                                    int nmat) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int group = q.group;
    const uint32_t n = (uint32_t)q.rows * (uint32_t)q.cols;
    const uint32_t e0 = (uint32_t)(u - ubeg[m]) * kQTile + 8u * threadIdx.x;
    const bool active = e0 < n;
    float x[8];
    if (active) {
        balanced8<DT>(q, e0, x);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = 0.f;
    }
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) { lo = fminf(lo, x[k]); hi = fmaxf(hi, x[k]); }
    const int lanes = group >> 3;  // power of two, <= 64
    for (int o = 1; o < lanes; o <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, o, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, o, kWave));
    }
    const GroupParams g = group_params<BITS>(lo, hi);
    if (!active) return;
    uint32_t c[8];
    code8<BITS>(x, g, c);
    store_codes<BITS>(q.codes, e0, c);
    if ((threadIdx.x & (lanes - 1)) == 0) {
        const uint32_t gi = e0 / (uint32_t)group;
        q.scales[gi] = g.delta;
        q.zeros[gi] = (uint8_t)g.z;
    }
}

__device__ __forceinline__ float block_min_f(float v, float* sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) r = fminf(r, sh[w]);
    return r;
}

__device__ __forceinline__ float block_max_f(float v, float* sh) {
    v = wave_maxf(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) r = fmaxf(r, sh[w]);
    return r;
}

__device__ __forceinline__ double block_sum_d(double v, double* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) r += sh[w];
    return r;
}

// Raw storage of 8 elements: a 16-byte bf16 vector or two float4.
template <int DT> struct Raw8;
template <> struct Raw8<WOQ_BF16> { uint4 v; };
template <> struct Raw8<WOQ_F32> { float4 a, b; };

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw(const void* base, uint32_t e) {
    Raw8<DT> r;
    if constexpr (DT == WOQ_BF16) {
        r.v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + e);
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + e);
        r.a = p[0];
        r.b = p[1];
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void raw_to_x(const Raw8<DT>& r, const QMat& q, float rsv,
                                         uint32_t col, float (&x)[8]) {
    if constexpr (DT == WOQ_BF16) {
        x[0] = bf_lo(r.v.x); x[1] = bf_hi(r.v.x); x[2] = bf_lo(r.v.y); x[3] = bf_hi(r.v.y);
        x[4] = bf_lo(r.v.z); x[5] = bf_hi(r.v.z); x[6] = bf_lo(r.v.w); x[7] = bf_hi(r.v.w);
    } else {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
    if (q.rs) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(x[k], rsv);
    }
    if (q.ct) {
        float c[8];
        load8f(q.ct + col, c);
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(x[k], c[k]);
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(kT) void k_quant_big(const QMat* __restrict__ mats,
                                                  const int64_t* __restrict__ ubeg,
                                                  int nmat) {
    constexpr int MAXV = (DT == WOQ_BF16) ? 16 : 8;
    __shared__ float sh[kT / 64];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int group = q.group;
    const uint32_t gl = (uint32_t)(u - ubeg[m]);
    const uint32_t gbase = gl * (uint32_t)group;
    const uint32_t row = gbase / (uint32_t)q.cols;
    const uint32_t col0 = gbase - row * (uint32_t)q.cols;
    const float rsv = q.rs ? q.rs[row] : 1.0f;
    const int nvg = group >> 3;

    Raw8<DT> raw[MAXV];
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nvg) {
            raw[k] = load_raw<DT>(q.data, gbase + 8u * v);
            float x[8];
            raw_to_x<DT>(raw[k], q, rsv, col0 + 8u * v, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) { lo = fminf(lo, x[e]); hi = fmaxf(hi, x[e]); }
        }
    }
    lo = block_min_f(lo, sh);
    hi = block_max_f(hi, sh);
    const GroupParams g = group_params<BITS>(lo, hi);
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nvg) {
            float x[8];
            raw_to_x<DT>(raw[k], q, rsv, col0 + 8u * v, x);
            uint32_t c[8];
            code8<BITS>(x, g, c);
            store_codes<BITS>(q.codes, gbase + 8u * v, c);
        }
    }
    if (threadIdx.x == 0) {
        q.scales[gl] = g.delta;
        q.zeros[gl] = (uint8_t)g.z;
    }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int BITS, int ODT>
__global__ __launch_bounds__(kT) void k_dequant(const QMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat,
                                                int zdef) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const QMat q = mats[m];
    const int group = q.group;
    const uint32_t n = (uint32_t)q.rows * (uint32_t)q.cols;
    const uint32_t e0 = (uint32_t)(u - ubeg[m]) * kQTile + 8u * threadIdx.x;
    if (e0 >= n) return;
    uint32_t c[8];
    load_codes<BITS>(q.codes, e0, c);
    const uint32_t gi = e0 / (uint32_t)group;
    const float delta = q.scales[gi];
    const int z = q.zeros ? (int)q.zeros[gi] : zdef;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = __fmul_rn((float)((int)c[k] - z), delta);
    if (q.rs || q.ct) {
        const uint32_t row = e0 / (uint32_t)q.cols;
        const uint32_t col = e0 - row * (uint32_t)q.cols;
        if (q.rs) {
            const float r = q.rs[row];
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(y[k], r);
        }
        if (q.ct) {
            float t[8];
            load8f(q.ct + col, t);
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(y[k], t[k]);
        }
    }
    if constexpr (ODT == WOQ_F32) {
        float4* o = reinterpret_cast<float4*>(const_cast<float*>(
            reinterpret_cast<const float*>(q.data)) + e0);
        o[0] = make_float4(y[0], y[1], y[2], y[3]);
        o[1] = make_float4(y[4], y[5], y[6], y[7]);
    } else {
        uint4 w;
        w.x = f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16);
        w.y = f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16);
        w.z = f32_to_bf16_rne(y[4]) | (f32_to_bf16_rne(y[5]) << 16);
        w.w = f32_to_bf16_rne(y[6]) | (f32_to_bf16_rne(y[7]) << 16);
        *reinterpret_cast<uint4*>(const_cast<uint16_t*>(
            reinterpret_cast<const uint16_t*>(q.data)) + e0) = w;
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
    const uint32_t rbase = row * (uint32_t)q.cols;
    const int nv = q.cols >> 3;
    Raw8<DT> raw[MAXV];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nv) {
            raw[k] = load_raw<DT>(q.data, rbase + 8u * v);
            float x[8];
            QMat plain = q;
            plain.rs = nullptr;
            plain.ct = nullptr;
            raw_to_x<DT>(raw[k], plain, 1.0f, 0, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (double)fabsf(x[e]);
        }
    }
    const double sum = block_sum_d(acc, shd);
    const float beta = (float)(sum / (double)q.cols);
    const float inv = __fdiv_rn(1.0f, beta);
    const bool ok = isfinite(inv);
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int v = threadIdx.x + kT * k;
        if (v < nv) {
            float x[8];
            QMat plain = q;
            plain.rs = nullptr;
            plain.ct = nullptr;
            raw_to_x<DT>(raw[k], plain, 1.0f, 0, x);
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = ok ? clampf(rintf(__fmul_rn(x[e], inv)), -1.f, 1.f) : 0.f;
                w |= (uint32_t)(int)(t + 1.0f) << (2 * e);
            }
            *reinterpret_cast<uint16_t*>(q.codes + ((rbase + 8u * v) >> 2)) = (uint16_t)w;
        }
    }
    if (threadIdx.x == 0) q.scales[row] = beta;
}

__global__ __launch_bounds__(kT) void k_recip(const RecipSeg* __restrict__ segs,
                                              const int64_t* __restrict__ ubeg, int nseg) {
    const int64_t u = blockIdx.x;
    const int s = find_unit_owner(ubeg, nseg, u);
    const RecipSeg sg = segs[s];
    const int64_t i = (u - ubeg[s]) * kT + threadIdx.x;
    if (i < sg.n) sg.dst[i] = __fdiv_rn(1.0f, sg.src[i]);
}

template <int DT>
hipError_t quant_small_dt(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                          int bits, hipStream_t s) {
    const dim3 grid((unsigned)n_units), block(kT);
    switch (bits) {
        case 2: k_quant_small<DT, 2><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        case 3: k_quant_small<DT, 3><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        case 4: k_quant_small<DT, 4><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        default: k_quant_small<DT, 8><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t quant_big_dt(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        int bits, hipStream_t s) {
    const dim3 grid((unsigned)n_units), block(kT);
    switch (bits) {
        case 2: k_quant_big<DT, 2><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        case 3: k_quant_big<DT, 3><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        case 4: k_quant_big<DT, 4><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
        default: k_quant_big<DT, 8><<<grid, block, 0, s>>>(mats, ubeg, nmat); break;
    }
    return hipGetLastError();
}

template <int ODT>
hipError_t dequant_dt(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                      int bits, hipStream_t s) {
    const dim3 grid((unsigned)n_units), block(kT);
    const int zdef = (1 << (bits - 1)) - 1;
    switch (bits) {
        case 2: k_dequant<2, ODT><<<grid, block, 0, s>>>(mats, ubeg, nmat, zdef); break;
        case 3: k_dequant<3, ODT><<<grid, block, 0, s>>>(mats, ubeg, nmat, zdef); break;
        case 4: k_dequant<4, ODT><<<grid, block, 0, s>>>(mats, ubeg, nmat, zdef); break;
        default: k_dequant<8, ODT><<<grid, block, 0, s>>>(mats, ubeg, nmat, zdef); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t recip(const RecipSeg* segs, const int64_t* ubeg, int nseg, int64_t n_units,
                 hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_recip<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(segs, ubeg, nseg);
    return hipGetLastError();
}

hipError_t quant_small(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                       int dtype, int bits, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    return dtype == WOQ_BF16 ? quant_small_dt<WOQ_BF16>(mats, ubeg, nmat, n_units, bits, s)
                             : quant_small_dt<WOQ_F32>(mats, ubeg, nmat, n_units, bits, s);
}

hipError_t quant_big(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     int dtype, int bits, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    return dtype == WOQ_BF16 ? quant_big_dt<WOQ_BF16>(mats, ubeg, nmat, n_units, bits, s)
                             : quant_big_dt<WOQ_F32>(mats, ubeg, nmat, n_units, bits, s);
}

hipError_t dequant(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                   int out_dtype, int bits, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    return out_dtype == WOQ_BF16 ? dequant_dt<WOQ_BF16>(mats, ubeg, nmat, n_units, bits, s)
                                 : dequant_dt<WOQ_F32>(mats, ubeg, nmat, n_units, bits, s);
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

}  // namespace woq
