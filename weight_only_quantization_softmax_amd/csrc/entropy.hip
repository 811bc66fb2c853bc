// EWQ softmax entropy of each weight matrix, block entropies and tiers.
//
// [EWQ] "Giai ma EWQ & FastEWQ" (2kvn.com), section "EWQ hoat dong nhu the
// nao?": step 1 flattens each matrix, softmaxes it and takes its Shannon
// entropy; a block's entropy is the size-weighted mean; step 2 sorts blocks,
// takes mu_H and sigma_H and tiers them against T = mu_H - X sigma_H.
//
// With c = max w, S = sum e^{w-c} and U = sum e^{w-c} (w - c), the entropy
// is H = ln S - U / S (since ln p = (w - c) - ln S).
//
// bf16 path: a bf16 weight has only 65,536 bit patterns, so S and U are sums
// over the distinct values weighted by exact integer counts.  One HBM pass
// counts occurrences: patterns whose magnitude lies in a 32-binade window
// ([2^-26, 2^6), where trained and synthetic weights live) go to an 8192-bin
// LDS histogram; the rest (zeros, tiny, huge, inf/nan) go straight to the
// matrix's global 65,536-bin histogram.  A second small kernel evaluates the
// fp64 sums over the non-empty bins.  Results are exact up to fp64 rounding
// and independent of scheduling (integer counts).
//
// fp32 path: two passes (max, then fp64 sums of exp(w - c) per work unit),
// partials combined in a fixed order.
//
// The histogram also gives each bf16 matrix's exponent histogram (the counts
// of its 256 exponent fields) for the lossless exponent code of the kept
// blocks, summed per part when the caller asks for it.
//
// A work unit is kEntChunk consecutive elements of a contiguous matrix, or
// rpu whole rows of a strided one (row stride ld > cols).  Non-finite
// weights (NaN, +-inf) make the entropy NaN and are counted into the
// caller's uint64 counter: for bf16 from the histogram bins with an all-ones
// exponent, for fp32 in the max pass.
#include "launch.h"

#include <math.h>
#include <string.h>

namespace woq {
namespace {

constexpr int kT = 256;
constexpr uint32_t kWinLo = 101u << 7;  // |w| bits in [101<<7, 133<<7)
constexpr int kWinBins = 8192;          // 2 signs x 32 binades x 128 mantissas

__device__ __forceinline__ void hist_one(uint32_t h, uint32_t* lh, uint32_t* gh) {
    const uint32_t t = (h & 0x7fffu) - kWinLo;
    if (t < 4096u) {
        __hip_atomic_fetch_add(&lh[t | ((h >> 3) & 0x1000u)], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        __hip_atomic_fetch_add(&gh[h], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void hist8(const uint4 v, uint32_t* lh, uint32_t* gh) {
    hist_one(v.x & 0xffffu, lh, gh); hist_one(v.x >> 16, lh, gh);
    hist_one(v.y & 0xffffu, lh, gh); hist_one(v.y >> 16, lh, gh);
    hist_one(v.z & 0xffffu, lh, gh); hist_one(v.z >> 16, lh, gh);
    hist_one(v.w & 0xffffu, lh, gh); hist_one(v.w >> 16, lh, gh);
}

__global__ __launch_bounds__(kT) void k_hist_bf16(const EntMat* __restrict__ mats,
                                                  const int64_t* __restrict__ ubeg,
                                                  int nmat, int64_t u0,
                                                  uint32_t* __restrict__ ghist) {
    __shared__ uint32_t lh[kWinBins];
    for (int i = threadIdx.x; i < kWinBins; i += kT) lh[i] = 0;
    __syncthreads();

    const int64_t u = u0 + blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const EntMat em = mats[m];
    uint32_t* gh = ghist + (size_t)m * 65536;
    if (em.rpu == 0) {
        const int64_t start = (u - ubeg[m]) * kEntChunk;
        const int64_t cnt = min(kEntChunk, em.n - start);
        const uint16_t* p = reinterpret_cast<const uint16_t*>(em.data) + start;
        const uint4* pv = reinterpret_cast<const uint4*>(p);
        const int64_t nv = cnt >> 3;

        int64_t i = threadIdx.x;
        for (; i + 3 * kT < nv; i += 4 * kT) {
            const uint4 a = pv[i], b = pv[i + kT], c = pv[i + 2 * kT], d = pv[i + 3 * kT];
            hist8(a, lh, gh); hist8(b, lh, gh); hist8(c, lh, gh); hist8(d, lh, gh);
        }
        for (; i < nv; i += kT) hist8(pv[i], lh, gh);
        for (int64_t e = nv * 8 + threadIdx.x; e < cnt; e += kT) hist_one(p[e], lh, gh);
    } else {
        // rows [r0, r1) of a strided matrix (cols % 8 == 0): vector idx of the
        // unit is row r0 + idx / vpr, columns 8 (idx % vpr) ..
        const int r0 = (int)(u - ubeg[m]) * em.rpu;
        const int r1 = min(em.rows, r0 + em.rpu);
        const uint32_t vpr = (uint32_t)(em.cols >> 3);
        const uint32_t nvu = (uint32_t)(r1 - r0) * vpr;
        const uint16_t* base = reinterpret_cast<const uint16_t*>(em.data);
        for (uint32_t idx = threadIdx.x; idx < nvu; idx += kT) {
            const uint32_t r = idx / vpr, v = idx - r * vpr;
            hist8(*reinterpret_cast<const uint4*>(base + (int64_t)(r0 + r) * em.ld + 8 * v), lh, gh);
        }
    }
    __syncthreads();

    for (int b = threadIdx.x; b < kWinBins; b += kT) {
        const uint32_t c = lh[b];
        if (c) {
            const uint32_t bits = ((uint32_t)(b >> 12) << 15) | ((uint32_t)(b & 4095) + kWinLo);
            __hip_atomic_fetch_add(&gh[bits], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Block-wide reductions for kT threads; every thread gets the result.
__device__ __forceinline__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) r += sh[w];
    return r;
}

__device__ __forceinline__ float block_maxf(float v, float* sh) {
    v = wave_maxf(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) r = fmaxf(r, sh[w]);
    return r;
}

// The 65,536 bins of a matrix are split into kHistParts parts of 4096 bins.
// Part w takes the largest finite non-empty value c_w of its bins and sums,
// relative to it, S_w = sum n_v e^{v - c_w} and U_w = sum n_v e^{v - c_w}
// (v - c_w) in fp64.  The combine rescales to the matrix maximum c:
//   S = sum_w S_w e^{c_w - c},  U = sum_w (U_w + (c_w - c) S_w) e^{c_w - c},
// so H = ln S - U / S exactly as from one pass (up to fp64 rounding).
constexpr int kHistParts = kHistBinParts;
constexpr int kPartBins = 65536 / kHistParts;

__global__ __launch_bounds__(kT) void k_hist_part(const EntMat* __restrict__ mats,
                                                  const uint32_t* __restrict__ ghist,
                                                  double4* __restrict__ part,
                                                  uint32_t* __restrict__ exp_hist) {
    __shared__ double shd[kT / 64];
    __shared__ float shf[kT / 64];
    __shared__ uint32_t lexp[32];
    const int m = blockIdx.x / kHistParts, w = blockIdx.x % kHistParts;
    const uint32_t* gh = ghist + (size_t)m * 65536 + (size_t)w * kPartBins;
    constexpr int PER = kPartBins / kT;
    uint32_t cnt[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt[i] = gload<uint32_t>(gh + threadIdx.x + kT * i);
    if (exp_hist) {
        // the part holds one sign and 32 exponent fields (128 mantissas
        // each): bin threadIdx.x + kT i has exponent 32 (w % 8) + 2 i +
        // threadIdx.x / 128
        if (threadIdx.x < 32) lexp[threadIdx.x] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (cnt[i]) atomicAdd(&lexp[2 * i + (threadIdx.x >> 7)], cnt[i]);
        __syncthreads();
        if (threadIdx.x < 32 && lexp[threadIdx.x])
            atomicAdd(exp_hist + (size_t)mats[m].slot * 256 + 32 * (w % 8) + threadIdx.x,
                      lexp[threadIdx.x]);
    }
    float mx = -INFINITY;
    double bad = 0.0;  // weights whose bin has an all-ones exponent (NaN, inf)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (cnt[i]) {
            const uint32_t b = (uint32_t)(w * kPartBins) + threadIdx.x + kT * i;
            const float v = __uint_as_float(b << 16);
            if (!isfinite(v)) bad += (double)cnt[i]; else mx = fmaxf(mx, v);
        }
    }
    mx = block_maxf(mx, shf);
    bad = block_sum(bad, shd);
    double S = 0.0, U = 0.0;
    const double c = (double)mx;
    if (mx > -INFINITY) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t b = (uint32_t)(w * kPartBins) + threadIdx.x + kT * i;
            const float v = __uint_as_float(b << 16);
            if (cnt[i] && isfinite(v)) {
                const double d = (double)v - c;
                const double e = (double)cnt[i] * exp(d);
                S += e;
                U += e * d;
            }
        }
    }
    S = block_sum(S, shd);
    U = block_sum(U, shd);
    if (threadIdx.x == 0) part[blockIdx.x] = make_double4(c, S, U, bad);
}

__global__ __launch_bounds__(kT) void k_hist_comb(const EntMat* __restrict__ mats, int nmat,
                                                  const double4* __restrict__ part,
                                                  double* __restrict__ h_mat,
                                                  unsigned long long* __restrict__ nonfinite) {
    const int m = blockIdx.x * kT + threadIdx.x;
    if (m >= nmat) return;
    const double4* p = part + (size_t)m * kHistParts;
    double c = -INFINITY, nbad = 0.0;
    for (int w = 0; w < kHistParts; ++w) {
        const double4 q = p[w];
        if (q.y > 0.0) c = fmax(c, q.x);
        nbad += q.w;  // integer counts below 2^31: exact in fp64
    }
    const bool bad = nbad != 0.0;
    if (bad) atomicAdd(nonfinite, (unsigned long long)nbad);
    double S = 0.0, U = 0.0;
    for (int w = 0; w < kHistParts; ++w) {
        const double4 q = p[w];
        if (q.y > 0.0) {
            const double f = exp(q.x - c);
            S += q.y * f;
            U += (q.z + (q.x - c) * q.y) * f;
        }
    }
    gstore<double>(h_mat + mats[m].slot, bad ? (double)NAN : log(S) - U / S);
}

// ---------------------------------------------------------------- fp32
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Calls f(value) for every element of work unit u of an fp32 matrix, thread
// t taking elements t, t + kT, ... of the unit.
template <class F>
__device__ __forceinline__ void f32_unit(const EntMat& em, int64_t ul, F&& f) {
    const float* base = reinterpret_cast<const float*>(em.data);
    if (em.rpu == 0) {
        const int64_t start = ul * kEntChunk;
        const int64_t cnt = min(kEntChunk, em.n - start);
        for (int64_t e = threadIdx.x; e < cnt; e += kT) f(base[start + e]);
    } else {
        const int r0 = (int)ul * em.rpu;
        const int r1 = min(em.rows, r0 + em.rpu);
        const uint32_t cols = (uint32_t)em.cols;
        const uint32_t ne = (uint32_t)(r1 - r0) * cols;
        for (uint32_t e = threadIdx.x; e < ne; e += kT) {
            const uint32_t r = e / cols, c = e - r * cols;
            f(base[(int64_t)(r0 + r) * em.ld + c]);
        }
    }
}

__global__ __launch_bounds__(kT) void k_f32_max(const EntMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat,
                                                uint32_t* __restrict__ keys,
                                                unsigned long long* __restrict__ nonfinite) {
    __shared__ float shf[kT / 64];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const EntMat em = mats[m];
    float mx = -INFINITY;
    uint32_t nbad = 0;
    f32_unit(em, u - ubeg[m], [&](float v) {
        if (!isfinite(v)) ++nbad; else mx = fmaxf(mx, v);
    });
    if (nbad) atomicAdd(nonfinite, (unsigned long long)nbad);
    mx = block_maxf(mx, shf);
    const float bad = block_maxf(nbad ? 1.f : 0.f, shf);
    if (threadIdx.x == 0) {
        atomicMax(&keys[2 * m], order_key(mx));
        if (bad != 0.f) atomicOr(&keys[2 * m + 1], 1u);
    }
}

__global__ __launch_bounds__(kT) void k_f32_sum(const EntMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat,
                                                const uint32_t* __restrict__ keys,
                                                double2* __restrict__ part) {
    __shared__ double shd[kT / 64];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const EntMat em = mats[m];
    const double c = (double)key_value(keys[2 * m]);
    double S = 0.0, U = 0.0;
    f32_unit(em, u - ubeg[m], [&](float v) {
        if (isfinite(v)) {
            const double d = (double)v - c;
            const double x = exp(d);
            S += x;
            U += x * d;
        }
    });
    S = block_sum(S, shd);
    U = block_sum(U, shd);
    if (threadIdx.x == 0) part[u] = make_double2(S, U);
}

__global__ void k_f32_final(const EntMat* __restrict__ mats, const int64_t* __restrict__ ubeg,
                            int nmat, const uint32_t* __restrict__ keys,
                            const double2* __restrict__ part, double* __restrict__ h_mat) {
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= nmat) return;
    double S = 0.0, U = 0.0;
    for (int64_t u = ubeg[m]; u < ubeg[m + 1]; ++u) { S += part[u].x; U += part[u].y; }
    h_mat[mats[m].slot] = keys[2 * m + 1] ? (double)NAN : log(S) - U / S;
}

// ---------------------------------------------------------------- blocks
__global__ __launch_bounds__(kT) void k_blocks(const int32_t* __restrict__ bmats,
                                               const int32_t* __restrict__ bbeg,
                                               const double* __restrict__ nsz,
                                               const double* __restrict__ h_mat, int nb,
                                               double x, double* __restrict__ hb,
                                               double* __restrict__ h_block,
                                               double* __restrict__ stats,
                                               int32_t* __restrict__ tier,
                                               int32_t* __restrict__ order) {
    __shared__ double shd[kT / 64];
    for (int b = threadIdx.x; b < nb; b += kT) {
        double num = 0.0, den = 0.0;
        for (int i = bbeg[b]; i < bbeg[b + 1]; ++i) {
            const int m = bmats[i];
            num += nsz[m] * h_mat[m];
            den += nsz[m];
        }
        const double h = num / den;
        hb[b] = h;
        if (h_block) h_block[b] = h;
    }
    __syncthreads();
    double acc = 0.0;
    for (int b = threadIdx.x; b < nb; b += kT) acc += hb[b];
    const double mu = block_sum(acc, shd) / nb;
    acc = 0.0;
    for (int b = threadIdx.x; b < nb; b += kT) { const double d = hb[b] - mu; acc += d * d; }
    const double sigma = sqrt(block_sum(acc, shd) / nb);
    const double t = mu - x * sigma;
    if (stats && threadIdx.x == 0) { stats[0] = mu; stats[1] = sigma; stats[2] = t; }
    for (int b = threadIdx.x; b < nb; b += kT) {
        const double h = hb[b];
        if (tier) tier[b] = (h <= t) ? 1 : ((h < mu) ? 2 : 3);
        if (order) {
            int rank = 0;
            for (int o = 0; o < nb; ++o) {
                const double g = hb[o];
                rank += (g < h) || (g == h && o < b);
            }
            order[rank] = b;
        }
    }
}

// Copies one chunk of bytes carried in the kernel's arguments (the staging
// path for calls captured into a graph: a captured kernel keeps its
// arguments by value, a copy from pageable host memory would not).
struct StageChunk {
    uint32_t w[kStageChunk / 4];
};
__global__ __launch_bounds__(256) void k_stage(uint32_t* dst, uint32_t nw, StageChunk c) {
    for (uint32_t i = threadIdx.x; i < nw; i += 256) dst[i] = c.w[i];
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

hipError_t fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = min((n + 255) / 256, (size_t)4096);
    k_fill_u32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n, v);
    return hipGetLastError();
}

hipError_t stage_bytes(void* dst, const void* src, size_t n, hipStream_t s) {
    for (size_t off = 0; off < n; off += kStageChunk) {
        StageChunk c;
        const size_t m = n - off < (size_t)kStageChunk ? n - off : (size_t)kStageChunk;
        memset(&c, 0, sizeof(c));
        memcpy(c.w, static_cast<const char*>(src) + off, m);
        k_stage<<<dim3(1), dim3(256), 0, s>>>(
            reinterpret_cast<uint32_t*>(static_cast<char*>(dst) + off), (uint32_t)(m / 4), c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t fill_f32(float* p, size_t n, float v, hipStream_t s) {
    uint32_t bits;
    memcpy(&bits, &v, sizeof(bits));
    return fill_u32(reinterpret_cast<uint32_t*>(p), n, bits, s);
}

hipError_t ent_hist_bf16(const EntMat* mats, const int64_t* ubeg, int nmat, int64_t u0,
                         int64_t n_units, uint32_t* ghist, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_hist_bf16<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, u0, ghist);
    return hipGetLastError();
}

hipError_t ent_hist_final(const EntMat* mats, int nmat, const uint32_t* ghist, double4* part,
                          double* h_mat, unsigned long long* nonfinite, uint32_t* exp_hist,
                          hipStream_t s) {
    if (nmat <= 0) return hipSuccess;
    k_hist_part<<<dim3(nmat * kHistParts), dim3(kT), 0, s>>>(mats, ghist, part, exp_hist);
    k_hist_comb<<<dim3((nmat + kT - 1) / kT), dim3(kT), 0, s>>>(mats, nmat, part, h_mat, nonfinite);
    return hipGetLastError();
}

hipError_t ent_f32(const EntMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                   uint32_t* keys, double2* part, double* h_mat, unsigned long long* nonfinite,
                   hipStream_t s) {
    if (nmat <= 0) return hipSuccess;
    hipError_t e = fill_u32(keys, 2 * (size_t)nmat, 0u, s);
    if (e != hipSuccess) return e;
    k_f32_max<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, keys, nonfinite);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_f32_sum<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, keys, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_f32_final<<<dim3((nmat + 63) / 64), dim3(64), 0, s>>>(mats, ubeg, nmat, keys, part, h_mat);
    return hipGetLastError();
}

hipError_t ent_blocks(const int32_t* bmats, const int32_t* bbeg, const double* nsz,
                      const double* h_mat, int n_blocks, double x, double* hb,
                      double* h_block, double* stats, int32_t* tier, int32_t* order,
                      hipStream_t s) {
    k_blocks<<<dim3(1), dim3(kT), 0, s>>>(bmats, bbeg, nsz, h_mat, n_blocks, x, hb, h_block,
                                           stats, tier, order);
    return hipGetLastError();
}

}  // namespace woq
