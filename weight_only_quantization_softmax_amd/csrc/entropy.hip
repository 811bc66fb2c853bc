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
// (k_hist_bf16, one workgroup per work unit) counts them: patterns whose
// magnitude lies in a 31-binade window ([2^-25, 2^6), where trained and
// synthetic weights live) in a 7,936-bin LDS histogram, added at the end to
// the matrix's window record; zeros and NaN / inf are counted; every other
// value (tiny, subnormal, |w| >= 64: rare) is appended to the matrix's list
// as its bit pattern.  A unit that meets more such values than its LDS list
// holds, or a matrix whose list fills, is marked spilled, and the final
// kernel recounts that matrix's other values from the weights (sixteen
// re-reads, each counting a sixteenth of the pattern space in LDS) - slow,
// and only for matrices full of values far outside the window.  The final
// kernel (k_hist_final, one workgroup per matrix) evaluates the fp64 sums
// over the window bins, the zeros and the sorted list.  Results are exact
// up to fp64 rounding and independent of scheduling (integer counts, sums
// in a fixed order).  A matrix needs a 32 KB record and a 16 KB list, not
// a 256 KB histogram, so the matrices of a whole model share one launch.
//
// fp32 path: one pass per work unit (a running maximum with fp64 sums of
// exp(w - m), rescaled when the maximum grows), the units' partials
// combined in a fixed order.
//
// The counts also give each bf16 matrix's exponent histogram (the counts
// of its 256 exponent fields) for the lossless exponent code of the kept
// blocks, when the caller asks for it.
//
// An fp32 work unit is an equal share (a multiple of 8 elements, between
// kEntMinChunk and kEntChunk) of a contiguous matrix, or rpu whole rows of a
// strided one (row stride ld > cols).  Non-finite weights (NaN, +-inf) make the entropy NaN and are
// counted into the caller's uint64 counter: for bf16 in the counting pass,
// for fp32 in the one pass.
#include "launch.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

namespace woq {
namespace {

constexpr int kT = 256;
// Monotone unsigned key of a float (larger value, larger key; never 0 for
// a non-NaN value), and its inverse.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- bf16
// Window: bf16 patterns whose magnitude bits lie in [kWinLo, kWinLo +
// kWinSpan), exponent fields 102..132 (|w| in [2^-25, 2^6)).  Window
// pattern h has bin (|h| - kWinLo) | sign << 12, in LDS and in the
// matrix's record alike (bins 3968..4095 of each sign unused).
constexpr uint32_t kWinLo = 102u << 7;
constexpr uint32_t kWinSpan = 31u << 7;
constexpr int kWinBins = 4096 + (int)kWinSpan;   // 8064
// LDS of the counting kernel: the window, then kExtra words: [0] +0 count,
// [1] -0 count, [2] non-finite count, [3] order key of the largest other
// value, [4] number of other values, [5] broadcast, then up to kLdsList
// other values as 16-bit patterns.  32 KiB in all.
constexpr int kExtra = 128;
constexpr uint32_t kLdsList = 2 * (kExtra - 8);  // 240
static_assert((kWinBins + kExtra) * 4 == 32768, "LDS of k_hist_bf16");
static_assert(kWinBins % 2 == 0, "bins are added in pairs");
// A matrix's record: the window counts, then kRecHdr words: [0..3] as the
// LDS words, [4] values appended to the matrix's list, [5] spilled flag.
constexpr int kRecHdr = 64;
constexpr int kRecWords = kWinBins + kRecHdr;
static_assert(kRecWords == kEntRecWords, "record size");
constexpr uint32_t kListCap = (uint32_t)kEntListCap;

// Values outside the window: zeros and non-finite values are counted; any
// other value (tiny, subnormal or |w| >= 64) is kept as its pattern, and
// the largest is tracked.
__device__ __forceinline__ void hist_other(uint32_t h, uint32_t* ex) {
    const uint32_t a = h & 0x7fffu;
    if (a == 0) {
        __hip_atomic_fetch_add(&ex[h >> 15], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else if (a >= 0x7f80u) {
        __hip_atomic_fetch_add(&ex[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        __hip_atomic_fetch_max(&ex[3], order_key(__uint_as_float(h << 16)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t i =
            __hip_atomic_fetch_add(&ex[4], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (i < kLdsList) reinterpret_cast<uint16_t*>(ex + 8)[i] = (uint16_t)h;
    }
}

__device__ __forceinline__ void hist_one(uint32_t h, uint32_t* lh, uint32_t* ex) {
    const uint32_t t = (h & 0x7fffu) - kWinLo;
    if (t < kWinSpan)
        __hip_atomic_fetch_add(&lh[t | ((h >> 3) & 0x1000u)], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    else
        hist_other(h, ex);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Eight patterns (two per word).  Both halves of a word are tested at once
// with 16-bit packed integer arithmetic: t = |h| - kWinLo (mod 2^16) is
// below kWinSpan exactly for window patterns, and t | sign << 12 is the
// bin.  One branch per eight patterns: when all eight are in the window
// (nearly always) each takes one LDS add; otherwise each goes through
// hist_one.
__device__ __forceinline__ void hist8(const uint4 v, uint32_t* lh, uint32_t* ex) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const u16x2 lo = {(unsigned short)kWinLo, (unsigned short)kWinLo};
    uint32_t bin[4];
    u16x2 mx = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u16x2 t = __builtin_bit_cast(u16x2, w[k] & 0x7fff7fffu) - lo;
        mx = __builtin_elementwise_max(mx, t);
        bin[k] = __builtin_bit_cast(uint32_t, t) | ((w[k] >> 3) & 0x10001000u);
    }
    if (max((uint32_t)mx.x, (uint32_t)mx.y) < kWinSpan) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            __hip_atomic_fetch_add(&lh[bin[k] & 0xffffu], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(&lh[bin[k] >> 16], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hist_one(w[k] & 0xffffu, lh, ex);
            hist_one(w[k] >> 16, lh, ex);
        }
    }
}

// Number of 16-byte vectors of a bf16 matrix: ceil(n / 8) when contiguous
// (the last one may be partial), rows * cols / 8 when strided.
__device__ __forceinline__ int64_t bf16_vectors(const EntMat& em) {
    return em.ld == em.cols ? (em.n + 7) >> 3 : (int64_t)em.rows * (em.cols >> 3);
}

// Calls f(v) for each full 8-pattern vector of vectors [a, b) of a bf16
// matrix and g(h) for each pattern of a partial last vector (thread t takes
// vectors a + t, a + t + kT, ...).
template <class F, class G>
__device__ __forceinline__ void bf16_vecs(const EntMat& em, int64_t a, int64_t b, F&& f, G&& g) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(em.data);
    if (em.ld == em.cols) {
        const int64_t nfull = em.n >> 3;
        const int64_t bf = min(b, nfull);
        int64_t i = a + threadIdx.x;
        for (; i + 3 * kT < bf; i += 4 * kT) {
            const uint4 v0 = gload_u4(base + 8 * i), v1 = gload_u4(base + 8 * (i + kT)),
                        v2 = gload_u4(base + 8 * (i + 2 * kT)), v3 = gload_u4(base + 8 * (i + 3 * kT));
            f(v0); f(v1); f(v2); f(v3);
        }
        for (; i < bf; i += kT) f(gload_u4(base + 8 * i));
        if (b > nfull)
            for (int64_t e = 8 * nfull + threadIdx.x; e < em.n; e += kT)
                g((uint32_t)gload<uint16_t>(base + e));
    } else {
        // strided (cols % 8 == 0): vector idx is row idx / vpr, columns
        // 8 (idx % vpr) ..
        const uint32_t vpr = (uint32_t)(em.cols >> 3);
        for (uint32_t idx = (uint32_t)a + threadIdx.x; idx < (uint32_t)b; idx += kT) {
            const uint32_t r = idx / vpr, v = idx - r * vpr;
            f(gload_u4(base + (int64_t)r * em.ld + 8 * v));
        }
    }
}

// Adds a segment's LDS counts to matrix m's record and its other values to
// the matrix's list (or marks the matrix spilled when they do not fit).
// Called by the whole workgroup after a barrier.
__device__ __forceinline__ void hist_flush(const uint32_t* lh, uint32_t* ex, uint32_t* rec,
                                           uint16_t* list) {
    uint32_t* hdr = rec + kWinBins;
    // two bins per 64-bit add (a matrix's counts stay below 2^31, so no
    // carry crosses into the upper bin)
    const unsigned long long* lh2 = reinterpret_cast<const unsigned long long*>(lh);
    unsigned long long* rec2 = reinterpret_cast<unsigned long long*>(rec);
    for (int b = threadIdx.x; b < kWinBins / 2; b += kT) {
        const unsigned long long c = lh2[b];
        if (c) __hip_atomic_fetch_add(&rec2[b], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x < 3 && ex[threadIdx.x])
        __hip_atomic_fetch_add(&hdr[threadIdx.x], ex[threadIdx.x], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 3 && ex[3])
        __hip_atomic_fetch_max(&hdr[3], ex[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t n = ex[4];   // the same for every thread
    if (n == 0) return;
    if (n > kLdsList) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(&hdr[5], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (threadIdx.x == 0)
        ex[5] = __hip_atomic_fetch_add(&hdr[4], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t pos = ex[5];
    if (pos + n > kListCap) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(&hdr[5], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const uint16_t* ll = reinterpret_cast<const uint16_t*>(ex + 8);
    for (uint32_t i = threadIdx.x; i < n; i += kT) list[pos + i] = ll[i];
}

// The counting pass over all bf16 matrices of a batch, as one sequence of
// vectors (vbeg[m] = first vector of matrix m; vbeg[nmat] - vbeg[0] = the
// total).  Workgroup g takes an equal share, [vbeg[0] + V g / G, vbeg[0] +
// V (g + 1) / G) with G = gridDim.x, a few times the workgroups the GPU
// holds at once: every workgroup streams the same number of bytes, and a
// matrix segment costs one clearing of the LDS counts and one flush.
__global__ __launch_bounds__(kT) void k_hist_bf16(const EntMat* __restrict__ mats,
                                                  const int64_t* __restrict__ vbeg, int nmat,
                                                  uint32_t* __restrict__ recs,
                                                  uint16_t* __restrict__ lists) {
    __shared__ __align__(8) uint32_t lh[kWinBins + kExtra];
    uint32_t* ex = lh + kWinBins;
    const int64_t V = vbeg[nmat] - vbeg[0];
    const int64_t v0 = vbeg[0] + V * (int64_t)blockIdx.x / gridDim.x;
    const int64_t v1 = vbeg[0] + V * (int64_t)(blockIdx.x + 1) / gridDim.x;
    if (v0 >= v1) return;
    int m = find_unit_owner(vbeg, nmat, v0);
    for (int64_t v = v0; v < v1; ++m) {
        const int64_t mb = vbeg[m];
        const int64_t e = min(v1, vbeg[m + 1]);
        for (int i = threadIdx.x; i < kWinBins + 8; i += kT) lh[i] = 0;
        __syncthreads();
        const EntMat em = mats[m];
        bf16_vecs(em, v - mb, e - mb, [&](const uint4 x) { hist8(x, lh, ex); },
                  [&](uint32_t h) { hist_one(h, lh, ex); });
        __syncthreads();
        hist_flush(lh, ex, recs + (size_t)m * kRecWords, lists + (size_t)m * kListCap);
        __syncthreads();
        v = e;
    }
}

// Block-wide reductions for NT threads; every thread gets the result.
template <int NT = kT>
__device__ __forceinline__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) r += sh[w];
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

__device__ __forceinline__ float win_value(int b) {
    const uint32_t h = ((uint32_t)(b >> 12) << 15) | ((uint32_t)(b & 4095) + kWinLo);
    return __uint_as_float(h << 16);
}

// Adds n e^{v - c} to S and n e^{v - c} (v - c) to U (fp64).
__device__ __forceinline__ void add_term(double n, float v, double c, double& S, double& U) {
    const double d = (double)v - c;
    const double e = n * exp(d);
    S += e;
    U += e * d;
}

// One workgroup per matrix: c = the largest finite value (window bins,
// the largest other value, zeros), then S = sum_v n_v e^{v - c} and U =
// sum_v n_v e^{v - c} (v - c) in fp64 over the window bins (bin order), the
// zeros, and the other values: from the list sorted by pattern, or, when
// the matrix spilled, from sixteen re-reads of the matrix that each count
// the other values of one sixteenth of the pattern space in LDS.  H = ln S -
// U / S, NaN when the matrix holds a non-finite value.  Every sum has a
// fixed order, so the result does not depend on scheduling.
__global__ __launch_bounds__(kT) void k_hist_final(const EntMat* __restrict__ mats,
                                                   const uint32_t* __restrict__ recs,
                                                   const uint16_t* __restrict__ lists,
                                                   double* __restrict__ h_mat,
                                                   unsigned long long* __restrict__ nonfinite,
                                                   uint32_t* __restrict__ exp_hist) {
    __shared__ double shd[kT / 64];
    __shared__ float shf[kT / 64];
    __shared__ uint32_t lexp[256];
    __shared__ uint32_t big[4096];   // the sorted list (16-bit) or one sixteenth's counts
    const int m = blockIdx.x;
    const EntMat em = mats[m];
    const uint32_t* rec = recs + (size_t)m * kRecWords;
    const uint32_t* hdr = rec + kWinBins;
    const uint32_t zp = hdr[0], zn = hdr[1], nf = hdr[2], mk = hdr[3], nl = hdr[4];
    const bool spilled = hdr[5] != 0 || nl > kListCap;
    // thread t holds the 32 consecutive bins [32 t, 32 t + 32): one
    // exponent field, wholly inside or outside the window's used bins
    constexpr int PER = 32;
    static_assert(kWinBins <= PER * kT && kWinSpan % PER == 0, "bin ownership");
    const int b0 = PER * threadIdx.x;
    const bool own = b0 < kWinBins && (uint32_t)(b0 & 4095) < kWinSpan;
    uint32_t cnt[PER];
    if (own) {
#pragma unroll
        for (int i = 0; i < PER / 4; ++i) {
            const uint4 v = gload_u4(rec + b0 + 4 * i);
            cnt[4 * i] = v.x; cnt[4 * i + 1] = v.y; cnt[4 * i + 2] = v.z; cnt[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) cnt[i] = 0u;
    }
    float mx = -INFINITY;
    uint32_t tot = 0;   // the thread's count (< 2^31: one matrix)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (cnt[i]) mx = fmaxf(mx, win_value(b0 + i));
        tot += cnt[i];
    }
    if (threadIdx.x == 0) {
        if (mk) mx = fmaxf(mx, key_value(mk));
        if (zp + zn) mx = fmaxf(mx, 0.0f);
    }
    if (exp_hist) {
        lexp[threadIdx.x] = 0;
        __syncthreads();
        if (tot) atomicAdd(&lexp[102 + ((b0 & 4095) >> 7)], tot);
        if (threadIdx.x == 0) {
            atomicAdd(&lexp[0], zp + zn);
            atomicAdd(&lexp[255], nf);
        }
    }
    const double c = (double)block_maxf(mx, shf);
    double S = 0.0, U = 0.0;
    if (c > -INFINITY) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (cnt[i]) add_term((double)cnt[i], win_value(b0 + i), c, S, U);
        if (threadIdx.x == 0 && zp + zn) add_term((double)(zp + zn), 0.0f, c, S, U);
    }
    if (!spilled && nl) {
        // sort the list (bitonic, padded to a power of two with 0xffff,
        // a pattern the list never holds), then thread t takes sorted
        // entries t, t + kT, ...
        uint16_t* s = reinterpret_cast<uint16_t*>(big);
        uint32_t n2 = 2;
        while (n2 < nl) n2 <<= 1;
        const uint16_t* src = lists + (size_t)m * kListCap;
        for (uint32_t i = threadIdx.x; i < n2; i += kT) s[i] = i < nl ? src[i] : (uint16_t)0xffff;
        __syncthreads();
        for (uint32_t k = 2; k <= n2; k <<= 1) {
            for (uint32_t j = k >> 1; j > 0; j >>= 1) {
                for (uint32_t i = threadIdx.x; i < n2; i += kT) {
                    const uint32_t l = i ^ j;
                    if (l > i) {
                        const uint16_t a = s[i], b = s[l];
                        if ((a > b) == ((i & k) == 0)) { s[i] = b; s[l] = a; }
                    }
                }
                __syncthreads();
            }
        }
        for (uint32_t i = threadIdx.x; i < nl; i += kT) {
            const uint32_t h = s[i];
            add_term(1.0, __uint_as_float(h << 16), c, S, U);
            if (exp_hist) atomicAdd(&lexp[(h >> 7) & 0xffu], 1u);
        }
    } else if (spilled) {
        for (uint32_t r = 0; r < 16; ++r) {
            __syncthreads();
            for (int i = threadIdx.x; i < 4096; i += kT) big[i] = 0;
            __syncthreads();
            auto one = [&](uint32_t h) {
                const uint32_t a = h & 0x7fffu;
                if ((h >> 12) == r && a - kWinLo >= kWinSpan && a != 0 && a < 0x7f80u)
                    atomicAdd(&big[h & 4095u], 1u);
            };
            bf16_vecs(em, 0, bf16_vectors(em),
                      [&](const uint4 v) {
                          one(v.x & 0xffffu); one(v.x >> 16); one(v.y & 0xffffu); one(v.y >> 16);
                          one(v.z & 0xffffu); one(v.z >> 16); one(v.w & 0xffffu); one(v.w >> 16);
                      },
                      one);
            __syncthreads();
            for (int i = threadIdx.x; i < 4096; i += kT) {
                const uint32_t n = big[i];
                if (n) {
                    const uint32_t h = (r << 12) | (uint32_t)i;
                    add_term((double)n, __uint_as_float(h << 16), c, S, U);
                    if (exp_hist) atomicAdd(&lexp[(h >> 7) & 0xffu], n);
                }
            }
        }
    }
    S = block_sum(S, shd);
    U = block_sum(U, shd);
    if (exp_hist) {
        __syncthreads();
        gstore<uint32_t>(exp_hist + (size_t)em.slot * 256 + threadIdx.x, lexp[threadIdx.x]);
    }
    if (threadIdx.x == 0) {
        if (nf) atomicAdd(nonfinite, (unsigned long long)nf);
        gstore<double>(h_mat + em.slot, nf ? (double)NAN : log(S) - U / S);
    }
}

// ---------------------------------------------------------------- fp32

// exp(x) for x <= 0 in fp64, by Tang's table-driven method (P. T. P. Tang,
// ACM TOMS 15(2), 1989): x = (64 M + j) ln2 / 64 + r with |r| <= ln2 / 128,
// exp(x) = 2^M 2^(j/64) exp(r), exp(r) - 1 by its Taylor series to r^5
// (the next term is below 4e-17 relative), 2^(j/64) from a 64-entry table
// (tab, in LDS).  ln2 / 64 is split into a 36-bit head, exact when
// multiplied by |n| < 2^17, and a tail.  x is clamped to -746 first (exp
// below that is 0 in fp64), so n stays small.  About 1 ulp from exp.
__device__ __forceinline__ double exp_nonpos(double x, const double* tab) {
    constexpr double kInvLn2x64 = 0x1.71547652b82fep+6;    // 64 / ln 2
    constexpr double kLn2d64Hi = 0x1.62e42fefa0000p-7;     // ln 2 / 64, head
    constexpr double kLn2d64Lo = 0x1.cf79abc9e3b3ap-46;    // ln 2 / 64, tail
    x = fmax(x, -746.0);
    const double n = rint(x * kInvLn2x64);
    const int ni = (int)n;
    const double r = fma(-n, kLn2d64Lo, fma(-n, kLn2d64Hi, x));
    double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p *= r;
    const double t = tab[ni & 63];
    return ldexp(fma(t, p, t), ni >> 6);
}

// Running sums of one thread over fp32 values: the largest finite value mx
// met so far, S = sum exp(w - mx) and U = sum exp(w - mx) (w - mx) over the
// finite values, nbad the NaN / inf values.  Values arrive in batches: the
// batch's maximum first, the sums moved to it when it is larger
// (exp(w - m') = exp(w - m) exp(m - m')), then one exponential per value.
struct F32Acc {
    const double* tab;   // 2^(j/64), j < 64, for exp_nonpos
    float mx = -INFINITY;
    double S = 0.0, U = 0.0;
    uint32_t nbad = 0;

    __device__ __forceinline__ void rebase(float m) {
        if (S != 0.0) {
            const double d = (double)mx - (double)m;   // <= 0
            const double r = exp_nonpos(d, tab);
            U = r * (U + S * d);
            S = r * S;
        }
        mx = m;
    }
    template <int K>
    __device__ __forceinline__ void add(const float (&v)[K]) {
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (isfinite(v[i])) bm = fmaxf(bm, v[i]);
            else ++nbad;
        }
        if (bm > mx) rebase(bm);
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (isfinite(v[i])) {
                const double d = (double)v[i] - (double)mx;
                const double x = exp_nonpos(d, tab);
                S += x;
                U += x * d;
            }
        }
    }
};

__device__ __forceinline__ void f32_load4(const float* p, bool vec, float* v) {
    if (vec) {
        const float4 a = gload_f4(p);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
        v[0] = p[0]; v[1] = p[1]; v[2] = p[2]; v[3] = p[3];
    }
}

// Thread t's groups of work unit ul: group g is 4 consecutive elements of a
// row at addr(g); the thread takes g = t, t + kT, ... in that order, four
// groups per batch while they last.  vec: every group is 16-byte aligned.
template <class A>
__device__ __forceinline__ void f32_groups(int ng, bool vec, A&& addr, F32Acc& acc) {
    int g = threadIdx.x;
    for (; g + 3 * kT < ng; g += 4 * kT) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) f32_load4(addr(g + j * kT), vec, v + 4 * j);
        acc.add<16>(v);
    }
    for (; g < ng; g += kT) {
        float v[4];
        f32_load4(addr(g), vec, v);
        acc.add<4>(v);
    }
}

// Adds work unit ul of an fp32 matrix to acc.  A contiguous unit is `chunk`
// consecutive elements (a multiple of 8 but in the last unit); a strided one
// is rpu whole rows (cols a multiple of 8).  The order in which a thread
// meets its values depends only on the unit's rows and columns, not on the
// row stride or the alignment, so a strided view and its contiguous copy
// with the same units give the same sums.
__device__ __forceinline__ void f32_unit(const EntMat& em, int64_t ul, F32Acc& acc) {
    const float* base = reinterpret_cast<const float*>(em.data);
    if (em.rpu == 0) {
        const int64_t start = ul * em.chunk;
        const int cnt = (int)min(em.chunk, em.n - start);
        const float* p = base + start;
        const int ng = cnt >> 2;
        f32_groups(ng, (reinterpret_cast<uintptr_t>(p) & 15) == 0,
                   [&](int g) { return p + 4 * g; }, acc);
        const int e = 4 * ng + (int)threadIdx.x;
        if (e < cnt) {
            const float v[1] = {p[e]};
            acc.add<1>(v);
        }
    } else {
        const int r0 = (int)ul * em.rpu;
        const int r1 = min(em.rows, r0 + em.rpu);
        const uint32_t gpr = (uint32_t)em.cols >> 2;
        const float* p = base + (int64_t)r0 * em.ld;
        const int64_t ld = em.ld;
        f32_groups((int)((uint32_t)(r1 - r0) * gpr),
                   (reinterpret_cast<uintptr_t>(base) & 15) == 0 && (ld & 3) == 0,
                   [&](int g) {
                       const uint32_t r = (uint32_t)g / gpr, c = (uint32_t)g - r * gpr;
                       return p + (int64_t)r * ld + 4 * c;
                   },
                   acc);
    }
}

// One pass per work unit: each thread's running sums (F32Acc), moved to the
// unit's maximum and added in a fixed order.  part[3u .. 3u + 2] = (unit
// maximum, S, U); S is NaN when the unit holds a NaN or +-inf.
__global__ __launch_bounds__(kT) void k_f32_part(const EntMat* __restrict__ mats,
                                                 const int64_t* __restrict__ ubeg, int nmat,
                                                 double* __restrict__ part,
                                                 unsigned long long* __restrict__ nonfinite) {
    __shared__ float shf[kT / 64];
    __shared__ double shd[kT / 64];
    __shared__ double tab[64];
    if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
    __syncthreads();
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const EntMat em = mats[m];
    F32Acc acc;
    acc.tab = tab;
    f32_unit(em, u - ubeg[m], acc);
    if (acc.nbad) atomicAdd(nonfinite, (unsigned long long)acc.nbad);
    const float c = block_maxf(acc.mx, shf);
    const float bad = block_maxf(acc.nbad ? 1.f : 0.f, shf);
    acc.rebase(c);
    const double S = block_sum(acc.S, shd);
    const double U = block_sum(acc.U, shd);
    if (threadIdx.x == 0) {
        part[3 * u] = (double)c;
        part[3 * u + 1] = bad != 0.f ? (double)NAN : S;
        part[3 * u + 2] = U;
    }
}

// One wave per matrix: lane l takes the matrix's units l, l + 64, ... in
// order, each moved to the matrix maximum c, and the lanes' sums are added
// in a fixed order.  exp_hist (may be NULL): the matrix's row of exponent
// counts is zeroed (the counts are kept for bf16 matrices only).
__global__ __launch_bounds__(64) void k_f32_final(const EntMat* __restrict__ mats,
                                                  const int64_t* __restrict__ ubeg, int nmat,
                                                  const double* __restrict__ part,
                                                  double* __restrict__ h_mat,
                                                  uint32_t* __restrict__ exp_hist) {
    const int m = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t u0 = ubeg[m], u1 = ubeg[m + 1];
    const int slot = mats[m].slot;
    if (exp_hist) gstore<u32x4>(exp_hist + (size_t)slot * 256 + 4 * lane, u32x4{0u, 0u, 0u, 0u});
    double c = -INFINITY;
    for (int64_t u = u0 + lane; u < u1; u += 64) c = fmax(c, part[3 * u]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c = fmax(c, __shfl_xor(c, o, 64));
    double S = 0.0, U = 0.0;
    for (int64_t u = u0 + lane; u < u1; u += 64) {
        const double su = part[3 * u + 1];
        if (su != 0.0) {
            const double d = part[3 * u] - c;
            const double r = exp(d);
            S += r * su;
            U += r * (part[3 * u + 2] + su * d);
        }
    }
    S = wave_sum(S);
    U = wave_sum(U);
    if (lane == 0) h_mat[slot] = log(S) - U / S;
}

// ---------------------------------------------------------------- blocks
constexpr int kBT = 1024;   // threads of k_blocks

__global__ __launch_bounds__(kBT) void k_blocks(const int32_t* __restrict__ bmats,
                                               const int32_t* __restrict__ bbeg,
                                               const double* __restrict__ nsz,
                                               const double* __restrict__ h_mat, int nb,
                                               double x, double* __restrict__ h_block,
                                               double* __restrict__ stats,
                                               int32_t* __restrict__ tier,
                                               int32_t* __restrict__ order) {
    __shared__ double shd[kBT / 64];
    __shared__ double H[kMaxBlocks];   // the block entropies (32 KB)
    // one wave per block: lane j takes the block's matrices j, j + 64, ...,
    // then the lanes' sums are combined in a fixed order
    const int lane = threadIdx.x & 63;
    for (int b = threadIdx.x >> 6; b < nb; b += kBT / 64) {
        double num = 0.0, den = 0.0;
        for (int i = bbeg[b] + lane; i < bbeg[b + 1]; i += 64) {
            const int m = bmats[i];
            num += nsz[m] * h_mat[m];
            den += nsz[m];
        }
        num = wave_sum(num);
        den = wave_sum(den);
        if (lane == 0) {
            const double h = num / den;
            H[b] = h;
            if (h_block) h_block[b] = h;
        }
    }
    __syncthreads();
    double acc = 0.0;
    for (int b = threadIdx.x; b < nb; b += kBT) acc += H[b];
    const double mu = block_sum<kBT>(acc, shd) / nb;
    acc = 0.0;
    for (int b = threadIdx.x; b < nb; b += kBT) { const double d = H[b] - mu; acc += d * d; }
    const double sigma = sqrt(block_sum<kBT>(acc, shd) / nb);
    const double t = mu - x * sigma;
    if (stats && threadIdx.x == 0) { stats[0] = mu; stats[1] = sigma; stats[2] = t; }
    for (int b = threadIdx.x; b < nb; b += kBT) {
        const double h = H[b];
        if (tier) tier[b] = (h <= t) ? 1 : ((h < mu) ? 2 : 3);
        if (order) {
            int rank = 0;
            for (int o = 0; o < nb; ++o) {
                const double g = H[o];
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

// p 16-byte aligned: 16-byte stores, then the last n % 4 words.
__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        const uint4 w = make_uint4(v, v, v, v);
        uint4* q = reinterpret_cast<uint4*>(p);
        const size_t n4 = n >> 2;
        for (size_t i = t; i < n4; i += stride) q[i] = w;
        for (size_t i = 4 * n4 + t; i < n; i += stride) p[i] = v;
    } else {
        for (size_t i = t; i < n; i += stride) p[i] = v;
    }
}

}  // namespace

hipError_t fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = min((n / 4 + 255) / 256 + 1, (size_t)4096);
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

hipError_t ent_hist_bf16(const EntMat* mats, const int64_t* vbeg, int nmat, int64_t n_vec,
                         uint32_t* recs, uint16_t* lists, hipStream_t s) {
    if (n_vec <= 0) return hipSuccess;
    // Workgroups: one per 1 MiB of weights, at least the number the device
    // holds at once and at most kHistWaves times that (measured on the 8B
    // and MoE stacks: 4 beat 1, 2 and 8 - shares small enough that the last
    // ones to finish leave little idle, large enough that a matrix
    // segment's clearing and flush stay rare; on one 8B block, 436 MB, one
    // round of 340 KB shares takes 0.138 ms against 0.170 with four rounds
    // of 85 KB)
    constexpr int kHistWaves = 4;
    constexpr int64_t kHistShareVecs = (int64_t(1) << 20) / 16;
    static std::atomic<int> resident[64];   // per device, 0 until first looked up
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int g_res = resident[dev].load(std::memory_order_relaxed);
    if (g_res == 0) {
        int per_cu = 0, cus = 0;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &per_cu, reinterpret_cast<const void*>(k_hist_bf16), kT, 0)) != hipSuccess)
            return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        g_res = std::max(1, per_cu) * std::max(1, cus);
        resident[dev].store(g_res, std::memory_order_relaxed);
    }
    const int64_t by_bytes = (n_vec + kHistShareVecs - 1) / kHistShareVecs;
    const int64_t g_want =
        std::min<int64_t>((int64_t)kHistWaves * g_res, std::max<int64_t>(g_res, by_bytes));
    const int64_t g = std::min<int64_t>(g_want, (n_vec + kT - 1) / kT);
    k_hist_bf16<<<dim3((unsigned)g), dim3(kT), 0, s>>>(mats, vbeg, nmat, recs, lists);
    return hipGetLastError();
}

hipError_t ent_hist_final(const EntMat* mats, int nmat, const uint32_t* recs,
                          const uint16_t* lists, double* h_mat, unsigned long long* nonfinite,
                          uint32_t* exp_hist, hipStream_t s) {
    if (nmat <= 0) return hipSuccess;
    k_hist_final<<<dim3((unsigned)nmat), dim3(kT), 0, s>>>(mats, recs, lists, h_mat, nonfinite,
                                                          exp_hist);
    return hipGetLastError();
}

hipError_t ent_f32(const EntMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                   double* part, double* h_mat, unsigned long long* nonfinite,
                   uint32_t* exp_hist, hipStream_t s) {
    if (nmat <= 0) return hipSuccess;
    k_f32_part<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, part, nonfinite);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_f32_final<<<dim3((unsigned)nmat), dim3(64), 0, s>>>(mats, ubeg, nmat, part, h_mat, exp_hist);
    return hipGetLastError();
}

hipError_t ent_blocks(const int32_t* bmats, const int32_t* bbeg, const double* nsz,
                      const double* h_mat, int n_blocks, double x,
                      double* h_block, double* stats, int32_t* tier, int32_t* order,
                      hipStream_t s) {
    k_blocks<<<dim3(1), dim3(kBT), 0, s>>>(bmats, bbeg, nsz, h_mat, n_blocks, x, h_block,
                                           stats, tier, order);
    return hipGetLastError();
}

}  // namespace woq
