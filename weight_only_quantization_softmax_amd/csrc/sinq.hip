// SINQ dual-axis scaling: Sinkhorn-Knopp-style alternating normalisation of
// the row and column standard deviations of each weight matrix.
//
// [SINQ] "Huawei gioi thieu SINQ" (asiadaily.org), sections "Dinh ty le tren
// hai truc" (one scale vector per row and one per column) and "Chuan hoa
// Sinkhorn Knopp" (rows and columns are rescaled in turn until their
// standard deviations reach the target; not a doubly stochastic matrix).
//
// One iteration: s_i = std_j(W_ij / t_j), then t_j = std_i(W_ij / s_i),
// centred population std, zero std -> 1; t starts at 1.  The kernels hold
// u = 1/t and v = 1/s (correctly rounded fp32) and compute x = w * u (or
// w * v) in fp32; per-lane fp32 sums of x and x^2 are combined in fp64 in a
// fixed order, so the result is deterministic.  The variance is
// E[x^2] - E[x]^2 in fp64.  For fp32 inputs every line is first shifted by
// its first element (exact zero variance for constant lines); bf16 values
// make the unshifted sums exact in that case already.
//
// Kernels per iteration (all matrices of the call in each launch):
//   k_rows     one wave per row: s_i and v_i.
//   k_colpart  one thread per 8 columns over a chunk of rows: fp32 partial
//              (sum, sum of squares) per column and chunk.
//   k_colfin   one thread per column: fp64 combine of the chunk partials,
//              t_j and u_j.
#include "launch.h"

#include <math.h>

namespace woq {
namespace {

constexpr int kT = 256;

template <int DT>
__device__ __forceinline__ void rows_body(const SinqMat& sm, int row, int lane, bool first) {
    const int nv = sm.cols >> 3;
    const int64_t rb = (int64_t)row * sm.cols;
    float K = 0.f;
    if constexpr (DT == WOQ_F32) {
        K = reinterpret_cast<const float*>(sm.data)[rb];
        if (!first) K = K * sm.u[0];
    }
    float S = 0.f, Q = 0.f;
    for (int j = lane; j < nv; j += kWave) {
        float x[8];
        load8<DT>(sm.data, rb + 8 * j, x);
        if (!first) {
            float uu[8];
            load8f(sm.u + 8 * j, uu);
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = x[k] * uu[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float y = x[k] - K;
            S += y;
            Q = fmaf(y, y, Q);
        }
    }
    const double Sd = wave_sum((double)S);
    const double Qd = wave_sum((double)Q);
    if (lane == 0) {
        const double n = (double)sm.cols;
        const double mean = Sd / n;
        const double var = Qd / n - mean * mean;
        const float s = var > 0.0 ? (float)sqrt(var) : 1.0f;
        sm.s[row] = s;
        sm.v[row] = __fdiv_rn(1.0f, s);
    }
}

__global__ __launch_bounds__(kT) void k_rows(const SinqMat* __restrict__ mats,
                                             const int64_t* __restrict__ ubeg, int nmat,
                                             int first) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const SinqMat sm = mats[m];
    const int row = (int)(u - ubeg[m]) * (kT / kWave) + (threadIdx.x >> 6);
    if (row >= sm.rows) return;  // no block-level synchronisation below
    const int lane = threadIdx.x & 63;
    if (sm.dtype == WOQ_BF16) rows_body<WOQ_BF16>(sm, row, lane, first != 0);
    else rows_body<WOQ_F32>(sm, row, lane, first != 0);
}

template <int DT>
__device__ __forceinline__ void colpart_body(const SinqMat& sm, int chunk, int cv) {
    const int r0 = chunk * sm.chunk_rows;
    const int r1 = min(sm.rows, r0 + sm.chunk_rows);
    const int c0 = 8 * cv;
    float K[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) K[k] = 0.f;
    if constexpr (DT == WOQ_F32) {
        float x0[8];
        load8<DT>(sm.data, c0, x0);
        const float v0 = sm.v[0];
#pragma unroll
        for (int k = 0; k < 8; ++k) K[k] = x0[k] * v0;
    }
    float cs[8], cq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) { cs[k] = 0.f; cq[k] = 0.f; }
    for (int r = r0; r < r1; ++r) {
        float x[8];
        load8<DT>(sm.data, (int64_t)r * sm.cols + c0, x);
        const float vr = sm.v[r];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float y = x[k] * vr - K[k];
            cs[k] += y;
            cq[k] = fmaf(y, y, cq[k]);
        }
    }
    float4* out = reinterpret_cast<float4*>(sm.part + (size_t)chunk * sm.cols + c0);
    out[0] = make_float4(cs[0], cq[0], cs[1], cq[1]);
    out[1] = make_float4(cs[2], cq[2], cs[3], cq[3]);
    out[2] = make_float4(cs[4], cq[4], cs[5], cq[5]);
    out[3] = make_float4(cs[6], cq[6], cs[7], cq[7]);
}

__global__ __launch_bounds__(kT) void k_colpart(const SinqMat* __restrict__ mats,
                                                const int64_t* __restrict__ ubeg, int nmat) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const SinqMat sm = mats[m];
    const int local = (int)(u - ubeg[m]);
    const int chunk = local / sm.col_tiles;
    const int tile = local - chunk * sm.col_tiles;
    const int cv = tile * kT + threadIdx.x;
    if (cv >= (sm.cols >> 3)) return;
    if (sm.dtype == WOQ_BF16) colpart_body<WOQ_BF16>(sm, chunk, cv);
    else colpart_body<WOQ_F32>(sm, chunk, cv);
}

__global__ __launch_bounds__(kT) void k_colfin(const SinqMat* __restrict__ mats,
                                               const int64_t* __restrict__ ubeg, int nmat) {
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(ubeg, nmat, u);
    const SinqMat sm = mats[m];
    const int j = (int)(u - ubeg[m]) * kT + threadIdx.x;
    if (j >= sm.cols) return;
    double S = 0.0, Q = 0.0;
    for (int c = 0; c < sm.n_chunks; ++c) {
        const float2 p = sm.part[(size_t)c * sm.cols + j];
        S += (double)p.x;
        Q += (double)p.y;
    }
    const double n = (double)sm.rows;
    const double mean = S / n;
    const double var = Q / n - mean * mean;
    const float t = var > 0.0 ? (float)sqrt(var) : 1.0f;
    sm.t[j] = t;
    sm.u[j] = __fdiv_rn(1.0f, t);
}

}  // namespace

hipError_t sinq_rows(const SinqMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     bool first, bool /*any_f32*/, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_rows<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, first ? 1 : 0);
    return hipGetLastError();
}

hipError_t sinq_colpart(const SinqMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        bool /*any_f32*/, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_colpart<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat);
    return hipGetLastError();
}

hipError_t sinq_colfin(const SinqMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                       hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_colfin<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat);
    return hipGetLastError();
}

}  // namespace woq
