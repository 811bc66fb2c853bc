// SINQ dual-axis scaling: Sinkhorn-Knopp-style alternating normalisation of
// the row and column standard deviations of each weight matrix.
//
// [SINQ] "Huawei gioi thieu SINQ" (asiadaily.org), sections "Dinh ty le tren
// hai truc" (one scale vector per row and one per column) and "Chuan hoa
// Sinkhorn Knopp" (rows and columns are rescaled in turn until their
// standard deviations reach the target; not a doubly stochastic matrix).
//
// One iteration: s_i = std_j(W_ij / t_j), then t_j = std_i(W_ij / s_i),
// centred population std, zero std -> 1; t starts at 1.  Variant: the root
// mean square (uncentred) in place of the std, from the same moments
// (M2 / n + mean^2 for rows, E[z^2] for columns).  Kernels hold
// u = 1/t and v = 1/s (correctly rounded fp32) and form x = w * u (w * v).
//
// Fused pass (one read of W per iteration), in two forms:
//  - k_sinq_wave, rows of at most 4096 bf16 (1536 fp32) columns: a
//    workgroup owns a strip of whole rows, dealt to its four waves in turn,
//    lane l the 8-column vectors l + 64 k, so the row statistics are
//    wave-local (no workgroup barrier);
//  - k_sinq_pass, wider rows: a workgroup owns a strip of whole rows, thread
//    t the vectors t + NT k, and the row statistics are combined over the
//    waves through LDS (one barrier per tile of R rows).
// In both, a thread's column partial sums stay in registers for the whole
// strip, the next rows' loads are in flight while the current ones are
// processed, and per row:
//   1. row moments of x = w*u in one pass: each lane sums y = x*u - K around
//      a lane-local shift K (its first product), giving its mean and centred
//      sum of squares M2 = sum y^2 - (sum y)^2 / n; lanes (then waves) are
//      merged with the pairwise update of Chan, Golub and LeVeque (1979)
//      -> s_i, v_i = 1/s_i;
//   2. the same registers give z = w*v_i, accumulated into the thread's
//      column (sum, sum of squares).
// At the end every workgroup writes one partial row; a second kernel combines
// the partial rows per column in fp64 in a fixed order -> t_j, u_j.  (A
// wave-form matrix swept by one workgroup is finished by that workgroup
// from the same sums, with the same arithmetic.)
// Everything runs in a fixed order, so results are deterministic.
//
// Accuracy.  Since K is one of the lane's own values, n (mean - K)^2 is at
// most n M2_lane, so the shifted sums lose about eps (n + 1) of M2_lane
// (n <= 64 per lane); a constant row at the first step gives y = 0 exactly
// (std 0 -> scale 1).  Column variance is E[z^2] - E[z]^2 in fp64 from fp32
// partials: relative accuracy ~1e-7 (1 + mean^2/var), ample for the
// near-zero column means of weight matrices.  A column with mean^2 > 64 var
// (few rows, or a large common offset) is recomputed by the reduction in one
// pass around its mean.  bf16 columns that are constant at the first step
// (or all zero) sum exactly, and fp32 inputs also track per-column min/max
// (a constant column has std 0).
//
// Matrices of one launch share their shape class (wave or workgroup form,
// vectors per lane / thread, threads per workgroup).  Rows are addressed
// through the matrix's row stride ld.
//
// Non-finite weights.  In the first iteration (t = 1) a NaN or inf weight
// makes its row's moments non-finite (so does a finite row whose squares
// overflow fp32), so the rows to inspect are known from the moments alone;
// only those rows are scanned element by element, and their NaN / inf
// weights are added to the call's uint64 counter.
#include "launch.h"

#include <math.h>

#include <type_traits>

namespace woq {
namespace {

constexpr int kMaxT = 512;

template <int DT> struct Vec8;
template <> struct Vec8<WOQ_BF16> { uint4 v; };
template <> struct Vec8<WOQ_F32> { float4 a, b; };

template <int DT>
__device__ __forceinline__ Vec8<DT> ldv(const void* base, int64_t e) {
    Vec8<DT> r;
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
__device__ __forceinline__ void unpack(const Vec8<DT>& r, float (&x)[8]) {
    if constexpr (DT == WOQ_BF16) {
        x[0] = bf_lo(r.v.x); x[1] = bf_hi(r.v.x); x[2] = bf_lo(r.v.y); x[3] = bf_hi(r.v.y);
        x[4] = bf_lo(r.v.z); x[5] = bf_hi(r.v.z); x[6] = bf_lo(r.v.w); x[7] = bf_hi(r.v.w);
    } else {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
}

// Rows per register tile, per dtype and vectors per thread.
constexpr int tile_rows(int dt, int nv) {
    return dt == WOQ_BF16 ? (nv == 1 ? 8 : (nv == 2 ? 4 : (nv <= 4 ? 2 : 1))) : (nv == 1 ? 4 : (nv == 2 ? 2 : 1));
}

template <int DT, int NV>
struct PassCfg {
    static constexpr int R = tile_rows(DT, NV);
    static constexpr bool U_LDS = NV >= 3;
    static constexpr bool F32 = DT == WOQ_F32;
    // wide rows: unpack bf16 again for each pass instead of keeping the
    // unpacked tile live across the barriers (register pressure)
    static constexpr bool REUNPACK = DT == WOQ_BF16 && NV >= 3;
};

// Empty asm that claims to modify the packed registers, so the compiler
// cannot reuse values unpacked before it (ALU registers only, no memory).
template <int DT>
__device__ __forceinline__ void opaque(Vec8<DT>& r) {
    if constexpr (DT == WOQ_BF16) asm volatile("" : "+v"(r.v.x), "+v"(r.v.y), "+v"(r.v.z), "+v"(r.v.w));
}

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads already in flight (the next tile) stay in flight across it.  The
// "memory" clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Row moments with one pass over the registers.  Each lane accumulates its
// own elements y = x*u - K around a lane-local shift K (its first element),
// giving its mean and centred sum of squares M2 = sum y^2 - (sum y)^2 / n.
// The cancellation in M2 is bounded by the lane's own spread: since K is one
// of the lane's values, n (mean - K)^2 <= n * M2_lane, so the rounding error
// is about eps * (n + 1) * M2_lane (n <= 64 here), far below the 1e-4
// tolerance on the scales.  A constant row at the first step (u = 1) gives
// y = 0 exactly and hence std 0.  Lane moments are then merged over the wave
// with the pairwise update of Chan, Golub and LeVeque (1979):
//   mean = (m_a n_a + m_b n_b) / n,  M2 = M2_a + M2_b + d^2 n_a n_b / n.
// For equal counts the update is symmetric in (a, b), so every lane of the
// butterfly computes the identical result.

// Equal counts n_a = n_b: hn = n_a / 2.
__device__ __forceinline__ void merge_eq(float& m, float& q, float pm, float pq, float hn) {
    const float d = m - pm;
    q = fmaf(d * d, hn, q + pq);
    m = (m + pm) * 0.5f;
}
// General counts (a = own, b = partner).
__device__ __forceinline__ void merge_gen(float& m, float& q, float& n, float pm, float pq, float pn) {
    const float nt = n + pn;
    const float w = nt > 0.f ? pn * __builtin_amdgcn_rcpf(nt) : 0.f;  // n_b / n
    const float d = pm - m;
    q = fmaf(d * d, n * w, q + pq);
    m = fmaf(d, w, m);
    n = nt;
}

// Merge (m, q) over the 64 lanes; every lane holds n elements.
__device__ __forceinline__ void wave_moments_eq(float& m, float& q, float n) {
    float bm = m, bq = q;
    swap32(m, bm);
    swap32(q, bq);
    merge_eq(m, q, bm, bq, 0.5f * n);
    bm = m;
    bq = q;
    swap16(m, bm);
    swap16(q, bq);
    merge_eq(m, q, bm, bq, n);
    merge_eq(m, q, dpp<kDppXor8>(m), dpp<kDppXor8>(q), 2.f * n);
    merge_eq(m, q, dpp<kDppMirror8>(m), dpp<kDppMirror8>(q), 4.f * n);
    merge_eq(m, q, dpp<kDppXor2>(m), dpp<kDppXor2>(q), 8.f * n);
    merge_eq(m, q, dpp<kDppXor1>(m), dpp<kDppXor1>(q), 16.f * n);
}
// Merge (m, q, n) over the 64 lanes with per-lane counts.  Lanes may end
// with results that differ in the last bits; callers use lane 0's.
__device__ __forceinline__ void wave_moments_gen(float& m, float& q, float& n) {
    float bm = m, bq = q, bn = n;
    swap32(m, bm);
    swap32(q, bq);
    swap32(n, bn);
    merge_gen(m, q, n, bm, bq, bn);
    bm = m;
    bq = q;
    bn = n;
    swap16(m, bm);
    swap16(q, bq);
    swap16(n, bn);
    merge_gen(m, q, n, bm, bq, bn);
    merge_gen(m, q, n, dpp<kDppXor8>(m), dpp<kDppXor8>(q), dpp<kDppXor8>(n));
    merge_gen(m, q, n, dpp<kDppMirror8>(m), dpp<kDppMirror8>(q), dpp<kDppMirror8>(n));
    merge_gen(m, q, n, dpp<kDppXor2>(m), dpp<kDppXor2>(q), dpp<kDppXor2>(n));
    merge_gen(m, q, n, dpp<kDppXor1>(m), dpp<kDppXor1>(q), dpp<kDppXor1>(n));
}

__device__ __forceinline__ float first_lane(float v) {
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

// NaN / inf weights among 8, from the packed bits (an all-ones exponent
// field), without unpacking.
__device__ __forceinline__ uint32_t nonfinite_bf16x2(uint32_t w) {
    return ((w & 0x7f80u) == 0x7f80u ? 1u : 0u) + ((w & 0x7f800000u) == 0x7f800000u ? 1u : 0u);
}
__device__ __forceinline__ uint32_t nonfinite_f32(float f) {
    return (__float_as_uint(f) & 0x7f800000u) == 0x7f800000u ? 1u : 0u;
}
template <int DT>
__device__ __forceinline__ uint32_t nonfinite8(const Vec8<DT>& r) {
    if constexpr (DT == WOQ_BF16) {
        return nonfinite_bf16x2(r.v.x) + nonfinite_bf16x2(r.v.y) + nonfinite_bf16x2(r.v.z) +
               nonfinite_bf16x2(r.v.w);
    } else {
        return nonfinite_f32(r.a.x) + nonfinite_f32(r.a.y) + nonfinite_f32(r.a.z) +
               nonfinite_f32(r.a.w) + nonfinite_f32(r.b.x) + nonfinite_f32(r.b.y) +
               nonfinite_f32(r.b.z) + nonfinite_f32(r.b.w);
    }
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Lane moments from the shifted sums: mean K + S/n and M2 = Q - S^2/n
// (clamped at 0 against rounding); a lane without elements gives (0, 0).
__device__ __forceinline__ void lane_moments(float K, float S, float Q, float n, float rn,
                                             float& m, float& q) {
    m = n > 0.f ? fmaf(S, rn, K) : 0.f;
    q = n > 0.f ? fmaxf(fmaf(-S, S * rn, Q), 0.f) : 0.f;
}

// Workgroup pass for wider rows: a workgroup owns a strip of whole rows and
// thread t owns the 8-column vectors t + NT k (k < NV).  The strip is walked
// in tiles of R rows held in registers (the next tile's loads are in flight
// while the current one is processed).  Per row: lane moments, merged over
// the wave (Chan), then over the waves through LDS in wave order (one
// barrier per tile); then the column partials of z = w * v.  RAG: NT * NV
// exceeds the row's vectors, so threads own unequal numbers of them.
template <int DT, int NV, bool FIRST, bool RAG>
__global__ __launch_bounds__(kMaxT) void k_sinq_pass(const SinqMat* __restrict__ mats,
                                                     const int64_t* __restrict__ sbeg, int nmat,
                                                     unsigned long long* __restrict__ nonfinite) {
    using C = PassCfg<DT, NV>;
    constexpr int R = C::R;
    __shared__ float2 red[2][kMaxT / 64][R];
    extern __shared__ float ulds[];  // u [cols + 8] when U_LDS

    const int m = find_unit_owner(sbeg, nmat, (int64_t)blockIdx.x);
    const SinqMat sm = mats[m];
    const int strip = (int)(blockIdx.x - sbeg[m]);
    const int r0 = strip * sm.strip_rows;
    const int r1 = min(sm.rows, r0 + sm.strip_rows);
    const int NT = blockDim.x;
    const int nw = NT >> 6;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int nvec = sm.cols >> 3;
    const int64_t cols = sm.cols;
    const int64_t ld = sm.ld;
    const float fn = (float)sm.cols;
    uint32_t nbad = 0;  // first iteration: NaN / inf weights this thread saw

    int vk[NV], ui[NV];
    bool own[NV];
    int nown = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        own[k] = !RAG || tid + NT * k < nvec;
        vk[k] = own[k] ? tid + NT * k : nvec - 1;  // clamped: loads stay in bounds
        ui[k] = own[k] ? vk[k] : nvec;              // LDS index: zero pad for non-owned
        nown += own[k] ? 1 : 0;
    }
    const float nl = 8.f * (float)nown;
    const float rnl = nown ? 1.0f / nl : 0.f;
    // elements of a row held by wave w
    auto wave_count = [&](int w) -> float {
        if constexpr (!RAG) return 512.f * NV;
        int c = 0;
#pragma unroll
        for (int k = 0; k < NV; ++k) c += min(64, max(0, nvec - NT * k - 64 * w));
        return 8.f * (float)c;
    };
    // Row multipliers u (0 for vectors this thread does not own).
    float uu[C::U_LDS ? 1 : NV][8];
    if constexpr (C::U_LDS) {
        for (int j = tid; j < sm.cols + 8; j += NT)
            ulds[j] = j < sm.cols ? (FIRST ? 1.0f : gload<float>(sm.u + j)) : 0.0f;
        __syncthreads();
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const float o = own[k] ? 1.0f : 0.0f;
            if constexpr (FIRST) {
#pragma unroll
                for (int e = 0; e < 8; ++e) uu[k][e] = o;
            } else {
                const float4 a = gload_f4(sm.u + 8 * vk[k]);
                const float4 b = gload_f4(sm.u + 8 * vk[k] + 4);
                uu[k][0] = a.x * o; uu[k][1] = a.y * o; uu[k][2] = a.z * o; uu[k][3] = a.w * o;
                uu[k][4] = b.x * o; uu[k][5] = b.y * o; uu[k][6] = b.z * o; uu[k][7] = b.w * o;
            }
        }
    }
    const f32x4* u4 = reinterpret_cast<const f32x4*>(ulds);
    auto uvec = [&](int k, float (&w)[8]) {
        if constexpr (C::U_LDS) {
            const f32x4 a = u4[2 * ui[k]], b = u4[2 * ui[k] + 1];
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = uu[k][e];
        }
    };

    float cs[NV][8], cq[NV][8];
    float cmn[C::F32 ? NV : 1][8], cmx[C::F32 ? NV : 1][8];
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            cs[k][e] = 0.f;
            cq[k][e] = 0.f;
            if constexpr (C::F32) { cmn[k][e] = INFINITY; cmx[k][e] = -INFINITY; }
        }

    int buf = 0;
    auto load_tile = [&](Vec8<DT> (&d)[R][NV], int rb) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = min(rb + r, r1 - 1);  // clamped into the strip
#pragma unroll
            for (int k = 0; k < NV; ++k) d[r][k] = ldv<DT>(sm.data, row * ld + 8 * vk[k]);
        }
    };

    // FULLT: every row of the tile lies in the strip (no masking needed)
    auto process = [&](Vec8<DT> (&d)[R][NV], int rb, auto fullc) {
        constexpr bool FULLT = decltype(fullc)::value;
        float xf[C::REUNPACK ? 1 : R][C::REUNPACK ? 1 : NV][8];
        if constexpr (!C::REUNPACK) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < NV; ++k) unpack<DT>(d[r][k], xf[r][k]);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < NV; ++k) opaque<DT>(d[r][k]);
        }
        auto xval = [&](int r, int k, float (&x)[8]) {
            if constexpr (C::REUNPACK) unpack<DT>(d[r][k], x);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = xf[r][k][e];
            }
        };
        // ---- lane moments per row, merged over the wave
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float S0 = 0.f, S1 = 0.f, Q0 = 0.f, Q1 = 0.f, K = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                float x[8], w[8];
                xval(r, k, x);
                uvec(k, w);
                if (k == 0) K = x[0] * w[0];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float y0 = fmaf(x[e], w[e], -K), y1 = fmaf(x[e + 1], w[e + 1], -K);
                    if (RAG && !own[k]) { y0 = 0.f; y1 = 0.f; }
                    S0 += y0;
                    S1 += y1;
                    Q0 = fmaf(y0, y0, Q0);
                    Q1 = fmaf(y1, y1, Q1);
                }
            }
            float mm, qq;
            lane_moments(K, S0 + S1, Q0 + Q1, nl, rnl, mm, qq);
            if constexpr (RAG) {
                float nn = nl;
                wave_moments_gen(mm, qq, nn);
            } else {
                wave_moments_eq(mm, qq, nl);
            }
            if (lane == 0) red[buf][wid][r] = make_float2(mm, qq);
        }
        lds_barrier();
        // ---- lane r < R merges row r over the waves in wave order
        float vv = 0.f;
        bool rbad = false;  // first iteration: the row's moments are not finite
        if (lane < R) {
            const int row = rb + lane;
            float2 a = red[buf][0][lane];
            float M = a.x, Q = a.y, N = wave_count(0);
            for (int w = 1; w < nw; ++w) {
                a = red[buf][w][lane];
                merge_gen(M, Q, N, a.x, a.y, wave_count(w));
            }
            const float var = sm.rms ? fmaf(M, M, Q / fn) : Q / fn;
            const float s = var > 0.f ? __fsqrt_rn(var) : 1.0f;
            if (row < r1) {
                vv = __fdiv_rn(1.0f, s);
                if (wid == 0) gstore<float>(sm.s + row, s);
                rbad = FIRST && !(isfinite(M) && isfinite(Q));
            }
        }
        if constexpr (FIRST) {
            // the tile's rows whose moments are not finite: count their NaN /
            // inf weights (each thread its own vectors; rare)
            const uint64_t badm = __ballot(rbad);
            if (badm) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if ((badm >> r) & 1u)
#pragma unroll
                        for (int k = 0; k < NV; ++k)
                            if (!RAG || own[k]) nbad += nonfinite8<DT>(d[r][k]);
            }
        }
        buf ^= 1;
        if constexpr (C::REUNPACK) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < NV; ++k) opaque<DT>(d[r][k]);
        }
        // ---- column partials of z = w * v with the new row scales
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float vr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(vv), r));
            const bool valid = rb + r < r1;
            const float rv = valid ? 1.0f : 0.0f;  // rows past the strip add nothing
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                float x[8];
                xval(r, k, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float z = x[e] * vr;
                    if constexpr (!FULLT) z *= rv;
                    cs[k][e] += z;
                    cq[k][e] = fmaf(z, z, cq[k][e]);
                    if constexpr (C::F32) {
                        if (FULLT || valid) { cmn[k][e] = fminf(cmn[k][e], z); cmx[k][e] = fmaxf(cmx[k][e], z); }
                    }
                }
            }
        }
    };

    // ---- tiles in pairs: the next tile's loads are issued before the
    //      current tile is processed (two register buffers)
    Vec8<DT> dA[R][NV], dB[R][NV];
    int rb = r0;
    if (rb < r1) load_tile(dA, rb);
    auto run = [&](Vec8<DT> (&d)[R][NV], int at) {
        if (at + R <= r1) process(d, at, std::true_type{});
        else process(d, at, std::false_type{});
    };
    while (rb < r1) {
        const int rn = rb + R;
        if (rn < r1) load_tile(dB, rn);
        run(dA, rb);
        if (rn >= r1) break;
        const int rn2 = rn + R;
        if (rn2 < r1) load_tile(dA, rn2);
        run(dB, rn);
        rb = rn2;
    }

    if constexpr (FIRST) {
        if (nbad) atomicAdd(nonfinite, (unsigned long long)nbad);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        if (!own[k]) continue;
        const int64_t c0 = (int64_t)strip * cols + 8 * vk[k];
        if constexpr (C::F32) {
            float4* p = reinterpret_cast<float4*>(sm.part) + c0;
#pragma unroll
            for (int e = 0; e < 8; ++e) gstore_f4(p + e, cs[k][e], cq[k][e], cmn[k][e], cmx[k][e]);
        } else {
            float4* p = reinterpret_cast<float4*>(reinterpret_cast<float2*>(sm.part) + c0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                gstore_f4(p + e, cs[k][2 * e], cq[k][2 * e], cs[k][2 * e + 1], cq[k][2 * e + 1]);
        }
    }
}

// A column whose squared mean exceeds this multiple of its variance is
// recomputed in the reduction (the fp32 partials would cost more than ~1e-5).
constexpr double kIllCond = 64.0;

// t_j and u_j = 1/t_j of column j from its fp64 sums S = sum z, Q = sum z^2
// over all rows (and, for fp32, the column's min and max of z).
template <int DT>
__device__ __forceinline__ void col_finish(const SinqMat& sm, int j, double S, double Q, float mn,
                                           float mx) {
    const double n = (double)sm.rows;
    const double mean = S / n;
    double var = sm.rms ? Q / n : Q / n - mean * mean;
    if (!sm.rms && mean * mean > kIllCond * var) {
        // E[z^2] - E[z]^2 from fp32 partials loses about eps * mean^2 / var:
        // recompute this column in one pass around the (accurate) mean, with
        // the same z = w * (1/s_i) as the sweep.
        double S2 = 0.0, Q2 = 0.0;
        for (int i = 0; i < sm.rows; ++i) {
            const float v = __fdiv_rn(1.0f, gload<float>(sm.s + i));
            float x;
            if constexpr (DT == WOQ_BF16)
                x = __uint_as_float((uint32_t)gload<uint16_t>(reinterpret_cast<const uint16_t*>(sm.data) + (int64_t)i * sm.ld + j) << 16);
            else
                x = gload<float>(reinterpret_cast<const float*>(sm.data) + (int64_t)i * sm.ld + j);
            const double dz = (double)(x * v) - mean;
            S2 += dz;
            Q2 += dz * dz;
        }
        var = Q2 / n - (S2 / n) * (S2 / n);
    }
    const bool constant = (DT == WOQ_F32) && !sm.rms && !(mx > mn);
    const float t = (var > 0.0 && !constant) ? (float)sqrt(var) : 1.0f;
    gstore<float>(sm.t + j, t);
    gstore<float>(sm.u + j, __fdiv_rn(1.0f, t));
}

// ---------------------------------------------------------------------------
// Wave-per-row pass for rows of at most 4096 bf16 (1536 fp32) columns.  A
// workgroup owns 4 * strip_rows consecutive rows of one matrix, dealt to its
// four waves in turn (chunks of RW rows: wave w takes chunks w, w + 4, ...),
// so the workgroup streams one contiguous region; the same rows split into
// four contiguous sub-strips, one per wave, streamed 7% slower (four times
// as many separate streams across the chip).  Lane l owns the 8-column
// vectors l + 64 k (k < NVL), so row statistics need no workgroup barrier and
// the column partials of the wave's rows stay in the lane's registers.  Rows
// go through two packed register buffers: the wave's next chunk is loaded
// while the current one is processed.  u = 1/t is staged once per workgroup in
// LDS.  At the end the four waves add their column partials in LDS in wave
// order and the workgroup writes one partial row.  RAG: the row is not a
// multiple of 512 columns, so lanes own unequal numbers of vectors.
// Shape constants of the wave pass.  KEEP: the row is kept unpacked between
// the two passes (rows of at most 3 vectors per lane); wider bf16 rows keep
// only the packed row and unpack it once per pass (register pressure).  Two
// waves per SIMD throughout (measured: more waves with re-unpacked narrow
// rows ran slower); narrow rows instead take RW rows per step.
template <int DT, int NVL>
struct WaveCfg {
    static constexpr bool F32 = DT == WOQ_F32;
    static constexpr int OCC = 2;  // waves per SIMD
    static constexpr bool KEEP = F32 || NVL <= 3;
    // rows per step: narrow bf16 rows go RW at a time, sharing each 1/t read
    // among RW rows (measured on MoE shapes: 2 rows help 4-vector rows by 5%,
    // and cost 3-vector ragged rows 4%)
    static constexpr int RW = (F32 || NVL >= 5 || NVL == 3) ? 1 : (NVL == 4 ? 2 : (NVL == 2 ? 2 : 4));
    static constexpr int NP = F32 ? 4 : 2;                  // partial floats per column
    static constexpr int UW = NVL * 512 + 8;                // LDS floats of u and its zero pad
    static constexpr size_t lds() { return sizeof(float) * ((size_t)UW + (size_t)NP * NVL * 512); }
};

template <int DT, int NVL, bool FIRST, bool RAG>
__global__ __launch_bounds__(256, (WaveCfg<DT, NVL>::OCC)) void k_sinq_wave(
    const SinqMat* __restrict__ mats, const int64_t* __restrict__ wgbeg, int nmat,
    unsigned long long* __restrict__ nonfinite) {
    using WC = WaveCfg<DT, NVL>;
    constexpr bool F32 = WC::F32;
    constexpr int NP = WC::NP;
    constexpr int kWaveU = WC::UW;
    // otherwise only the packed row is kept and unpacked once per pass
    constexpr bool KEEP = WC::KEEP;
    extern __shared__ float ul[];    // u [kWaveU], then the partial sum [cols][NP]
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int m = find_unit_owner(wgbeg, nmat, (int64_t)blockIdx.x);
    const SinqMat sm = mats[m];
    const int wg = (int)(blockIdx.x - wgbeg[m]);
    const int cols = sm.cols;
    const int64_t ld = sm.ld;
    const int nvec = cols >> 3;
    uint32_t nbad = 0;  // first iteration: NaN / inf weights of this wave's bad rows
    float* u = ul;
    float* cp = ul + kWaveU;
    for (int j = 4 * threadIdx.x; j < kWaveU; j += 4 * 256) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j < cols) v = FIRST ? f32x4{1.f, 1.f, 1.f, 1.f} : gload<f32x4>(sm.u + j);
        *reinterpret_cast<f32x4*>(u + j) = v;
    }
    __syncthreads();
    // the workgroup's rows [g0, r1); this wave's chunks start at r0, 4 RW apart
    const int g0 = min(sm.rows, 4 * wg * sm.strip_rows);
    const int r1 = min(sm.rows, g0 + 4 * sm.strip_rows);
    const int r0 = g0 + wid * WaveCfg<DT, NVL>::RW;

    int vk[NVL];
    bool own[NVL];
    int nown = 0;
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
        own[k] = !RAG || lane + 64 * k < nvec;
        vk[k] = own[k] ? lane + 64 * k : nvec - 1;  // clamped: loads stay in bounds
        nown += own[k] ? 1 : 0;
    }
    const float nl = 8.f * (float)nown;           // elements of the row in this lane
    const float rnl = nown ? 1.0f / nl : 0.f;
    const float fn = (float)cols;
    const f32x4* u4 = reinterpret_cast<const f32x4*>(u);

    float cs[NVL][8], cq[NVL][8];
    float cmn[F32 ? NVL : 1][8], cmx[F32 ? NVL : 1][8];
#pragma unroll
    for (int k = 0; k < NVL; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            cs[k][e] = 0.f;
            cq[k][e] = 0.f;
            if constexpr (F32) { cmn[k][e] = INFINITY; cmx[k][e] = -INFINITY; }
        }

    constexpr int RW = WC::RW;
    // rows row0 .. row0 + RW - 1 (clamped into the strip: loads stay in bounds)
    auto load_rows = [&](Vec8<DT> (&P)[RW][NVL], int row0) {
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int64_t row = min(row0 + rr, r1 - 1);
#pragma unroll
            for (int k = 0; k < NVL; ++k) P[rr][k] = ldv<DT>(sm.data, row * ld + 8 * vk[k]);
        }
    };
    auto process = [&](Vec8<DT> (&P)[RW][NVL], int row0) {
        float xk[KEEP ? RW : 1][KEEP ? NVL : 1][8];
        if constexpr (KEEP) {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int k = 0; k < NVL; ++k) unpack<DT>(P[rr][k], xk[rr][k]);
        } else {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int k = 0; k < NVL; ++k) opaque<DT>(P[rr][k]);
        }
        auto xval = [&](int rr, int k, float (&x)[8]) {
            if constexpr (KEEP) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = xk[rr][k][e];
            } else {
                unpack<DT>(P[rr][k], x);
            }
        };
        // lane moments of x*u around K = the lane's first product, per row
        float S0[RW], S1[RW], Q0[RW], Q1[RW], K[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) S0[rr] = S1[rr] = Q0[rr] = Q1[rr] = K[rr] = 0.f;
#pragma unroll
        for (int k = 0; k < NVL; ++k) {
            const f32x4 ua = u4[2 * vk[k]], ub = u4[2 * vk[k] + 1];
            const float uu[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                float x[8];
                xval(rr, k, x);
                if (k == 0) K[rr] = x[0] * uu[0];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float y0 = fmaf(x[e], uu[e], -K[rr]), y1 = fmaf(x[e + 1], uu[e + 1], -K[rr]);
                    if (RAG && !own[k]) { y0 = 0.f; y1 = 0.f; }
                    S0[rr] += y0;
                    S1[rr] += y1;
                    Q0[rr] = fmaf(y0, y0, Q0[rr]);
                    Q1[rr] = fmaf(y1, y1, Q1[rr]);
                }
            }
        }
        float v[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            float mm, qq;
            lane_moments(K[rr], S0[rr] + S1[rr], Q0[rr] + Q1[rr], nl, rnl, mm, qq);
            if constexpr (RAG) {
                float nn = nl;
                wave_moments_gen(mm, qq, nn);
            } else {
                wave_moments_eq(mm, qq, nl);
            }
            const float q1 = first_lane(qq) / fn;
            const float m1 = first_lane(mm);
            const float var = sm.rms ? fmaf(m1, m1, q1) : q1;
            const float s = var > 0.f ? __fsqrt_rn(var) : 1.0f;
            v[rr] = __fdiv_rn(1.0f, s);
            if (lane == 0 && row0 + rr < r1) gstore<float>(sm.s + row0 + rr, s);
            if constexpr (FIRST) {
                // wave-uniform: a row whose moments are not finite (rare)
                if (row0 + rr < r1 && !(isfinite(m1) && isfinite(q1))) {
#pragma unroll
                    for (int k = 0; k < NVL; ++k)
                        if (!RAG || own[k]) nbad += nonfinite8<DT>(P[rr][k]);
                }
            }
        }
        if constexpr (!KEEP) {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int k = 0; k < NVL; ++k) opaque<DT>(P[rr][k]);
        }
        // column partials with each row's scale (rows past the strip add nothing)
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            if (row0 + rr >= r1) break;
#pragma unroll
            for (int k = 0; k < NVL; ++k) {
                float x[8];
                xval(rr, k, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float z = x[e] * v[rr];
                    cs[k][e] += z;
                    cq[k][e] = fmaf(z, z, cq[k][e]);
                    if constexpr (F32) { cmn[k][e] = fminf(cmn[k][e], z); cmx[k][e] = fmaxf(cmx[k][e], z); }
                }
            }
        }
    };

    Vec8<DT> PA[RW][NVL], PB[RW][NVL];
    if (r0 < r1) load_rows(PA, r0);
    for (int row = r0; row < r1; row += 8 * RW) {
        if (row + 4 * RW < r1) load_rows(PB, row + 4 * RW);
        process(PA, row);
        if (row + 4 * RW >= r1) break;
        if (row + 8 * RW < r1) load_rows(PA, row + 8 * RW);
        process(PB, row + 4 * RW);
    }
    if constexpr (FIRST) {
        if (nbad) atomicAdd(nonfinite, (unsigned long long)nbad);
    }
    // the four waves' column partials, added in wave order in LDS
    for (int w = 0; w < 4; ++w) {
        if (wid == w) {
#pragma unroll
            for (int k = 0; k < NVL; ++k) {
                if (!own[k]) continue;
                f32x4* p = reinterpret_cast<f32x4*>(cp + (size_t)NP * 8 * vk[k]);
#pragma unroll
                for (int i = 0; i < 2 * NP; ++i) {
                    f32x4 v;
                    if constexpr (F32) {
                        v = f32x4{cs[k][i], cq[k][i], cmn[k][i], cmx[k][i]};
                    } else {
                        v = f32x4{cs[k][2 * i], cq[k][2 * i], cs[k][2 * i + 1], cq[k][2 * i + 1]};
                    }
                    if (w > 0) {
                        const f32x4 o = p[i];
                        if constexpr (F32) {
                            v = f32x4{o.x + v.x, o.y + v.y, fminf(o.z, v.z), fmaxf(o.w, v.w)};
                        } else {
                            v = o + v;
                        }
                    }
                    p[i] = v;
                }
            }
        }
        __syncthreads();
    }
    if (sm.n_strips == 1) {
        // this workgroup sweeps the whole matrix, so its partial row is the
        // column sums: t and u from them directly, with the arithmetic of
        // k_sinq_reduce for one partial row (the reduction skips the matrix)
        for (int j = threadIdx.x; j < cols; j += 256) {
            const float* pc = cp + (size_t)NP * j;
            col_finish<DT>(sm, j, (double)pc[0], (double)pc[1], F32 ? pc[2] : INFINITY,
                           F32 ? pc[3] : -INFINITY);
        }
        return;
    }
    // one partial row per workgroup
    const f32x4* c4 = reinterpret_cast<const f32x4*>(cp);
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(sm.part) + (size_t)wg * cols * NP);
    for (int j = threadIdx.x; j < cols * NP / 4; j += 256) gstore<f32x4>(dst + j, c4[j]);
}

template <int DT, int NVL, bool RAG>
hipError_t launch_wave(const SinqMat* mats, const int64_t* wgbeg, int nmat, int64_t n_wgs,
                       bool first, unsigned long long* nf, hipStream_t s) {
    // u, then the workgroup's partial row (wave mode: <= 4096 bf16 / 1536 fp32 columns)
    const size_t lds = WaveCfg<DT, NVL>::lds();
    const unsigned grid = (unsigned)n_wgs;
    if (first) k_sinq_wave<DT, NVL, true, RAG><<<dim3(grid), dim3(256), lds, s>>>(mats, wgbeg, nmat, nf);
    else k_sinq_wave<DT, NVL, false, RAG><<<dim3(grid), dim3(256), lds, s>>>(mats, wgbeg, nmat, nf);
    return hipGetLastError();
}

template <int DT, bool RAG>
hipError_t launch_wave_nv(const SinqMat* mats, const int64_t* wbeg, int nmat, int64_t n_waves,
                          int nvl, bool first, unsigned long long* nf, hipStream_t s) {
    switch (nvl) {
        case 1: return launch_wave<DT, 1, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 2: return launch_wave<DT, 2, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 3: return launch_wave<DT, 3, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 4: return launch_wave<DT, 4, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 5: return launch_wave<DT, 5, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 6: return launch_wave<DT, 6, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 7: return launch_wave<DT, 7, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        default: return launch_wave<DT, 8, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
    }
}

template <int DT>
hipError_t launch_wave_dt(const SinqMat* mats, const int64_t* wbeg, int nmat, int64_t n_waves,
                          SinqShape sh, bool first, unsigned long long* nf, hipStream_t s) {
    if (sh.rag) return launch_wave_nv<DT, true>(mats, wbeg, nmat, n_waves, sh.nv, first, nf, s);
    return launch_wave_nv<DT, false>(mats, wbeg, nmat, n_waves, sh.nv, first, nf, s);
}
// fp32 rows use the wave pass up to kWaveMaxF32 vectors per lane only.
template <bool RAG>
hipError_t launch_wave_f32(const SinqMat* mats, const int64_t* wbeg, int nmat, int64_t n_waves,
                           int nvl, bool first, unsigned long long* nf, hipStream_t s) {
    switch (nvl) {
        case 1: return launch_wave<WOQ_F32, 1, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        case 2: return launch_wave<WOQ_F32, 2, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
        default: return launch_wave<WOQ_F32, 3, RAG>(mats, wbeg, nmat, n_waves, first, nf, s);
    }
}

// Column combine: a workgroup takes 256 / S columns; S slices of threads
// each sum every S-th partial row (16 loads in flight), then the slice totals
// are added in slice order.  S (a power of two, 1..16) follows the number of
// partial rows, so each thread handles about 16 of them.  The summation order
// is fixed for a given launch plan, so results are deterministic.
constexpr int kRedInflight = 16;


template <int DT>
__global__ __launch_bounds__(256) void k_sinq_reduce(const SinqMat* __restrict__ mats,
                                                     const int64_t* __restrict__ cbeg, int nmat,
                                                     int slices) {
    __shared__ double sS[256], sQ[256];
    __shared__ float sMn[256], sMx[256];
    const int64_t u = blockIdx.x;
    const int m = find_unit_owner(cbeg, nmat, u);
    const SinqMat sm = mats[m];
    const int ncol = 256 / slices;
    const int c = threadIdx.x % ncol, sl = threadIdx.x / ncol;
    const int j = (int)(u - cbeg[m]) * ncol + c;
    double S = 0.0, Q = 0.0;
    float mn = INFINITY, mx = -INFINITY;
    if (j < sm.cols) {
        for (int g0 = sl; g0 < sm.n_strips; g0 += kRedInflight * slices) {
            if constexpr (DT == WOQ_F32) {
                float4 p[kRedInflight];
#pragma unroll
                for (int q = 0; q < kRedInflight; ++q) {
                    const int g = g0 + q * slices;
                    p[q] = g < sm.n_strips ? gload_f4(reinterpret_cast<const float4*>(sm.part) + (int64_t)g * sm.cols + j)
                                           : make_float4(0.f, 0.f, INFINITY, -INFINITY);
                }
#pragma unroll
                for (int q = 0; q < kRedInflight; ++q) {
                    S += (double)p[q].x;
                    Q += (double)p[q].y;
                    mn = fminf(mn, p[q].z);
                    mx = fmaxf(mx, p[q].w);
                }
            } else {
                float2 p[kRedInflight];
#pragma unroll
                for (int q = 0; q < kRedInflight; ++q) {
                    const int g = g0 + q * slices;
                    p[q] = g < sm.n_strips ? gload_f2(reinterpret_cast<const float2*>(sm.part) + (int64_t)g * sm.cols + j)
                                           : make_float2(0.f, 0.f);
                }
#pragma unroll
                for (int q = 0; q < kRedInflight; ++q) { S += (double)p[q].x; Q += (double)p[q].y; }
            }
        }
    }
    if (slices > 1) {
        sS[threadIdx.x] = S;
        sQ[threadIdx.x] = Q;
        sMn[threadIdx.x] = mn;
        sMx[threadIdx.x] = mx;
        __syncthreads();
        if (sl != 0) return;
        for (int q = 1; q < slices; ++q) {
            const int t = q * ncol + c;
            S += sS[t];
            Q += sQ[t];
            mn = fminf(mn, sMn[t]);
            mx = fmaxf(mx, sMx[t]);
        }
    }
    if (j >= sm.cols) return;
    col_finish<DT>(sm, j, S, Q, mn, mx);
}

template <int DT, int NV, bool RAG>
hipError_t launch_pass(const SinqMat* mats, const int64_t* sbeg, int nmat, int64_t n_strips,
                       int nt, int cols_max, bool first, unsigned long long* nf, hipStream_t s) {
    const size_t lds = PassCfg<DT, NV>::U_LDS ? sizeof(float) * ((size_t)cols_max + 8) : 0;
    if (first)
        k_sinq_pass<DT, NV, true, RAG><<<dim3((unsigned)n_strips), dim3(nt), lds, s>>>(mats, sbeg, nmat, nf);
    else
        k_sinq_pass<DT, NV, false, RAG><<<dim3((unsigned)n_strips), dim3(nt), lds, s>>>(mats, sbeg, nmat, nf);
    return hipGetLastError();
}

template <int DT, bool RAG>
hipError_t launch_pass_nv(const SinqMat* mats, const int64_t* sbeg, int nmat, int64_t n_strips,
                          SinqShape sh, int cols_max, bool first, unsigned long long* nf,
                          hipStream_t s) {
    switch (sh.nv) {
        case 1: return launch_pass<DT, 1, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 2: return launch_pass<DT, 2, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 3: return launch_pass<DT, 3, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 4: return launch_pass<DT, 4, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 5: return launch_pass<DT, 5, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 6: return launch_pass<DT, 6, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        case 7: return launch_pass<DT, 7, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
        default: return launch_pass<DT, 8, RAG>(mats, sbeg, nmat, n_strips, sh.nt, cols_max, first, nf, s);
    }
}

template <int DT>
hipError_t launch_pass_dt(const SinqMat* mats, const int64_t* sbeg, int nmat, int64_t n_strips,
                          SinqShape sh, int cols_max, bool first, unsigned long long* nf,
                          hipStream_t s) {
    if (sh.rag) return launch_pass_nv<DT, true>(mats, sbeg, nmat, n_strips, sh, cols_max, first, nf, s);
    return launch_pass_nv<DT, false>(mats, sbeg, nmat, n_strips, sh, cols_max, first, nf, s);
}

}  // namespace

// Wider rows: bf16 rows of at most 8192 columns take NV = ceil(vectors / 128)
// (up to 128 threads, four workgroups per CU); otherwise NV = ceil(vectors /
// 256) (up to 256 threads, two workgroups per CU) while that is <= 8 (bf16)
// or 4 (fp32), else ceil(vectors / 512) (up to 512 threads).  NT is the
// smallest multiple of 64 covering the row, e.g. 8192 columns -> 128 threads
// x 8 vectors, 14336 columns -> 256 threads x 7 vectors.
SinqShape sinq_shape(int cols, int dtype) {
    const int nvec = cols / 8;
    if (cols <= (dtype == WOQ_BF16 ? 4096 : 1536)) {
        const int nvl = (nvec + 63) / 64;
        return SinqShape{256, nvl < 1 ? 1 : nvl, 1, (nvec % 64) != 0};
    }
    if (dtype == WOQ_BF16 && nvec <= 1024) {
        // at most 8192 bf16 columns: two-wave workgroups of up to 8 vectors
        // per thread (70B stack, 8192 columns: the Sinkhorn step 596 ms per
        // pass against 630 with 256 threads x 4 vectors)
        const int nv = (nvec + 127) / 128;
        const int nt = ((nvec + nv - 1) / nv + 63) / 64 * 64;
        return SinqShape{nt, nv, 0, nt * nv != nvec};
    }
    int nv = (nvec + 255) / 256;
    if (nv > (dtype == WOQ_BF16 ? 8 : 4)) nv = (nvec + 511) / 512;
    if (nv < 1) nv = 1;
    const int nt = ((nvec + nv - 1) / nv + 63) / 64 * 64;
    return SinqShape{nt, nv, 0, nt * nv != nvec};
}

int sinq_tile_rows(int dtype, int nv) { return tile_rows(dtype, nv); }

int sinq_wave_occupancy(int, int) { return 2; }

int sinq_reduce_slices(int max_strips) {
    int sl = 1;
    while (sl < 16 && sl * kRedInflight < max_strips) sl *= 2;
    return sl;
}

hipError_t sinq_iteration(const SinqMat* mats, const int64_t* sbeg, const int64_t* cbeg, int nmat,
                          int64_t n_strips, int64_t n_col_units, int max_strips, int dtype,
                          SinqShape sh, int cols_max, bool first, unsigned long long* nonfinite,
                          hipStream_t s) {
    hipError_t e;
    unsigned long long* nf = nonfinite;
    if (sh.mode == 1)
        e = dtype == WOQ_BF16 ? launch_wave_dt<WOQ_BF16>(mats, sbeg, nmat, n_strips, sh, first, nf, s)
                              : (sh.rag ? launch_wave_f32<true>(mats, sbeg, nmat, n_strips, sh.nv, first, nf, s)
                                        : launch_wave_f32<false>(mats, sbeg, nmat, n_strips, sh.nv, first, nf, s));
    else
        e = dtype == WOQ_BF16
                ? launch_pass_dt<WOQ_BF16>(mats, sbeg, nmat, n_strips, sh, cols_max, first, nf, s)
                : launch_pass_dt<WOQ_F32>(mats, sbeg, nmat, n_strips, sh, cols_max, first, nf, s);
    if (e != hipSuccess) return e;
    if (n_col_units == 0) return hipSuccess;   // every matrix finished by its sweep
    const int slices = sinq_reduce_slices(max_strips);
    if (dtype == WOQ_BF16)
        k_sinq_reduce<WOQ_BF16><<<dim3((unsigned)n_col_units), dim3(256), 0, s>>>(mats, cbeg, nmat, slices);
    else
        k_sinq_reduce<WOQ_F32><<<dim3((unsigned)n_col_units), dim3(256), 0, s>>>(mats, cbeg, nmat, slices);
    return hipGetLastError();
}

}  // namespace woq
