// Streaming ceilings of the GPU the pass runs on: how fast plain kernels with
// no arithmetic read HBM, copy through it, and re-read a buffer that stays in
// the on-package caches.  Built into a separate library (libwoq_probe.so)
// used by the benchmark only; it is not part of the quantisation library.
//
// Entry points (extern "C", plain device pointers, enqueued on `stream`):
//   probe_read(buf, bytes, passes, grid, chunked, sink, stream)
//       reads `bytes` (a multiple of 16) `passes` times in one launch of
//       `grid` workgroups of 256 threads, eight 16-byte loads in flight per
//       lane.  chunked = 0: grid-stride order (workgroup g, pass p reads
//       the same 4 KB rows every pass); chunked = 1: workgroup g reads one
//       contiguous 1/grid of the buffer per pass.  sink: device
//       uint32[grid * 256] (written, so the loads cannot be removed).
//   probe_copy(src, dst, bytes, grid, stream)
//       copies `bytes` (a multiple of 16) with the same grid-stride order.
//   probe_fma(out, iters, grid, stream)
//       `iters` dependent-chain steps of 8 independent fp32 FMAs per lane
//       (no packed fp32): the plain VALU issue rate.  out: device
//       float[grid * 256] (written).
//   probe_barrier(counters, err, n_bar, grid, team, spin_limit, mode, stream)
//       `n_bar` barriers among the workgroups of one cooperative launch of
//       `grid` workgroups of 256 threads: teams of `team` workgroups
//       (team = grid: a grid-wide barrier).  Teams are strided: workgroup b
//       is in team b mod (grid / team), so when grid / team is a multiple of
//       8 and workgroups are dealt to the 8 XCDs in turn, each team sits on
//       one XCD.  Each arrival is an
//       agent-scope atomic add on the team's counter (mode 2: first on one
//       of eight sub-counters); each wait polls it with agent-scope loads
//       (mode 0: acquire loads; modes 1-3: relaxed loads, then one acquire
//       fence; mode 3 adds a release and an acquire by every wave) and gives
//       up after spin_limit polls, setting *err and returning (so a launch
//       that cannot meet never hangs).  Mode 2 needs team % 8 == 0.
//       counters: device uint32[grid / team * 9 * 64] (zeroed by the caller);
//       err: device uint32 (zeroed by the caller).
// Each returns the hipError_t of its launch (0 = success) and -1 on an
// argument error (NULL pointer, a size not a multiple of 16, grid < 1 or
// passes < 1), checked before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kU = 8;       // 16-byte loads in flight per lane
constexpr int kT = 256;     // threads per workgroup

// Hides the pointer's value from the optimiser so that a later pass cannot
// reuse the loads of an earlier one (no memory access, scalar registers).
__device__ __forceinline__ const u32x4* launder(const u32x4* p) {
    uintptr_t v = reinterpret_cast<uintptr_t>(p);
    asm volatile("" : "+s"(v));
    return reinterpret_cast<const u32x4*>(v);
}

__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    typedef const __attribute__((address_space(1))) u32x4* gptr;
    return *(gptr)p;
}

__global__ __launch_bounds__(kT) void k_read_stride(const u32x4* buf, int64_t n16, int passes,
                                                    uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kT;
    const int64_t tid = (int64_t)blockIdx.x * kT + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int ps = 0; ps < passes; ++ps) {
        const u32x4* p = launder(buf);
        int64_t i = tid;
        for (; i + (kU - 1) * stride < n16; i += kU * stride) {
            u32x4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = ld(p + i + u * stride);
#pragma unroll
            for (int u = 0; u < kU; ++u) acc ^= v[u];
        }
        for (; i < n16; i += stride) acc ^= ld(p + i);
    }
    sink[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kT) void k_read_chunk(const u32x4* buf, int64_t n16, int passes,
                                                   uint32_t* sink) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b = (int64_t)blockIdx.x * per;
    const int64_t e = b + per < n16 ? b + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int ps = 0; ps < passes; ++ps) {
        const u32x4* p = launder(buf);
        int64_t i = b + threadIdx.x;
        for (; i + (kU - 1) * kT < e; i += kU * kT) {
            u32x4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = ld(p + i + u * kT);
#pragma unroll
            for (int u = 0; u < kU; ++u) acc ^= v[u];
        }
        for (; i < e; i += kT) acc ^= ld(p + i);
    }
    sink[(int64_t)blockIdx.x * kT + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kT) void k_copy(const u32x4* src, u32x4* dst, int64_t n16) {
    typedef __attribute__((address_space(1))) u32x4* gptr;
    const int64_t stride = (int64_t)gridDim.x * kT;
    int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
    for (; i + (kU - 1) * stride < n16; i += kU * stride) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = ld(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kU; ++u) *(gptr)(dst + i + u * stride) = v[u];
    }
    for (; i < n16; i += stride) *(gptr)(dst + i) = ld(src + i);
}

__global__ __launch_bounds__(kT) void k_fma(float* out, int iters) {
    const int64_t tid = (int64_t)blockIdx.x * kT + threadIdx.x;
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = (float)(threadIdx.x + k) * 1e-3f;
    const float m = 0.999f, c = 1e-4f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += a[k];
    out[tid] = s;
}

// Teams are strided: workgroup b belongs to team b % n_teams, and its rank
// among the team is b / n_teams.  Counters sit 256 bytes apart; a team's
// eight sub-counters (mode 2) follow its counter, 256 bytes apart too.
//   mode 0: arrival = release add on the team counter; each poll is an
//           acquire load (every poll invalidates the XCD's L2);
//   mode 1: the same arrival; relaxed polls, then one acquire fence;
//   mode 2: mode 1 with two-level arrival: rank r adds to sub-counter r % 8
//           (acquire-release), and the last of each sub-counter's arrivals
//           adds to the team counter, so at most team / 8 + 8 adds meet on
//           any one address;
//   mode 3: mode 1, and every wave releases at agent scope before the
//           workgroup barrier and acquires after it.  The workgroup barrier
//           compiles to a bare s_barrier (no wait for the other waves'
//           stores), so one thread's release publishes only its own wave's
//           writes: a step that hands data written by all waves to other
//           workgroups needs this form.
__global__ __launch_bounds__(kT) void k_barrier(unsigned* counters, unsigned* err, int n_bar,
                                                int team, unsigned spin_limit, int mode) {
    const unsigned n_teams = gridDim.x / (unsigned)team;
    const unsigned tm = blockIdx.x % n_teams, rank = blockIdx.x / n_teams;
    unsigned* c = counters + tm * 9u * 64u;
    unsigned* sub = c + 64u * (1u + rank % 8u);
    const unsigned per_sub = (unsigned)team / 8u;
    __shared__ unsigned bad;
    for (int b = 1; b <= n_bar; ++b) {
        if (mode == 3) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0) {
            bad = 0;
            unsigned target = (unsigned)b * (unsigned)team;
            if (mode == 2) {
                const unsigned old =
                    __hip_atomic_fetch_add(sub, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                if (old + 1u == (unsigned)b * per_sub)
                    __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                target = (unsigned)b * 8u;
            } else {
                __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
            unsigned spins = 0;
            for (;;) {
                const unsigned v = mode == 0
                                       ? __hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                                       : __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v >= target) break;
                if (++spins > spin_limit ||
                    __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    bad = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (mode != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (mode == 3) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (bad) return;
    }
}

}  // namespace

extern "C" {

int probe_read(const void* buf, size_t bytes, int passes, int grid, int chunked, uint32_t* sink,
               hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 || grid < 1 || passes < 1) return -1;
    const int64_t n16 = (int64_t)(bytes / 16);
    const u32x4* p = static_cast<const u32x4*>(buf);
    if (chunked)
        k_read_chunk<<<dim3((unsigned)grid), dim3(kT), 0, stream>>>(p, n16, passes, sink);
    else
        k_read_stride<<<dim3((unsigned)grid), dim3(kT), 0, stream>>>(p, n16, passes, sink);
    return (int)hipGetLastError();
}

int probe_copy(const void* src, void* dst, size_t bytes, int grid, hipStream_t stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 || grid < 1) return -1;
    k_copy<<<dim3((unsigned)grid), dim3(kT), 0, stream>>>(static_cast<const u32x4*>(src),
                                                          static_cast<u32x4*>(dst),
                                                          (int64_t)(bytes / 16));
    return (int)hipGetLastError();
}

int probe_barrier(unsigned* counters, unsigned* err, int n_bar, int grid, int team,
                  unsigned spin_limit, int mode, hipStream_t stream) {
    if (!counters || !err || n_bar < 1 || grid < 1 || team < 1 || grid % team || spin_limit < 1 ||
        mode < 0 || mode > 3 || (mode == 2 && team % 8))
        return -1;
    void* args[] = {&counters, &err, &n_bar, &team, &spin_limit, &mode};
    return (int)hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_barrier), dim3((unsigned)grid),
                                           dim3(kT), args, 0, stream);
}

int probe_fma(float* out, int iters, int grid, hipStream_t stream) {
    if (!out || iters < 1 || grid < 1) return -1;
    k_fma<<<dim3((unsigned)grid), dim3(kT), 0, stream>>>(out, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
