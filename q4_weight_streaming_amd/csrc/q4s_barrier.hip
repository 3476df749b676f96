// Grid-barrier measurement kernels: the cost of the barriers that separate the
// dependent phases of a chained decode step.  Persistent cooperative launches;
// every poll is bounded (past the limit the workgroup records an error and
// leaves), so no launch can hang.  Scratch layout, in 128-byte lines: line 0
// holds the counter or release word (word 0) and the error flag (word 1);
// line 1 the top counter of the tree; lines 2.. one line per workgroup.
//  * kind 0: the monotonic arrival counter of milestone M19 of the "minfer"
//    README -- one device-scope atomic add per arrival on one word; every
//    workgroup polls it with acquire loads until the phase is complete;
//  * kind 1: each workgroup stores its phase number into its own line,
//    workgroup 0 polls all lines with its 256 threads, then stores the
//    release word that the others poll;
//  * kind 2: a combining tree of monotonic counters: workgroup b arrives on
//    sub-counter b mod 16 (one line each), the last arrival of a sub-counter
//    arrives on the top counter, the last arrival there stores the release
//    word; polls are relaxed loads followed by one acquire fence;
//  * kind 3: kind 0 with relaxed polls, one acquire fence and no sleep;
//  * kinds 4, 5, 6: kind 2 with each sub-counter in its own 1 KB, 4 KB or
//    64 KB slot (so the slots fall into different memory channels), and a
//    copy of the release word in every slot: the last arrival at the top
//    stores all copies and each workgroup polls the copy of its sub-counter;
//  * kind 7: kind 2 with relaxed arrivals (no release fence) and one acquire
//    fence after the poll; kind 8: kind 2 with no fence at all; kind 9: kind 0
//    with no fence at all.  These measure what the fences cost; they order no
//    data and are not barriers a data-carrying phase may rely on.
#include <algorithm>

#include "q4s_device.h"

namespace q4s {
namespace {

constexpr int64_t kSpinLimit = 1 << 22;
constexpr int kLine = 32;     // words per 128-byte line
constexpr int kTreeFan = 16;  // sub-counters of the tree
constexpr int kSpreadBase = 2 * kLine;  // first word of the spread slots

// words per slot of kinds 4, 5, 6
inline int64_t spread_slot_words(int kind) { return kind == 4 ? 256 : (kind == 5 ? 1024 : 16384); }

__global__ __launch_bounds__(256) void k_barrier_zero(uint32_t* w, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) w[i] = 0;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* w, bool acquire) {
    return acquire ? __hip_atomic_load(w, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                   : __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *w >= target; false (and the error flag set) past the spin limit.
template <bool kAcquirePoll, bool kSleep>
__device__ bool wait_geq(const uint32_t* w, uint32_t target, uint32_t* err) {
    int64_t spins = 0;
    while (ld_agent(w, kAcquirePoll) < target) {
        if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        if (kSleep) __builtin_amdgcn_s_sleep(1);
    }
    if (!kAcquirePoll) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

template <bool kAcquirePoll, bool kSleep>
__global__ __launch_bounds__(256) void k_grid_barrier(uint32_t* scratch, int phases) {
    __shared__ int failed;
    uint32_t* counter = scratch;
    uint32_t* err = scratch + 1;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            if (!wait_geq<kAcquirePoll, kSleep>(counter, (uint32_t)(p + 1) * gridDim.x, err)) failed = 1;
        }
        __syncthreads();
        if (failed) return;
    }
}

__global__ __launch_bounds__(256) void k_grid_barrier_flags(uint32_t* scratch, int phases) {
    __shared__ int failed;
    uint32_t* release = scratch;
    uint32_t* err = scratch + 1;
    uint32_t* flags = scratch + 2 * kLine;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        const uint32_t gen = (uint32_t)p + 1;
        if (threadIdx.x == 0)
            __hip_atomic_store(flags + (int64_t)blockIdx.x * kLine, gen, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (blockIdx.x == 0) {
            // every thread watches its share of the lines
            for (int i = threadIdx.x; i < (int)gridDim.x; i += 256)
                if (!wait_geq<true, true>(flags + (int64_t)i * kLine, gen, err)) {
                    failed = 1;
                    break;
                }
            __syncthreads();
            if (threadIdx.x == 0 && !failed)
                __hip_atomic_store(release, gen, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else if (threadIdx.x == 0) {
            if (!wait_geq<true, true>(release, gen, err)) failed = 1;
        }
        __syncthreads();
        if (failed) return;
    }
}

template <int kArrive, bool kFence>
__device__ __forceinline__ uint32_t arrive(uint32_t* w) {
    return __hip_atomic_fetch_add(w, 1u, kArrive, __HIP_MEMORY_SCOPE_AGENT);
}

template <int kArrive, bool kFence>
__global__ __launch_bounds__(256) void k_grid_barrier_tree(uint32_t* scratch, int phases) {
    __shared__ int failed;
    uint32_t* release = scratch;
    uint32_t* err = scratch + 1;
    uint32_t* top = scratch + kLine;
    const int n = (int)gridDim.x;
    const int fan = n < kTreeFan ? n : kTreeFan;
    const int sub = (int)blockIdx.x % fan;
    const uint32_t sub_size = (uint32_t)((n - sub + fan - 1) / fan);  // workgroups b < n with b mod fan == sub
    uint32_t* mine = scratch + (int64_t)(2 + sub) * kLine;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        const uint32_t gen = (uint32_t)p + 1;
        if (threadIdx.x == 0) {
            const uint32_t old = arrive<kArrive, kFence>(mine);
            if (old + 1 == gen * sub_size) {
                const uint32_t t = arrive<kArrive, kFence>(top);
                if (t + 1 == gen * (uint32_t)fan)
                    __hip_atomic_store(release, gen, kArrive == __ATOMIC_RELAXED ? __ATOMIC_RELAXED : __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            int64_t spins = 0;
            while (ld_agent(release, false) < gen) {
                if (++spins > kSpinLimit) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    failed = 1;
                    break;
                }
            }
            if (kFence) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (failed) return;
    }
}

__global__ __launch_bounds__(256) void k_grid_barrier_nofence(uint32_t* scratch, int phases) {
    __shared__ int failed;
    uint32_t* counter = scratch;
    uint32_t* err = scratch + 1;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t target = (uint32_t)(p + 1) * gridDim.x;
            int64_t spins = 0;
            while (ld_agent(counter, false) < target) {
                if (++spins > kSpinLimit) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    failed = 1;
                    break;
                }
            }
        }
        __syncthreads();
        if (failed) return;
    }
}

// kinds 4..6: slot i holds sub-counter i (word 0) and release copy i (word kLine)
__global__ __launch_bounds__(256) void k_grid_barrier_spread(uint32_t* scratch, int phases, int64_t slot_words) {
    __shared__ int failed;
    uint32_t* err = scratch + 1;
    uint32_t* top = scratch + kLine;
    const int n = (int)gridDim.x;
    const int fan = n < kTreeFan ? n : kTreeFan;
    const int sub = (int)blockIdx.x % fan;
    const uint32_t sub_size = (uint32_t)((n - sub + fan - 1) / fan);
    uint32_t* slot = scratch + kSpreadBase + (int64_t)sub * slot_words;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        const uint32_t gen = (uint32_t)p + 1;
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(slot, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == gen * sub_size) {
                const uint32_t t = __hip_atomic_fetch_add(top, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                if (t + 1 == gen * (uint32_t)fan)
                    for (int i = 0; i < fan; ++i)
                        __hip_atomic_store(scratch + kSpreadBase + (int64_t)i * slot_words + kLine, gen,
                                           __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (!wait_geq<false, false>(slot + kLine, gen, err)) failed = 1;
        }
        __syncthreads();
        if (failed) return;
    }
}

}  // namespace

size_t grid_barrier_scratch_words(int n_wg) {
    return std::max<size_t>((size_t)kLine * (size_t)(n_wg + 2), kSpreadBase + kTreeFan * spread_slot_words(6));
}

hipError_t launch_grid_barrier(int kind, int n_wg, int phases, uint32_t* scratch, hipStream_t st) {
    const int64_t words = (int64_t)grid_barrier_scratch_words(n_wg);
    hipLaunchKernelGGL(k_barrier_zero, dim3((unsigned)std::min<int64_t>(64, (words + 255) / 256)), dim3(256), 0, st,
                       scratch, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const void* fn = kind == 0   ? (const void*)k_grid_barrier<true, true>
                     : kind == 1 ? (const void*)k_grid_barrier_flags
                     : kind == 2 ? (const void*)k_grid_barrier_tree<__ATOMIC_ACQ_REL, true>
                     : kind == 3 ? (const void*)k_grid_barrier<false, false>
                     : kind == 7 ? (const void*)k_grid_barrier_tree<__ATOMIC_RELAXED, true>
                     : kind == 8 ? (const void*)k_grid_barrier_tree<__ATOMIC_RELAXED, false>
                                 : (const void*)k_grid_barrier_nofence;
    if (kind >= 4 && kind <= 6) {
        int64_t slot_words = spread_slot_words(kind);
        void* args[] = {&scratch, &phases, &slot_words};
        return hipLaunchCooperativeKernel((const void*)k_grid_barrier_spread, dim3(n_wg), dim3(256), args, 0, st);
    }
    void* args[] = {&scratch, &phases};
    return hipLaunchCooperativeKernel(fn, dim3(n_wg), dim3(256), args, 0, st);
}

hipError_t grid_barrier_max_workgroups(int* n) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const void* fns[] = {(const void*)k_grid_barrier<true, true>, (const void*)k_grid_barrier_flags,
                         (const void*)k_grid_barrier_tree<__ATOMIC_ACQ_REL, true>,
                         (const void*)k_grid_barrier<false, false>, (const void*)k_grid_barrier_spread,
                         (const void*)k_grid_barrier_tree<__ATOMIC_RELAXED, true>,
                         (const void*)k_grid_barrier_tree<__ATOMIC_RELAXED, false>,
                         (const void*)k_grid_barrier_nofence};
    int per_cu = 1 << 30;
    for (const void* f : fns) {
        int c = 0;
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, f, 256, 0);
        per_cu = std::min(per_cu, c);
    }
    *n = e == hipSuccess ? cus * per_cu : 0;
    return e;
}

}  // namespace q4s
