// ar_pipe.hip -- the ring with the simple protocol between logical ranks,
// for gfx950 (MI355X).
//
// Each logical rank q has its own workgroups (workgroup w plays rank
// w mod R, so with R = 8 and the round-robin dispatch of workgroups over the
// 8 XCDs, rank q's workgroups share one XCD and its L2).  A segment is cut
// into flagged chunks; chunk k of every segment is always handled by the
// same workgroup index g = k mod G of whichever rank holds it, so a chunk
// passes point to point from workgroup (q-1, g) to workgroup (q, g).
//
// Simple protocol per chunk: the producer's threads store the chunk, every
// wave issues an agent-scope release fence (on gfx950: write back the L2 and
// wait for its own stores), the workgroup meets at a barrier, and one thread
// stores the chunk's ready flag coherently; the consumer's thread polls the
// flag with relaxed agent-scope loads, takes one agent-scope acquire fence
// when it matches (invalidating stale L1/L2 lines), and the workgroup meets
// at a barrier before reading the chunk.
// The ordering rules follow the fence/quiet distinction ("Demystifying
// NVSHMEM ..." summary: a fence orders, only a completed release makes data
// visible to the target).
//
// Flags are 64-bit and never reset: between calls every chunk's flag holds
// at most `base`, a call of n steps publishes base+1 .. base+n, and the last
// workgroup to finish raises base by n.  A step-s consumer waits for a
// value >= base+s, which only this call's producers write.
//
// Step numbering: all-reduce steps s = 0 .. 2R-3 and reduce-scatter steps
// s = 0 .. R-2 handle segment c = (q - s - 2) mod R (reduce for s <= R-2,
// copy after); all-gather steps s = 0 .. R-1 handle segment c = (q - s) mod R
// (step 0 places the rank's own shard, then copies).
//
// All R*G workgroups must be resident together; the host sizes the grid by
// the occupancy limit, and every wait is bounded in time.
#include <algorithm>

#include "ar_elem.h"
#include "ar_internal.h"
#include "ar_slots.h"

namespace ar {
namespace {

// Poll a ready flag with relaxed agent-scope loads; one acquire fence once it
// has the wanted value (so the cache invalidation happens once, not per poll).
__device__ inline bool wait_flag(const uint64_t* flag, uint64_t want, uint64_t deadline,
                                 const uint32_t* err)
{
    for (uint32_t spin = 0;; ++spin) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            return true;
        }
        if ((spin & 31u) == 31u) {
            if ((uint64_t)wall_clock64() > deadline)
                return false;
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
                return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int DT, int V, int OP>
__global__ __launch_bounds__(kBlock) void k_ring_pipelined(RingArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int R = a.R;
    const int q = blockIdx.x % R;
    const int g = blockIdx.x / R;
    const int G = a.per_rank_wg;
    const int nsteps = (OP == kOpAllReduce) ? 2 * (R - 1) : (OP == kOpReduceScatter) ? R - 1 : R;
    uint32_t* err = &a.ctrl[kCtrlError];
    uint64_t* basep = reinterpret_cast<uint64_t*>(a.ctrl + kCtrlPipeBase);

    __shared__ uint64_t s_base, s_deadline;
    __shared__ int s_fail;
    if (threadIdx.x == 0) {
        s_base = __hip_atomic_load(basep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_deadline = (uint64_t)wall_clock64() + a.timeout_ticks;
        s_fail = 0;
    }
    __syncthreads();
    const uint64_t base = s_base;
    const uint64_t slot_step = (uint64_t)kBlock * kUnroll;
    T* out = static_cast<T*>(a.out);

    for (int s = 0; s < nsteps; ++s) {
        const int c = (OP == kOpAllGather) ? mod_r(q - s, R) : mod_r(q - s - 2, R);
        const uint64_t lo = seg_lo(a.N, a.S, c), hi = seg_lo(a.N, a.S, c + 1);
        const uint64_t len = hi - lo;
        for (uint64_t k = (uint64_t)g; k < a.nunits; k += (uint64_t)G) {
            const uint64_t ulo = k * a.unit;
            if (ulo >= len)
                break;  // a short trailing segment has fewer chunks (same for every rank)
            const uint64_t ulen = min(a.unit, len - ulo);
            uint64_t* flag = a.flags + (uint64_t)c * a.flag_stride + k;
            if (s > 0) {
                if (threadIdx.x == 0 && !wait_flag(flag, base + (uint64_t)s, s_deadline, err))
                    s_fail = 1;
                __syncthreads();
            }
            const uint64_t nslots = (ulen + V - 1) / V;
            if (OP != kOpAllGather && s <= R - 2) {
                ReducePtrs<E> p = reduce_ptrs<E>(a, q, c, lo + ulo);
                if (OP == kOpReduceScatter)
                    p.dstT = static_cast<T*>(a.out) + (uint64_t)q * a.out_row + ulo;
                for (uint64_t j0 = threadIdx.x; j0 < nslots; j0 += slot_step)
                    reduce_step_slots<E, V>(p, s, R, ulen, j0, kBlock);
            } else if (OP == kOpAllGather && s == 0) {
                const T* src = static_cast<const T*>(a.send) + (uint64_t)q * a.send_row + ulo;
                T* dst = out + (uint64_t)q * a.out_row + lo + ulo;
                for (uint64_t j0 = threadIdx.x; j0 < nslots; j0 += slot_step)
                    copy_slots<E, V>(src, dst, ulen, j0, kBlock);
            } else {
                const int p = mod_r(q - 1, R);
                const T* src = out + (uint64_t)p * a.out_row + lo + ulo;
                T* dst = out + (uint64_t)q * a.out_row + lo + ulo;
                for (uint64_t j0 = threadIdx.x; j0 < nslots; j0 += slot_step)
                    copy_slots<E, V>(src, dst, ulen, j0, kBlock);
            }
            // publish: every wave releases its own stores at agent scope, the
            // workgroup meets, then one thread stores the flag
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_store(flag, base + (uint64_t)s + 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    __syncthreads();
    if (threadIdx.x == 0) {
        if (s_fail)
            __hip_atomic_fetch_or(err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kCtrlPipeDone], 1u, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.ctrl[kCtrlPipeDone], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(basep, base + (uint64_t)nsteps, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, int V>
hipError_t pipe_launch(const RingArgs& a, int grid, hipStream_t st)
{
    if (a.op == kOpAllReduce)
        hipLaunchKernelGGL((k_ring_pipelined<DT, V, kOpAllReduce>), dim3(grid), dim3(kBlock), 0,
                           st, a);
    else if (a.op == kOpReduceScatter)
        hipLaunchKernelGGL((k_ring_pipelined<DT, V, kOpReduceScatter>), dim3(grid), dim3(kBlock),
                           0, st, a);
    else
        hipLaunchKernelGGL((k_ring_pipelined<DT, V, kOpAllGather>), dim3(grid), dim3(kBlock), 0,
                           st, a);
    return hipGetLastError();
}

template <int DT>
int resident_pipe_dt(bool vec)
{
    int dev = 0, ncu = 0, per_cu = 0, per_cu2 = 0, per_cu3 = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    constexpr int VV = Elem<DT>::VEC;
    hipError_t e1, e2, e3;
    if (vec) {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_pipelined<DT, VV, kOpAllReduce>, kBlock, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, k_ring_pipelined<DT, VV, kOpReduceScatter>, kBlock, 0);
        e3 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu3, k_ring_pipelined<DT, VV, kOpAllGather>, kBlock, 0);
    } else {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_pipelined<DT, 1, kOpAllReduce>, kBlock, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, k_ring_pipelined<DT, 1, kOpReduceScatter>, kBlock, 0);
        e3 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu3, k_ring_pipelined<DT, 1, kOpAllGather>, kBlock, 0);
    }
    if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess)
        return 0;
    return std::min(per_cu, std::min(per_cu2, per_cu3)) * ncu;
}

}  // namespace

hipError_t launch_ring_pipelined(int dtype, bool vec, const RingArgs& a, int grid, hipStream_t st)
{
    switch (dtype) {
    case AR_INT32:
        return vec ? pipe_launch<AR_INT32, 4>(a, grid, st) : pipe_launch<AR_INT32, 1>(a, grid, st);
    case AR_FLOAT32:
        return vec ? pipe_launch<AR_FLOAT32, 4>(a, grid, st) : pipe_launch<AR_FLOAT32, 1>(a, grid, st);
    case AR_BF16:
        return vec ? pipe_launch<AR_BF16, 8>(a, grid, st) : pipe_launch<AR_BF16, 1>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

int resident_ring_pipelined(int dtype, bool vec)
{
    switch (dtype) {
    case AR_INT32:
        return resident_pipe_dt<AR_INT32>(vec);
    case AR_FLOAT32:
        return resident_pipe_dt<AR_FLOAT32>(vec);
    case AR_BF16:
        return resident_pipe_dt<AR_BF16>(vec);
    }
    return 0;
}

}  // namespace ar
