// ar_ll.h -- the LL protocol's line store and polling waits, shared by the
// tree (ar_tree.hip) and the ring with LL (ar_ring_ll.hip).
//
// An LL line is 8 bytes: the data bits in the low half and the arrival flag
// in the high half, written and read as one 64-bit agent-scope atomic, so a
// reader that sees the flag also sees the data ("Demystifying NVSHMEM ..."
// summary, paragraph on collectives: data and flag in one atomic write).
#pragma once

#include "ar_elem.h"

namespace ar {

// s_waitcnt vmcnt(0), leaving the other counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ inline void ll_store(uint64_t* line, uint32_t data, uint32_t flag)
{
    __hip_atomic_store(line, ((uint64_t)flag << 32) | (uint64_t)data, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for K lines at once, without per-lane branches in the poll: every
// pass loads line k in every lane of a wave in which any lane waits for it
// (a lane that does not, want[k] == false, must still hold a valid address;
// its value is ignored), then checks all flags.  Line k is skipped as a whole
// (a scalar branch) when no lane of the wave waits for it, so a short message
// polls one line, not K.  A line that has arrived keeps its value for the
// rest of the call (one writer per call), so loading it again is harmless; a
// pass is a handful of instructions, so a line is seen soon after it lands.
// Gives up (returns false) when `deadline` passes or the error word is set.
template <int K>
__device__ inline bool ll_wait_all(const uint64_t* const (&line)[K], const bool (&want)[K],
                                   const uint32_t (&flag)[K], uint64_t deadline,
                                   const uint32_t* err, uint32_t (&data)[K])
{
    bool live[K];  // wave-uniform
#pragma unroll
    for (int k = 0; k < K; ++k)
        live[k] = __builtin_amdgcn_ballot_w64(want[k]) != 0;
    for (uint32_t spin = 0;; ++spin) {
        uint64_t v[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            v[k] = live[k] ? __hip_atomic_load(line[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        bool done = true;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            done &= !want[k] || (uint32_t)(v[k] >> 32) == flag[k];
            data[k] = (uint32_t)v[k];
        }
        if (done)
            return true;
        if ((spin & 63u) == 63u) {
            if ((uint64_t)wall_clock64() > deadline)
                return false;
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
                return false;
            __builtin_amdgcn_s_sleep(1);
        }
    }
}

// The same with one flag for every line.
template <int K>
__device__ inline bool ll_wait_batch(const uint64_t* const (&line)[K], const bool (&want)[K],
                                     uint32_t flag, uint64_t deadline, const uint32_t* err,
                                     uint32_t (&data)[K])
{
    uint32_t f[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        f[k] = flag;
    return ll_wait_all<K>(line, want, f, deadline, err, data);
}

}  // namespace ar
