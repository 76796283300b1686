// ar_ring_ll.hip -- the ring with the LL protocol, for gfx950 (MI355X).
//
// Same schedule as the other ring forms (R-1 reduce steps, then R-1 copy
// steps around q -> q+1; rank c owns segment c), but every value a rank
// passes to its successor travels as an 8-byte LL line: 4 bytes of data (the
// accumulator's bits, or T's bits zero-extended) and 4 bytes of flag, in one
// 64-bit atomic store ("Demystifying NVSHMEM ..." summary, paragraph on
// collectives: LL packs data and arrival flag into one atomic write).  No
// chunk flags, barriers or fences: each element carries its own arrival
// flag, and the consumer polls it.
//
// Line slot lines[q][c][i] is written by rank q for segment c.  In one call
// a slot may carry two values: the reduce-phase partial (flag 2*epoch) and,
// later, the copy-phase final (flag 2*epoch+1).  The final is only produced
// after the whole reduce chain of the segment has run, which includes the
// successor's read of the partial, so the overwrite never races the read.
// Each rank has its own workgroups (workgroup w plays rank w mod R), and the
// workgroup with index g of rank q handles the same element positions as the
// workgroup g of every other rank, so a line passes point to point.  All
// workgroups must be resident together (the host caps the grid); every wait
// is bounded by the kernel-wide deadline.
#include "ar_elem.h"
#include "ar_internal.h"
#include "ar_ll.h"

namespace ar {
namespace {

// The reduction operator is a template argument (the host picks the
// instantiation; the all-gather has none and takes AR_SUM).  K is the number
// of sub-blocks a thread takes per pass: 1 when every workgroup has at most
// one sub-block per step (small messages), else kRingLLEPT.  A step is
// latency-bound, and a lone wave issues about one instruction every few
// cycles, so the step's own instruction count is part of every hop: with
// K = 1 there is one line per lane and no per-line branches.
template <int DT, int OP, int RED, int K>
__global__ __launch_bounds__(kBlock) void k_ring_ll(RingLLArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    using A = typename E::A;
    const int R = a.R;
    // set g of R workgroups (one per rank), all on one XCD (ll_set_of)
    const uint32_t n = a.xcd_sets > 1 ? (uint32_t)a.xcd_sets : 1u;
    const int q = (int)ll_rank_of(blockIdx.x, n, (uint32_t)R);
    const int g = (int)ll_set_of(blockIdx.x, n, (uint32_t)R);
    const int G = a.per_rank_wg;
    const bool idle = g >= G;  // past the last set: no lines, only the done counter
    const int m = a.m;
    const int p = mod_r(q - m, R);
    const int nsteps = (OP == kOpAllReduce) ? 2 * (R - 1) : (OP == kOpReduceScatter) ? R - 1 : R;
    uint32_t* err = &a.ctrl[kCtrlError];

    // Every wave reads the epoch itself (no barrier), so the load overlaps the
    // first input loads; only the last workgroup to finish writes it.
    const uint32_t epoch = __hip_atomic_load(&a.ctrl[kCtrlRingLLEpoch], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const uint32_t f_red = 2u * epoch, f_copy = 2u * epoch + 1u;
    const uint64_t deadline = (uint64_t)wall_clock64() + a.timeout_ticks;
    const bool publish = (q != a.mute_rank);
    const T* send = static_cast<const T*>(a.send);
    T* out = static_cast<T*>(a.out);
    const float fr = (float)R;
    bool timed_out = false;

    // segment of step 0; every later step takes the one m below (no division)
    int c = (OP == kOpAllGather) ? q : mod_r(q - 2 * m, R);
    for (int s = 0; s < (idle ? 0 : nsteps); ++s, c = (c >= m) ? c - m : c - m + R) {
        uint64_t lo, hi;
        seg_range(a.N, a.S, c, a.sub_lo, a.sub_len, &lo, &hi);
        const uint64_t len = hi - lo;
        const uint64_t plen = a.piece_lo < len ? min(a.piece_len, len - a.piece_lo) : 0;
        const uint64_t e0 = lo + a.piece_lo;  // element of offset 0 in a full row
        const uint64_t in_seg = e0 - (uint64_t)c * a.S;  // its offset within segment c
        uint64_t* mine = a.lines + ((uint64_t)q * R + c) * a.piece_cap;
        const uint64_t* theirs = a.lines + ((uint64_t)p * R + c) * a.piece_cap;
        const bool reduce = (OP != kOpAllGather) && s <= R - 2;
        const bool last_reduce = reduce && s == R - 2;
        // the last receiver of a segment's final does not pass it on
        const bool forward = !reduce && (((c >= m) ? c - m : c - m + R) != q);
        // sub-blocks of kBlock offsets: sub-block j belongs to workgroup j mod G
        // of every rank; a thread takes K of its workgroup's sub-blocks at once
        const uint64_t nsub = (plen + kBlock - 1) / kBlock;
        for (uint64_t j0 = (uint64_t)g; j0 < nsub; j0 += (uint64_t)G * K) {
            uint64_t i[K];
            bool ok[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                i[k] = (j0 + (uint64_t)k * G) * kBlock + threadIdx.x;
                ok[k] = i[k] < plen;
            }
            // Loads are unconditional (a lane past the end reads offset 0 of
            // the piece and never uses it) and all come before the first
            // store: with conditional loads, or a load after a store, the
            // compiler's waits would make each store wait for the ones before
            // it (vmcnt counts loads and stores in one in-order count).
            if (reduce) {
                A in[K];
                T own[K];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    own[k] = send[(uint64_t)q * a.send_row + e0 + (ok[k] ? i[k] : 0)];
                if (s == 0) {
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        in[k] = E::widen(send[(uint64_t)p * a.send_row + e0 + (ok[k] ? i[k] : 0)]);
                } else {
                    const uint64_t* ln[K];
                    uint32_t d[K];
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        ln[k] = theirs + (ok[k] ? i[k] : 0);
                    if (!ll_wait_batch<K>(ln, ok, f_red, deadline, err, d))
                        timed_out = true;
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        in[k] = E::from_bits(d[k]);
                }
                wait_vmem_all();  // on every path: nothing outstanding before the stores
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (!ok[k])
                        continue;
                    A v = combine<E, RED>(in[k], E::widen(own[k]));
                    if (!last_reduce) {
                        if (publish)
                            ll_store(mine + i[k], E::to_bits(v), f_red);
                    } else {
                        if constexpr (RED == AR_AVG)
                            v = finalize<E, AR_AVG>(v, fr);
                        if (OP == kOpAllReduce && publish)  // the owner starts the copy phase
                            ll_store(mine + i[k], E::to_bits(v), f_copy);
                        const uint64_t at = (OP == kOpReduceScatter) ? in_seg + i[k] : e0 + i[k];
                        out[(uint64_t)q * a.out_row + at] = E::narrow(v);
                    }
                }
            } else if (OP == kOpAllGather && s == 0) {
                // place the rank's own shard and pass it on (T bits)
                T v[K];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    v[k] = send[(uint64_t)q * a.send_row + in_seg + (ok[k] ? i[k] : 0)];
                wait_vmem_all();
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (!ok[k])
                        continue;
                    if (publish)
                        ll_store(mine + i[k], E::t_bits(v[k]), f_copy);
                    out[(uint64_t)q * a.out_row + e0 + i[k]] = v[k];
                }
            } else {
                const uint64_t* ln[K];
                uint32_t d[K];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    ln[k] = theirs + (ok[k] ? i[k] : 0);
                if (!ll_wait_batch<K>(ln, ok, f_copy, deadline, err, d))
                    timed_out = true;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (!ok[k])
                        continue;
                    if (forward && publish)  // pass it on first: the next rank waits for it
                        ll_store(mine + i[k], d[k], f_copy);
                    if (OP == kOpAllGather)
                        out[(uint64_t)q * a.out_row + e0 + i[k]] = E::t_from_bits(d[k]);
                    else
                        out[(uint64_t)q * a.out_row + e0 + i[k]] = E::narrow(E::from_bits(d[k]));
                }
            }
        }
    }
    if (timed_out)
        __hip_atomic_fetch_or(err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (threadIdx.x == 0) {
        // Only the next launch on the stream reads the counter and the epoch, and
        // the kernel boundary orders this launch's memory before it, so relaxed
        // atomics suffice (acquire-release here would write back and invalidate
        // the XCD's L2 in every workgroup).
        uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kCtrlRingLLDone], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.ctrl[kCtrlRingLLDone], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[kCtrlRingLLEpoch], epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, int OP, int K>
void ring_ll_launch_op(const RingLLArgs& a, int grid, hipStream_t st)
{
    switch (a.redop) {
    case AR_MAX:
        hipLaunchKernelGGL((k_ring_ll<DT, OP, AR_MAX, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    case AR_MIN:
        hipLaunchKernelGGL((k_ring_ll<DT, OP, AR_MIN, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    case AR_AVG:
        if constexpr (DT != AR_INT32)  // no integer average (refused by the host)
            hipLaunchKernelGGL((k_ring_ll<DT, OP, AR_AVG, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    default:
        hipLaunchKernelGGL((k_ring_ll<DT, OP, AR_SUM, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    }
}

template <int DT, int K>
void ring_ll_launch_k(const RingLLArgs& a, int grid, hipStream_t st)
{
    if (a.op == kOpAllReduce)
        ring_ll_launch_op<DT, kOpAllReduce, K>(a, grid, st);
    else if (a.op == kOpReduceScatter)
        ring_ll_launch_op<DT, kOpReduceScatter, K>(a, grid, st);
    else
        hipLaunchKernelGGL((k_ring_ll<DT, kOpAllGather, AR_SUM, K>), dim3(grid), dim3(kBlock), 0, st,
                           a);
}

template <int DT>
hipError_t ring_ll_launch(const RingLLArgs& a, int grid, hipStream_t st)
{
    // one sub-block per workgroup and step at most: one line per thread
    const uint64_t nsub = (a.piece_len + kBlock - 1) / kBlock;
    if (nsub <= (uint64_t)a.per_rank_wg)
        ring_ll_launch_k<DT, 1>(a, grid, st);
    else
        ring_ll_launch_k<DT, kRingLLEPT>(a, grid, st);
    return hipGetLastError();
}

template <int DT>
int resident_ring_ll_dt()
{
    int dev = 0, ncu = 0, a1 = 0, a2 = 0, a3 = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a1, k_ring_ll<DT, kOpAllReduce, AR_SUM, kRingLLEPT>, kBlock, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&a2, k_ring_ll<DT, kOpReduceScatter, AR_SUM, kRingLLEPT>, kBlock, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&a3, k_ring_ll<DT, kOpAllGather, AR_SUM, kRingLLEPT>, kBlock, 0) != hipSuccess)
        return 0;
    return min(a1, min(a2, a3)) * ncu;
}

}  // namespace

hipError_t launch_ring_ll(int dtype, const RingLLArgs& a, int grid, hipStream_t st)
{
    switch (dtype) {
    case AR_INT32:
        return ring_ll_launch<AR_INT32>(a, grid, st);
    case AR_FLOAT32:
        return ring_ll_launch<AR_FLOAT32>(a, grid, st);
    case AR_BF16:
        return ring_ll_launch<AR_BF16>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

int resident_ring_ll(int dtype)
{
    switch (dtype) {
    case AR_INT32:
        return resident_ring_ll_dt<AR_INT32>();
    case AR_FLOAT32:
        return resident_ring_ll_dt<AR_FLOAT32>();
    case AR_BF16:
        return resident_ring_ll_dt<AR_BF16>();
    }
    return 0;
}

}  // namespace ar
