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
// Simple protocol per chunk: the producer's threads store the chunk with
// device-scope (write-through) stores, every wave waits for its own stores
// to complete, the workgroup meets at a barrier, and one thread stores the
// chunk's ready flag coherently; the consumer's thread polls the flag with
// relaxed agent-scope loads, the workgroup meets at a barrier, and the chunk
// is read with device-scope loads.  Nothing is left dirty in an XCD's L2 for
// another XCD to miss, so no whole-cache writeback or invalidation is needed
// per chunk.
// The ordering rules follow the fence/quiet distinction ("Demystifying
// NVSHMEM ..." summary: a fence orders, only a completed release makes data
// visible to the target).
//
// Flags are 64-bit and never reset: between calls every chunk's flag holds
// at most `base`, a call of n steps publishes base+1 .. base+n, and the last
// workgroup to finish raises base by n.  A step-s consumer waits for a
// value >= base+s, which only this call's producers write.
//
// Step numbering (ring stride m, 1 for a single channel): all-reduce steps
// s = 0 .. 2R-3 and reduce-scatter steps s = 0 .. R-2 handle segment
// c = (q - (s+2)m) mod R (reduce for s <= R-2, copy after); all-gather steps
// s = 0 .. R-1 handle segment c = (q - s m) mod R (step 0 places the rank's
// own shard, then copies).
//
// All R*G workgroups must be resident together; the host sizes the grid by
// the occupancy limit, and every wait is bounded in time.
#include <algorithm>

#include "ar_elem.h"
#include "ar_internal.h"

namespace ar {
namespace {

// ---- device-scope coherent accesses ----------------------------------------
// Data that one logical rank writes and another reads inside this kernel goes
// through buffer instructions with the sc1 cache policy (device scope): a
// store is written through the XCD's L2 to the device's coherence point and
// is complete, for s_waitcnt, only once it is there; a load is served from
// the coherence point, never from a stale line of another XCD's L2.  So the
// producer needs only to wait for its own stores before the flag, and the
// consumer needs no cache invalidation -- no whole-L2 writeback per chunk.
// Each buffer resource covers exactly the chunk it addresses, so an access
// past the chunk is dropped by the hardware rather than reaching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCoherent = 16;  // sc1
constexpr int kPlain = 0;

__device__ inline rsrc_t make_rsrc(const void* p, uint64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                             (int)(bytes < 0x7fffffffull ? bytes : 0x7fffffffull),
                                             0x00020000);
}

// Wait until every memory access this wave issued has completed (stores
// included: on gfx950 they count in vmcnt).  Also a compiler barrier, so no
// store is moved past it.
__device__ inline void wait_own_stores() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

template <class E, int V, int POL>
__device__ inline void cload_t(rsrc_t r, uint32_t elem, typename E::A (&o)[V])
{
    using T = typename E::T;
    const uint32_t off = elem * (uint32_t)sizeof(T);
    if constexpr (V == 1) {
        if constexpr (sizeof(T) == 4)
            o[0] = E::from_bits(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL));
        else
            o[0] = E::widen((T)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POL));
    } else {
        u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = E::from_bits(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[2 * i] = E::widen((T)(w[i] & 0xffffu));
                o[2 * i + 1] = E::widen((T)(w[i] >> 16));
            }
        }
    }
}

template <class E, int V, int POL>
__device__ inline void cstore_t(rsrc_t r, uint32_t elem, const typename E::A (&v)[V])
{
    using T = typename E::T;
    const uint32_t off = elem * (uint32_t)sizeof(T);
    if constexpr (V == 1) {
        if constexpr (sizeof(T) == 4)
            __builtin_amdgcn_raw_buffer_store_b32(E::to_bits(v[0]), r, off, 0, POL);
        else
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)E::narrow(v[0]), r, off, 0, POL);
    } else {
        u32x4 w;
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = E::to_bits(v[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = (uint32_t)E::narrow(v[2 * i]) | ((uint32_t)E::narrow(v[2 * i + 1]) << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, POL);
    }
}

// A chunk's accumulators (4 bytes per element): slot j of V elements keeps
// its V/4 16-byte halves in runs of their own, half h of slot j at
// (h * nfull + j) * 16 bytes for the chunk's nfull whole slots, so one
// 16-byte-per-lane instruction covers whole lines.  For 32-bit T (V = 4)
// and on the scalar path (V = 1) this is plain element order.  The ragged
// end's elements follow at 4 bytes each, in element order.  Producer and
// consumer of a chunk have the same length, so they agree on the layout.
template <class E, int V, int POL>
__device__ inline void cload_a(rsrc_t r, uint32_t j, uint32_t nfull, typename E::A (&o)[V])
{
    if constexpr (V == 1) {
        o[0] = E::from_bits(__builtin_amdgcn_raw_buffer_load_b32(r, j * 4u, 0, POL));
        return;
    }
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, ((uint32_t)h * nfull + j) * 16u, 0, POL);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[4 * h + i] = E::from_bits(w[i]);
    }
}

template <class E, int V, int POL>
__device__ inline void cstore_a(rsrc_t r, uint32_t j, uint32_t nfull, const typename E::A (&v)[V])
{
    if constexpr (V == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(E::to_bits(v[0]), r, j * 4u, 0, POL);
        return;
    }
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = E::to_bits(v[4 * h + i]);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, ((uint32_t)h * nfull + j) * 16u, 0, POL);
    }
}

// One accumulator at element e (the scalar path and the ragged end).
template <class E, int POL>
__device__ inline typename E::A cload_a1(rsrc_t r, uint32_t e)
{
    return E::from_bits(__builtin_amdgcn_raw_buffer_load_b32(r, e * 4u, 0, POL));
}

template <class E, int POL>
__device__ inline void cstore_a1(rsrc_t r, uint32_t e, typename E::A v)
{
    __builtin_amdgcn_raw_buffer_store_b32(E::to_bits(v), r, e * 4u, 0, POL);
}

// Reduce one chunk of ulen elements: dst = prev + own.  prev is the
// predecessor's input (FIRST) or its accumulator row; dst is this rank's
// accumulator row or, at the last reduce step, its output (LAST).  Whole
// slots move as 16-byte vectors; the ragged end element by element.
template <class E, int V, bool FIRST, bool LAST, int RED>
__device__ inline void chunk_reduce(rsrc_t prev, rsrc_t own, rsrc_t dst, uint64_t ulen, float R)
{
    using A = typename E::A;
    constexpr int PREV_POL = FIRST ? kPlain : kCoherent;  // inputs predate the kernel
    const uint32_t nfull = (uint32_t)(ulen / V);
    for (uint32_t j0 = threadIdx.x; j0 < nfull; j0 += kBlock * kUnroll) {
        A x[kUnroll][V], y[kUnroll][V];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = j0 + u * kBlock;
            if (j < nfull) {
                if constexpr (FIRST)
                    cload_t<E, V, PREV_POL>(prev, j * V, x[u]);
                else
                    cload_a<E, V, PREV_POL>(prev, j, nfull, x[u]);
                cload_t<E, V, kPlain>(own, j * V, y[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = j0 + u * kBlock;
            if (j < nfull) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    x[u][i] = combine<E, RED>(x[u][i], y[u][i]);
                    if constexpr (LAST)
                        x[u][i] = finalize<E, RED>(x[u][i], R);
                }
                if constexpr (LAST)
                    cstore_t<E, V, kCoherent>(dst, j * V, x[u]);
                else
                    cstore_a<E, V, kCoherent>(dst, j, nfull, x[u]);
            }
        }
    }
    const uint32_t e = nfull * V + threadIdx.x;
    if (e < ulen) {
        A x[1], y[1];
        if constexpr (FIRST)
            cload_t<E, 1, PREV_POL>(prev, e, x);
        else
            x[0] = cload_a1<E, PREV_POL>(prev, e);
        cload_t<E, 1, kPlain>(own, e, y);
        x[0] = combine<E, RED>(x[0], y[0]);
        if constexpr (LAST) {
            x[0] = finalize<E, RED>(x[0], R);
            cstore_t<E, 1, kCoherent>(dst, e, x);
        } else {
            cstore_a1<E, kCoherent>(dst, e, x[0]);
        }
    }
}

template <class E, int V, int RED>
__device__ inline void chunk_reduce_step(bool first, bool last, rsrc_t prevT, rsrc_t prevA,
                                         rsrc_t own, rsrc_t dstA, rsrc_t dstT, uint64_t ulen,
                                         float R)
{
    if (first && last)
        chunk_reduce<E, V, true, true, RED>(prevT, own, dstT, ulen, R);
    else if (first)
        chunk_reduce<E, V, true, false, RED>(prevT, own, dstA, ulen, R);
    else if (last)
        chunk_reduce<E, V, false, true, RED>(prevA, own, dstT, ulen, R);
    else
        chunk_reduce<E, V, false, false, RED>(prevA, own, dstA, ulen, R);
}

// Copy one chunk of T (SRC_POL: kPlain when the source predates the kernel).
template <class E, int V, int SRC_POL>
__device__ inline void chunk_copy(rsrc_t src, rsrc_t dst, uint64_t ulen)
{
    using T = typename E::T;
    const uint32_t nfull = (uint32_t)(ulen / V);
    for (uint32_t j0 = threadIdx.x; j0 < nfull; j0 += kBlock * kUnroll) {
        u32x4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = j0 + u * kBlock;
            if (j < nfull)
                w[u] = __builtin_amdgcn_raw_buffer_load_b128(src, j * 16u, 0, SRC_POL);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = j0 + u * kBlock;
            if (j < nfull)
                __builtin_amdgcn_raw_buffer_store_b128(w[u], dst, j * 16u, 0, kCoherent);
        }
    }
    const uint32_t e = nfull * V + threadIdx.x;
    if (V > 1 && e < ulen) {
        if constexpr (sizeof(T) == 4)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_amdgcn_raw_buffer_load_b32(src, e * 4u, 0, SRC_POL), dst, e * 4u, 0, kCoherent);
        else
            __builtin_amdgcn_raw_buffer_store_b16(
                __builtin_amdgcn_raw_buffer_load_b16(src, e * 2u, 0, SRC_POL), dst, e * 2u, 0, kCoherent);
    }
}

template <class E, int V>
__device__ inline void chunk_copy_scalar(rsrc_t src, rsrc_t dst, uint64_t ulen, bool src_coherent)
{
    using T = typename E::T;
    for (uint32_t e = threadIdx.x; e < ulen; e += kBlock) {
        if constexpr (sizeof(T) == 4) {
            uint32_t v = src_coherent ? __builtin_amdgcn_raw_buffer_load_b32(src, e * 4u, 0, kCoherent)
                                      : __builtin_amdgcn_raw_buffer_load_b32(src, e * 4u, 0, kPlain);
            __builtin_amdgcn_raw_buffer_store_b32(v, dst, e * 4u, 0, kCoherent);
        } else {
            uint16_t v = src_coherent ? __builtin_amdgcn_raw_buffer_load_b16(src, e * 2u, 0, kCoherent)
                                      : __builtin_amdgcn_raw_buffer_load_b16(src, e * 2u, 0, kPlain);
            __builtin_amdgcn_raw_buffer_store_b16(v, dst, e * 2u, 0, kCoherent);
        }
    }
}

// Poll a ready flag with relaxed agent-scope loads (coherent, no cache
// invalidation).
__device__ inline bool wait_flag(const uint64_t* flag, uint64_t want, uint64_t deadline,
                                 const uint32_t* err)
{
    for (uint32_t spin = 0;; ++spin) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want)
            return true;
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
    using A = typename E::A;
    const int R = a.R;
    const int q = blockIdx.x % R;
    const int g = blockIdx.x / R;
    const int G = a.per_rank_wg;
    const int nsteps = (OP == kOpAllReduce) ? 2 * (R - 1) : (OP == kOpReduceScatter) ? R - 1 : R;
    uint32_t* err = &a.ctrl[kCtrlError];
    uint64_t* basep = reinterpret_cast<uint64_t*>(a.ctrl + kCtrlPipeBase);
    const T* send = static_cast<const T*>(a.send);
    A* part = static_cast<A*>(a.part);
    T* out = static_cast<T*>(a.out);

    __shared__ uint64_t s_base, s_deadline;
    __shared__ int s_fail;
    if (threadIdx.x == 0) {
        s_base = __hip_atomic_load(basep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_deadline = (uint64_t)wall_clock64() + a.timeout_ticks;
        s_fail = 0;
    }
    __syncthreads();
    const uint64_t base = s_base;
    const int m = a.m;
    const int p = mod_r(q - m, R);

    for (int s = 0; s < nsteps; ++s) {
        const int c = (OP == kOpAllGather) ? mod_r(q - s * m, R) : mod_r(q - (s + 2) * m, R);
        uint64_t lo, hi;
        seg_range(a.N, a.S, c, a.sub_lo, a.sub_len, &lo, &hi);
        const uint64_t len = hi - lo;
        for (uint64_t k = (uint64_t)g; k < a.nunits; k += (uint64_t)G) {
            const uint64_t ulo = k * a.unit;
            if (ulo >= len)
                break;  // a short trailing segment has fewer chunks (same for every rank)
            const uint64_t ulen = min(a.unit, len - ulo);
            const uint64_t e0 = lo + ulo;  // first element of the chunk in a full row
            uint64_t* flag = a.flags + (uint64_t)c * a.flag_stride + k;
            if (s > 0) {
                if (threadIdx.x == 0 && !wait_flag(flag, base + (uint64_t)s, s_deadline, err))
                    s_fail = 1;
                __syncthreads();
            }
            if (OP != kOpAllGather && s <= R - 2) {
                const bool first = (s == 0), last = (s == R - 2);
                const rsrc_t own = make_rsrc(send + (uint64_t)q * a.send_row + e0, ulen * sizeof(T));
                const rsrc_t prevT = make_rsrc(send + (uint64_t)p * a.send_row + e0, ulen * sizeof(T));
                // the hand-off slot: rank p wrote it, rank q overwrites it
                const rsrc_t accA = make_rsrc(part + (uint64_t)c * a.part_seg + e0, ulen * 4);
                const rsrc_t& prevA = accA;
                const rsrc_t& dstA = accA;
                T* dT = out + (uint64_t)q * a.out_row +
                        (OP == kOpReduceScatter ? e0 - (uint64_t)c * a.S : e0);
                const rsrc_t dstT = make_rsrc(dT, ulen * sizeof(T));
                const float fr = (float)R;
                switch (a.redop) {
                case AR_MAX:
                    chunk_reduce_step<E, V, AR_MAX>(first, last, prevT, prevA, own, dstA, dstT, ulen, fr);
                    break;
                case AR_MIN:
                    chunk_reduce_step<E, V, AR_MIN>(first, last, prevT, prevA, own, dstA, dstT, ulen, fr);
                    break;
                case AR_AVG:
                    chunk_reduce_step<E, V, AR_AVG>(first, last, prevT, prevA, own, dstA, dstT, ulen, fr);
                    break;
                default:
                    chunk_reduce_step<E, V, AR_SUM>(first, last, prevT, prevA, own, dstA, dstT, ulen, fr);
                    break;
                }
            } else {
                // a copy step; at all-gather step 0 the source is the rank's own
                // shard in send (written before the kernel), else the
                // predecessor's output row (written in this kernel)
                const bool placement = (OP == kOpAllGather && s == 0);
                const T* srcp = placement ? send + (uint64_t)q * a.send_row + (e0 - (uint64_t)q * a.S)
                                          : out + (uint64_t)p * a.out_row + e0;
                const rsrc_t src = make_rsrc(srcp, ulen * sizeof(T));
                const rsrc_t dst = make_rsrc(out + (uint64_t)q * a.out_row + e0, ulen * sizeof(T));
                if constexpr (V == 1)
                    chunk_copy_scalar<E, V>(src, dst, ulen, !placement);
                else if (placement)
                    chunk_copy<E, V, kPlain>(src, dst, ulen);
                else
                    chunk_copy<E, V, kCoherent>(src, dst, ulen);
            }
            // publish: each wave waits for its own (write-through) stores, the
            // workgroup meets, one thread stores the flag coherently
            wait_own_stores();
            __syncthreads();
            if (threadIdx.x == 0 && q != a.mute_rank)
                __hip_atomic_store(flag, base + (uint64_t)s + 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    __syncthreads();
    if (threadIdx.x == 0) {
        if (s_fail)
            __hip_atomic_fetch_or(err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        // Only the next launch on the stream reads the counter and the flag base, and
        // the kernel boundary orders this launch's memory before it, so relaxed
        // atomics suffice (acquire-release here would write back and invalidate
        // the XCD's L2 in every workgroup).
        uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kCtrlPipeDone], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.ctrl[kCtrlPipeDone], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(basep, base + (uint64_t)nsteps, __ATOMIC_RELAXED,
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
