// ar_slots.h -- the reduce-copy and copy inner loops shared by every ring
// kernel form (step-per-launch, fused, pipelined).
#pragma once

#include "ar_elem.h"
#include "ar_internal.h"

namespace ar {

// Reduce kUnroll slots j0 + u*jstep (u < kUnroll) of one segment of length
// len.  FIRST: the received value comes from the predecessor's input (T);
// else from its accumulator row (A).  LAST: the result is final and is
// narrowed to T; else it is this rank's accumulator.
// prevA and dstA are the same slots (a hop overwrites the running value in
// place), and dstT may be too: every slot is read before it is written, by the
// same thread, so no pointer here is restrict.  Callers guarantee j0 < the
// number of slots (the thread's first slot is in range).
template <class E, int V, bool FIRST, bool LAST, int RED>
__device__ inline void reduce_slots(const typename E::T* prevT, const typename E::A* prevA,
                                    const typename E::T* own, typename E::A* dstA,
                                    typename E::T* dstT, uint64_t len, uint64_t j0,
                                    uint64_t jstep, float R)
{
    using A = typename E::A;
    if constexpr (V == 1) {
        // One element per slot.  Every load is unconditional (a slot past the
        // end reads the thread's first slot again and is dropped) and all come
        // before the first store: a conditional load, or one after a store,
        // makes the compiler wait for every earlier store too (vmcnt counts
        // loads and stores in one in-order count).
        A xs[kUnroll], ys[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            const uint64_t jj = j < len ? j : j0;
            xs[u] = FIRST ? E::widen(prevT[jj]) : prevA[jj];
            ys[u] = E::widen(own[jj]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            if (j < len) {
                A r = combine<E, RED>(xs[u], ys[u]);
                if constexpr (LAST)
                    dstT[j] = E::narrow(finalize<E, RED>(r, R));
                else
                    dstA[j] = r;
            }
        }
        return;
    }
    A x[kUnroll][V], y[kUnroll][V];
    if ((j0 + (kUnroll - 1) * jstep + 1) * V <= len) {
        // every slot is whole: straight-line code, all loads in flight at once
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            if constexpr (FIRST)
                load_t<E, V>(prevT + j * V, x[u]);
            else
                load_a<E, V>(prevA + j * V, x[u]);
            load_t<E, V>(own + j * V, y[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                x[u][i] = combine<E, RED>(x[u][i], y[u][i]);
                if constexpr (LAST)
                    x[u][i] = finalize<E, RED>(x[u][i], R);
            }
            if constexpr (LAST)
                store_t<E, V>(dstT + j * V, x[u]);
            else
                store_a<E, V>(dstA + j * V, x[u]);
        }
        return;
    }
    // the end of a segment: whole slots, then the ragged last slot element by
    // element
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t j = j0 + (uint64_t)u * jstep;
        if ((j + 1) * V <= len) {
            if constexpr (FIRST)
                load_t<E, V>(prevT + j * V, x[0]);
            else
                load_a<E, V>(prevA + j * V, x[0]);
            load_t<E, V>(own + j * V, y[0]);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                x[0][i] = combine<E, RED>(x[0][i], y[0][i]);
                if constexpr (LAST)
                    x[0][i] = finalize<E, RED>(x[0][i], R);
            }
            if constexpr (LAST)
                store_t<E, V>(dstT + j * V, x[0]);
            else
                store_a<E, V>(dstA + j * V, x[0]);
        } else if (j * V < len) {
            for (uint64_t e = j * V; e < len; ++e) {
                A xv = FIRST ? E::widen(prevT[e]) : prevA[e];
                A r = combine<E, RED>(xv, E::widen(own[e]));
                if constexpr (LAST)
                    dstT[e] = E::narrow(finalize<E, RED>(r, R));
                else
                    dstA[e] = r;
            }
        }
    }
}

// Copy kUnroll slots of T from src to dst (bit copy).  Callers guarantee j0
// < the number of slots.
template <class E, int V>
__device__ inline void copy_slots(const typename E::T* __restrict__ src,
                                  typename E::T* __restrict__ dst, uint64_t len, uint64_t j0,
                                  uint64_t jstep)
{
    if constexpr (V == 1) {
        // loads first and unconditional (as in reduce_slots), then the stores
        typename E::T r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            r[u] = src[j < len ? j : j0];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            if (j < len)
                dst[j] = r[u];
        }
    } else {
        if ((j0 + (kUnroll - 1) * jstep + 1) * V <= len) {
            u32x4 r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                r[u] = *reinterpret_cast<const u32x4*>(src + (j0 + (uint64_t)u * jstep) * V);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                *reinterpret_cast<u32x4*>(dst + (j0 + (uint64_t)u * jstep) * V) = r[u];
            return;
        }
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * jstep;
            if ((j + 1) * V <= len) {
                *reinterpret_cast<u32x4*>(dst + j * V) = *reinterpret_cast<const u32x4*>(src + j * V);
            } else if (j * V < len) {
                for (uint64_t e = j * V; e < len; ++e)
                    dst[e] = src[e];
            }
        }
    }
}

// Row pointers of reduce step s for rank q, segment c = (q-(s+2)m) mod R.
template <class E>
struct ReducePtrs {
    const typename E::T* prevT;
    const typename E::A* prevA;
    const typename E::T* own;
    typename E::A* dstA;
    typename E::T* dstT;
};

template <class E>
__device__ inline ReducePtrs<E> reduce_ptrs(const RingArgs& a, int q, int c, uint64_t lo)
{
    using T = typename E::T;
    using A = typename E::A;
    const int p = mod_r(q - a.m, a.R);
    ReducePtrs<E> r;
    const T* send = static_cast<const T*>(a.send);
    A* part = static_cast<A*>(a.part);
    T* out = static_cast<T*>(a.out);
    r.prevT = send + (uint64_t)p * a.send_row + lo;
    r.prevA = part + (uint64_t)c * a.part_seg + lo;  // the hand-off from rank p ...
    r.own = send + (uint64_t)q * a.send_row + lo;
    r.dstA = part + (uint64_t)c * a.part_seg + lo;   // ... and to rank q + m: one slot
    // the final value (q == c): all-reduce writes it in place in the full
    // row; reduce-scatter at the same offset within rank c's shard row
    r.dstT = out + (uint64_t)q * a.out_row + (a.op == kOpReduceScatter ? lo - (uint64_t)c * a.S : lo);
    return r;
}

template <class E, int V, int RED>
__device__ inline void reduce_step_slots_op(const ReducePtrs<E>& p, int s, int R, uint64_t len,
                                            uint64_t j0, uint64_t jstep)
{
    const bool first = (s == 0), last = (s == R - 2);
    const float fr = (float)R;
    if (first && last)
        reduce_slots<E, V, true, true, RED>(p.prevT, p.prevA, p.own, p.dstA, p.dstT, len, j0, jstep, fr);
    else if (first)
        reduce_slots<E, V, true, false, RED>(p.prevT, p.prevA, p.own, p.dstA, p.dstT, len, j0, jstep, fr);
    else if (last)
        reduce_slots<E, V, false, true, RED>(p.prevT, p.prevA, p.own, p.dstA, p.dstT, len, j0, jstep, fr);
    else
        reduce_slots<E, V, false, false, RED>(p.prevT, p.prevA, p.own, p.dstA, p.dstT, len, j0, jstep, fr);
}

// The reduction operator is uniform per launch: one branch per step picks
// the code path.
template <class E, int V>
__device__ inline void reduce_step_slots(const ReducePtrs<E>& p, int s, int R, int redop,
                                         uint64_t len, uint64_t j0, uint64_t jstep)
{
    switch (redop) {
    case AR_MAX:
        reduce_step_slots_op<E, V, AR_MAX>(p, s, R, len, j0, jstep);
        break;
    case AR_MIN:
        reduce_step_slots_op<E, V, AR_MIN>(p, s, R, len, j0, jstep);
        break;
    case AR_AVG:
        reduce_step_slots_op<E, V, AR_AVG>(p, s, R, len, j0, jstep);
        break;
    default:
        reduce_step_slots_op<E, V, AR_SUM>(p, s, R, len, j0, jstep);
        break;
    }
}

}  // namespace ar
