// ar_ring.hip -- ring all-reduce / reduce-scatter / all-gather kernels for
// gfx950 (MI355X).
//
// The ring takes 2(R-1) steps ("GPU MODE lecture 68 notes", section 05,
// "SHARP -- in-network reduction").  Reading used here: R-1 reduce steps,
// then R-1 copy steps, around the ring q -> q+1.  Rank c owns segment c.
//   reduce step s (0..R-2), rank q, segment c = (q-s-2) mod R:
//       acc_q = (s == 0 ? x_{q-1} : acc_{q-1}) + x_q   over segment c;
//       at s = R-2 (q == c) the result is final and is written as T.
//   copy step s (0..R-2), rank q, segment c = (q-1-s) mod R:
//       y_q = y_{q-1} over segment c.
// So an element of segment c is the left fold x_{c+1} + x_{c+2} + ... + x_c.
// With several channels (the multi-rail idea, "GPU MODE lecture 68 notes",
// section 06: one channel per rail), each segment is cut into one sub-range
// per channel and channel k runs its own ring q -> q + m_k with a stride m_k
// coprime with R: every formula above with 1 replaced by m_k.
//
// All R logical ranks live in one HBM: rank q's buffers are row q of
// rank-major arrays, and "receiving from q-1" is reading row q-1 in place
// (the symmetric-heap idea of a remote address being a base plus the local
// offset: "Demystifying NVSHMEM ..." summary, paragraph on the symmetric
// heap).  A reduce step hands its running value to the next rank through one
// accumulator slot per element: rank q-1 stores it, rank q loads it, adds
// x_q and stores over it.  The slot is the owner's output row when the
// accumulator type is the element type (the final value then needs no extra
// row), else a workspace row.  Every step is a reduce-copy of two 16-byte
// vector loads and one 16-byte store per slot (a copy step: one load, one
// store); there is no MFMA because nothing here is a contraction.
//
// Two launch forms live in this file:
//   step  -- one launch per step over all R ranks; the kernel boundary
//            orders the steps.
//   fused, scalar path -- one persistent launch; a workgroup takes a tile of
//            a segment through all 2(R-1) steps in order, one element per
//            thread and step.  Each thread touches the same element positions
//            at every step, so the value it stored for rank q is the one it
//            loads back as rank q+1's input (same-thread program order; the
//            compiler is kept from forwarding it in registers, so every step
//            really reads the hand-off slot).  It serves views whose rows are
//            not 16-byte aligned and counts too small for a vector tile.
// The fused form's vector path (wave tiles, 16-byte buffer loads and stores)
// lives in ar_fused.hip; ar_comm.cpp chooses between the two paths per call.
// Tiles of a step are independent, so neither fused path has flags or
// fences; the slot a step writes is still hot in this XCD's L2 when the next
// step reads and overwrites it.
#include "ar_elem.h"
#include "ar_internal.h"
#include "ar_slots.h"

namespace ar {
namespace {

// ---- one launch per step --------------------------------------------------

// grid = (gx, R): blockIdx.y is the logical rank.
template <int DT, int V>
__global__ __launch_bounds__(kBlock) void k_ring_reduce_step(RingArgs a)
{
    using E = Elem<DT>;
    const int q = blockIdx.y;
    const int s = a.step;
    const int c = mod_r(q - (s + 2) * a.m, a.R);
    uint64_t lo, hi;
    seg_range(a.N, a.S, c, a.sub_lo, a.sub_len, &lo, &hi);
    const uint64_t len = hi - lo;
    const uint64_t nslots = (len + V - 1) / V;
    const ReducePtrs<E> p = reduce_ptrs<E>(a, q, c, lo);
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * kUnroll;
    for (uint64_t j0 = (uint64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; j0 < nslots;
         j0 += stride)
        reduce_step_slots<E, V>(p, s, a.R, a.redop, len, j0, kBlock);
}

template <int DT, int V>
__global__ __launch_bounds__(kBlock) void k_ring_copy_step(RingArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int q = blockIdx.y;
    const int s = a.step;
    const int c = mod_r(q - (1 + s) * a.m, a.R);
    const int p = mod_r(q - a.m, a.R);
    uint64_t lo, hi;
    seg_range(a.N, a.S, c, a.sub_lo, a.sub_len, &lo, &hi);
    const uint64_t len = hi - lo;
    const uint64_t nslots = (len + V - 1) / V;
    T* out = static_cast<T*>(a.out);
    const T* src = out + (uint64_t)p * a.out_row + lo;
    T* dst = out + (uint64_t)q * a.out_row + lo;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * kUnroll;
    for (uint64_t j0 = (uint64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; j0 < nslots;
         j0 += stride)
        copy_slots<E, V>(src, dst, len, j0, kBlock);
}

// All-gather: rank q places its own shard at segment q of its output row.
template <int DT, int V>
__global__ __launch_bounds__(kBlock) void k_ring_placement(RingArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int q = blockIdx.y;
    uint64_t lo, hi;
    seg_range(a.N, a.S, q, a.sub_lo, a.sub_len, &lo, &hi);
    const uint64_t len = hi - lo;
    const uint64_t nslots = (len + V - 1) / V;
    const T* src = static_cast<const T*>(a.send) + (uint64_t)q * a.send_row + (lo - (uint64_t)q * a.S);
    T* dst = static_cast<T*>(a.out) + (uint64_t)q * a.out_row + lo;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * kUnroll;
    for (uint64_t j0 = (uint64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; j0 < nslots;
         j0 += stride)
        copy_slots<E, V>(src, dst, len, j0, kBlock);
}

// ---- fused: a tile runs every step ------------------------------------------

// One reduce step of the scalar path (one element per slot; slot u of this
// thread is element e[u], stored only if ok[u]).  The same structure as
// fused_step: the hand-off is loaded after the previous step's store, the
// next step's input is prefetched into `nxt`, and `own` was prefetched one
// step earlier.  The empty asm takes the loaded hand-off values as operands,
// so the compiler waits for them right there (leaving the prefetch in
// flight) instead of moving each load into its store's branch and waiting
// for everything outstanding.
template <class E, int RED, int U, bool LOADX, bool PREFETCH, bool LAST>
__device__ inline void scalar_step(typename E::A (&x)[U], const typename E::T (&own)[U],
                                   typename E::T (&nxt)[U], typename E::A* acc,
                                   typename E::T* fin, const typename E::T* next_row,
                                   const uint64_t (&e)[U], const bool (&ok)[U], float R)
{
    using A = typename E::A;
    if constexpr (LOADX) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = acc[e[u]];
    }
    if constexpr (PREFETCH) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            nxt[u] = next_row[e[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        __asm__ __volatile__("" ::"v"(x[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) {
        A v = combine<E, RED>(x[u], E::widen(own[u]));
        if constexpr (LAST)
            v = finalize<E, RED>(v, R);
        if (U == 1 || ok[u]) {  // with one slot per thread, every active thread's slot is in range
            if constexpr (LAST)
                fin[e[u]] = E::narrow(v);
            else
                acc[e[u]] = v;
        }
        x[u] = v;
    }
    step_boundary();
}

// The R-1 reduce steps of a tile on the scalar path (segments shorter than
// one 128-byte line).  Each active thread has the U elements j0 + u*js of
// segment c (U = 1 when the tile has at most one element per thread); one
// past the end reads the thread's first element instead and stores nothing,
// so every load is unconditional.  As on the vector path, the input of the
// next step's rank is loaded before this step's store, into the other of two
// register sets, so its HBM latency overlaps the hand-off instead of adding
// to each step.  The rank whose row a step reads advances by m (no division:
// each step is latency-bound, and its instruction count is part of it).
template <class E, int RED, int U>
__device__ inline void fused_reduce_scalar(const RingArgs& a, int c, uint64_t lo, uint64_t len,
                                           uint64_t j0, uint64_t js)
{
    using T = typename E::T;
    using A = typename E::A;
    const int R = a.R;
    const int m = a.m;
    const float fr = (float)R;
    const T* send = static_cast<const T*>(a.send) + lo;
    A* acc = static_cast<A*>(a.part) + (uint64_t)c * a.part_seg + lo;
    T* fin = static_cast<T*>(a.out) + (uint64_t)c * a.out_row +
             (a.op == kOpReduceScatter ? lo - (uint64_t)c * a.S : lo);
    // x_{c+km}: the input of the rank that adds at step k-2; rk walks c+m, c+2m, ...
    int rk = c;
    auto next_row = [&]() {
        rk += m;
        if (rk >= R)
            rk -= R;
        return send + (uint64_t)rk * a.send_row;
    };
    uint64_t e[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t j = j0 + (uint64_t)u * js;
        ok[u] = j < len;
        e[u] = ok[u] ? j : j0;
    }
    A x[U];
    T b0[U], b1[U];
    const T* r1 = next_row();
    const T* r2 = next_row();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        x[u] = E::widen(r1[e[u]]);
        b0[u] = r2[e[u]];
    }
    if (R == 2) {
        scalar_step<E, RED, U, false, false, true>(x, b0, b1, acc, fin, nullptr, e, ok, fr);
        return;
    }
    // R >= 3: steps 0 .. R-3 hand off, step R-2 is the owner's
    scalar_step<E, RED, U, false, true, false>(x, b0, b1, acc, fin, next_row(), e, ok, fr);
    int s = 1;  // the next step; its input is in b1
    for (; s + 1 <= R - 3; s += 2) {
        scalar_step<E, RED, U, true, true, false>(x, b1, b0, acc, fin, next_row(), e, ok, fr);
        scalar_step<E, RED, U, true, true, false>(x, b0, b1, acc, fin, next_row(), e, ok, fr);
    }
    if (s == R - 3) {
        scalar_step<E, RED, U, true, true, false>(x, b1, b0, acc, fin, next_row(), e, ok, fr);
        scalar_step<E, RED, U, true, false, true>(x, b0, b1, acc, fin, nullptr, e, ok, fr);
    } else {
        scalar_step<E, RED, U, true, false, true>(x, b1, b0, acc, fin, nullptr, e, ok, fr);
    }
}

template <class E, int U>
__device__ inline void fused_reduce_scalar_op(const RingArgs& a, int c, uint64_t lo, uint64_t len,
                                              uint64_t j0, uint64_t js)
{
    switch (a.redop) {
    case AR_MAX:
        fused_reduce_scalar<E, AR_MAX, U>(a, c, lo, len, j0, js);
        break;
    case AR_MIN:
        fused_reduce_scalar<E, AR_MIN, U>(a, c, lo, len, j0, js);
        break;
    case AR_AVG:
        fused_reduce_scalar<E, AR_AVG, U>(a, c, lo, len, j0, js);
        break;
    default:
        fused_reduce_scalar<E, AR_SUM, U>(a, c, lo, len, j0, js);
        break;
    }
}

// The copy steps of a tile on the scalar path: U elements per thread (the
// same ones the reduce steps took), loads first and unconditional, then the
// stores.
template <class E, int U>
__device__ inline void copy_scalar(const typename E::T* __restrict__ src,
                                   typename E::T* __restrict__ dst, uint64_t len, uint64_t j0,
                                   uint64_t js)
{
    typename E::T r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t j = j0 + (uint64_t)u * js;
        r[u] = src[j < len ? j : j0];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t j = j0 + (uint64_t)u * js;
        if (U == 1 || j < len)
            dst[j] = r[u];
    }
}

// One tile's whole chain on the scalar path with U slots per thread.
template <class E, int OP, int U>
__device__ inline void fused_tile_scalar(const RingArgs& a, int c, uint64_t lo, uint64_t len,
                                         uint64_t j0, uint64_t js)
{
    using T = typename E::T;
    T* out = static_cast<T*>(a.out);
    const int R = a.R, m = a.m;
    if constexpr (OP != kOpAllGather)
        fused_reduce_scalar_op<E, U>(a, c, lo, len, j0, js);
    if constexpr (OP != kOpReduceScatter) {
        if constexpr (OP == kOpAllGather) {
            const T* src = static_cast<const T*>(a.send) + (uint64_t)c * a.send_row +
                           (lo - (uint64_t)c * a.S);
            copy_scalar<E, U>(src, out + (uint64_t)c * a.out_row + lo, len, j0, js);
            step_boundary();
        }
        int p = c;
        for (int s = 0; s <= R - 2; ++s) {
            int q = p + m;
            if (q >= R)
                q -= R;
            copy_scalar<E, U>(out + (uint64_t)p * a.out_row + lo, out + (uint64_t)q * a.out_row + lo,
                              len, j0, js);
            step_boundary();
            p = q;
        }
    }
}

// Tile t of a fused launch on the scalar path (segments shorter than
// AR_SCALAR_SEG_BYTES, one element per slot): segment c, its range [lo, lo +
// len) of a full row, and this thread's first element j0 (elements j0 + u*js).
// False for an empty tile of a short trailing segment (uniform per
// workgroup).  Tiles are numbered segment by segment.  A tile the segment
// fills only in part puts one element on each thread (up to kBlock threads),
// so that a wave's elements are adjacent and each step stores them with one
// instruction (four elements of one thread in one cache line took four
// stores: 8.5 against 6 us a call).
__device__ inline bool scalar_tile(const RingArgs& a, uint64_t t, int* c, uint64_t* lo,
                                   uint64_t* len, uint64_t* j0, uint64_t* js, bool* active)
{
    const uint64_t tile_slots = a.tile_slots;
    const uint64_t tiles_per_seg = (a.sub_len + tile_slots - 1) / tile_slots;
    *c = (int)(t / tiles_per_seg);
    const uint64_t k = t % tiles_per_seg;
    uint64_t hi;
    seg_range(a.N, a.S, *c, a.sub_lo, a.sub_len, lo, &hi);
    *len = hi - *lo;
    const uint64_t first = k * tile_slots;
    const uint64_t n = *len > first ? *len - first : 0;
    // a tile of at most kBlock slots has one per thread, a larger one kUnroll
    uint64_t stride = tile_slots <= (uint64_t)kBlock ? tile_slots : tile_slots / kUnroll;
    if (n < tile_slots)
        stride = n < (uint64_t)kBlock ? n : (uint64_t)kBlock;
    *js = stride;
    *active = threadIdx.x < stride;
    *j0 = first + threadIdx.x;
    return first < *len;
}

// The fused form on the scalar path: a workgroup takes a tile of a segment
// through all 2(R-1) steps (the vector path is k_ring_fused_vec).
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_ring_fused(RingArgs a)
{
    using E = Elem<DT>;
    const uint64_t tile_slots = a.tile_slots;
    const uint64_t tiles_per_seg = (a.sub_len + tile_slots - 1) / tile_slots;
    const uint64_t ntiles = tiles_per_seg * (uint64_t)a.R;

    // with xcd_pack = n only every n-th workgroup works: workgroups are
    // dispatched to the XCDs round-robin, so the working ones share an XCD
    const uint32_t pack = a.xcd_pack > 1 ? (uint32_t)a.xcd_pack : 1u;
    if (blockIdx.x % pack)
        return;
    const uint64_t wg = blockIdx.x / pack, nwg = gridDim.x / pack;
    for (uint64_t t = wg; t < ntiles; t += nwg) {
        int c;
        uint64_t lo, len, j0, js;
        bool active;
        if (!scalar_tile(a, t, &c, &lo, &len, &j0, &js, &active))
            continue;  // empty tile of a short trailing segment (uniform per workgroup)
        if (!active)
            continue;  // this thread has no element in a part-filled tile

        // a tile whose stride covers all its elements (one per thread)
        // takes the one-slot chain
        const uint64_t first = j0 - threadIdx.x;
        const uint64_t nt = len - first < tile_slots ? len - first : tile_slots;
        if (js >= nt)
            fused_tile_scalar<E, OP, 1>(a, c, lo, len, j0, js);
        else
            fused_tile_scalar<E, OP, kUnroll>(a, c, lo, len, j0, js);
    }
}

// ---- dispatch -----------------------------------------------------------------

template <int DT, int V>
hipError_t step_launch(const RingArgs& a, int gx, hipStream_t st, bool copy)
{
    dim3 grid(gx, a.R), block(kBlock);
    if (copy)
        hipLaunchKernelGGL((k_ring_copy_step<DT, V>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_ring_reduce_step<DT, V>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DT>
hipError_t fused_launch(const RingArgs& a, int grid, hipStream_t st)
{
    if (a.op == kOpAllReduce)
        hipLaunchKernelGGL((k_ring_fused<DT, kOpAllReduce>), dim3(grid), dim3(kBlock), 0, st, a);
    else if (a.op == kOpReduceScatter)
        hipLaunchKernelGGL((k_ring_fused<DT, kOpReduceScatter>), dim3(grid), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_ring_fused<DT, kOpAllGather>), dim3(grid), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <int DT>
int resident_fused_dt()
{
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_fused<DT, kOpAllReduce>, kBlock,
                                                     0) != hipSuccess)
        return 0;
    return per_cu * ncu;
}

}  // namespace

// The step a.step of the ring: reduce steps are 0..R-2 (a.op decides where
// the final value goes); copy steps are R-1..2R-3 of the all-reduce, or
// 0..R-2 of an all-gather after the placement launch.
hipError_t launch_ring_step(int dtype, bool vec, const RingArgs& a0, int gx, hipStream_t st)
{
    RingArgs a = a0;
    bool copy = false;
    if (a.op == kOpAllGather) {
        copy = true;
    } else if (a.step >= a.R - 1) {
        copy = true;
        a.step -= a.R - 1;
    }
    switch (dtype) {
    case AR_INT32:
        return vec ? step_launch<AR_INT32, 4>(a, gx, st, copy) : step_launch<AR_INT32, 1>(a, gx, st, copy);
    case AR_FLOAT32:
        return vec ? step_launch<AR_FLOAT32, 4>(a, gx, st, copy)
                   : step_launch<AR_FLOAT32, 1>(a, gx, st, copy);
    case AR_BF16:
        return vec ? step_launch<AR_BF16, 8>(a, gx, st, copy) : step_launch<AR_BF16, 1>(a, gx, st, copy);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ring_placement(int dtype, bool vec, const RingArgs& a, int gx, hipStream_t st)
{
    dim3 grid(gx, a.R), block(kBlock);
    switch (dtype) {
    case AR_INT32:
        if (vec)
            hipLaunchKernelGGL((k_ring_placement<AR_INT32, 4>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((k_ring_placement<AR_INT32, 1>), grid, block, 0, st, a);
        break;
    case AR_FLOAT32:
        if (vec)
            hipLaunchKernelGGL((k_ring_placement<AR_FLOAT32, 4>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((k_ring_placement<AR_FLOAT32, 1>), grid, block, 0, st, a);
        break;
    case AR_BF16:
        if (vec)
            hipLaunchKernelGGL((k_ring_placement<AR_BF16, 8>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((k_ring_placement<AR_BF16, 1>), grid, block, 0, st, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The fused form's scalar path; the vector path is launch_ring_fused_vec.
hipError_t launch_ring_fused(int dtype, bool vec, const RingArgs& a, int grid, hipStream_t st)
{
    if (vec)
        return launch_ring_fused_vec(dtype, a, grid, st);
    switch (dtype) {
    case AR_INT32:
        return fused_launch<AR_INT32>(a, grid, st);
    case AR_FLOAT32:
        return fused_launch<AR_FLOAT32>(a, grid, st);
    case AR_BF16:
        return fused_launch<AR_BF16>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

int resident_ring_fused(int dtype, bool vec)
{
    if (vec)
        return resident_ring_fused_vec(dtype);
    switch (dtype) {
    case AR_INT32:
        return resident_fused_dt<AR_INT32>();
    case AR_FLOAT32:
        return resident_fused_dt<AR_FLOAT32>();
    case AR_BF16:
        return resident_fused_dt<AR_BF16>();
    }
    return 0;
}

// ---- small fills (used instead of hipMemsetAsync so the calls stay safe
// inside a captured graph) -----------------------------------------------------

namespace {
__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}
__global__ void k_fill_u64(uint64_t* p, uint64_t v, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}
int fill_grid(size_t n)
{
    size_t g = (n + 255) / 256;
    return (int)(g < 4096 ? (g ? g : 1) : 4096);
}
}  // namespace

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3(fill_grid(n)), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t* p, uint64_t v, size_t n, hipStream_t st)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_fill_u64, dim3(fill_grid(n)), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

}  // namespace ar
