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

// One reduce step of the scalar path (one element per thread, element e).
// The same structure as
// fused_step: the hand-off is loaded after the previous step's store, the
// next step's input is prefetched into `nxt`, and `own` was prefetched one
// step earlier.  The empty asm takes the loaded hand-off values as operands,
// so the compiler waits for them right there (leaving the prefetch in
// flight) instead of moving each load into its store's branch and waiting
// for everything outstanding.
template <class E, int RED, bool LOADX, bool PREFETCH, bool LAST>
__device__ inline void scalar_step(typename E::A& x, const typename E::T& own,
                                   typename E::T& nxt, typename E::A* slot, typename E::T* fin,
                                   const typename E::T* next_row, uint64_t e, float R)
{
    using A = typename E::A;
    if constexpr (LOADX)
        x = *slot;
    if constexpr (PREFETCH)
        nxt = next_row[e];
    __asm__ __volatile__("" ::"v"(x));
    A v = combine<E, RED>(x, E::widen(own));
    if constexpr (LAST) {
        v = finalize<E, RED>(v, R);
        fin[e] = E::narrow(v);
    } else {
        *slot = v;
    }
    x = v;
    step_boundary();
}

// The R-1 reduce steps of a tile on the scalar path: each active thread has
// one element e of segment c.  As on the vector path, the input of the next
// step's rank is loaded before this step's store, into the other of two
// registers, so its HBM latency overlaps the hand-off instead of adding to
// each step.  The rank whose row a step reads advances by m (no division:
// each step is latency-bound, and its instruction count is part of it).
template <class E, int RED>
__device__ inline void fused_reduce_scalar(const RingArgs& a, int c, uint64_t lo, uint64_t e,
                                           typename E::A* slot)
{
    using T = typename E::T;
    using A = typename E::A;
    const int R = a.R;
    const int m = a.m;
    const float fr = (float)R;
    const T* send = static_cast<const T*>(a.send) + lo;
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
    A x = E::widen(next_row()[e]);
    T b0 = next_row()[e], b1;
    if (R == 2) {
        scalar_step<E, RED, false, false, true>(x, b0, b1, slot, fin, nullptr, e, fr);
        return;
    }
    // R >= 3: steps 0 .. R-3 hand off, step R-2 is the owner's
    scalar_step<E, RED, false, true, false>(x, b0, b1, slot, fin, next_row(), e, fr);
    int s = 1;  // the next step; its input is in b1
    for (; s + 1 <= R - 3; s += 2) {
        scalar_step<E, RED, true, true, false>(x, b1, b0, slot, fin, next_row(), e, fr);
        scalar_step<E, RED, true, true, false>(x, b0, b1, slot, fin, next_row(), e, fr);
    }
    if (s == R - 3) {
        scalar_step<E, RED, true, true, false>(x, b1, b0, slot, fin, next_row(), e, fr);
        scalar_step<E, RED, true, false, true>(x, b0, b1, slot, fin, nullptr, e, fr);
    } else {
        scalar_step<E, RED, true, false, true>(x, b1, b0, slot, fin, nullptr, e, fr);
    }
}

template <class E>
__device__ inline void fused_reduce_scalar_op(const RingArgs& a, int c, uint64_t lo, uint64_t e,
                                              typename E::A* slot)
{
    switch (a.redop) {
    case AR_MAX:
        fused_reduce_scalar<E, AR_MAX>(a, c, lo, e, slot);
        break;
    case AR_MIN:
        fused_reduce_scalar<E, AR_MIN>(a, c, lo, e, slot);
        break;
    case AR_AVG:
        fused_reduce_scalar<E, AR_AVG>(a, c, lo, e, slot);
        break;
    default:
        fused_reduce_scalar<E, AR_SUM>(a, c, lo, e, slot);
        break;
    }
}

// One tile's whole chain on the scalar path: element e of segment c.
template <class E, int OP>
__device__ inline void fused_tile_scalar(const RingArgs& a, int c, uint64_t lo, uint64_t e,
                                         typename E::A* slot)
{
    using T = typename E::T;
    T* out = static_cast<T*>(a.out);
    const int R = a.R, m = a.m;
    if constexpr (OP != kOpAllGather)
        fused_reduce_scalar_op<E>(a, c, lo, e, slot);
    if constexpr (OP != kOpReduceScatter) {
        if constexpr (OP == kOpAllGather) {
            const T* src = static_cast<const T*>(a.send) + (uint64_t)c * a.send_row +
                           (lo - (uint64_t)c * a.S);
            out[(uint64_t)c * a.out_row + lo + e] = src[e];
            step_boundary();
        }
        int p = c;
        for (int s = 0; s <= R - 2; ++s) {
            int q = p + m;
            if (q >= R)
                q -= R;
            out[(uint64_t)q * a.out_row + lo + e] = out[(uint64_t)p * a.out_row + lo + e];
            step_boundary();
            p = q;
        }
    }
}

// Tile t of a fused launch on the scalar path: kBlock elements of one
// segment, one per thread (tiles are numbered segment by segment).  Sets the
// segment c, its range start lo in a full row, and this thread's element e
// within the segment; false when the thread has no element (past the end of
// a part-filled tile, or an empty tile of a short trailing segment).
__device__ inline bool scalar_tile(const RingArgs& a, uint64_t tiles_per_seg, uint64_t t, int* c,
                                   uint64_t* lo, uint64_t* e)
{
    *c = (int)(t / tiles_per_seg);
    const uint64_t k = t % tiles_per_seg;
    uint64_t hi;
    seg_range(a.N, a.S, *c, a.sub_lo, a.sub_len, lo, &hi);
    *e = k * (uint64_t)kBlock + threadIdx.x;
    return *e < hi - *lo;
}

// The fused form on the scalar path (the vector path is k_ring_fused_vec): a
// workgroup takes a tile of kBlock elements, one per thread, through all
// 2(R-1) steps.  Each step of a tile's chain is latency-bound (a store, then
// the next step's load of the same address), so one element per thread
// keeps the step to the fewest instructions, and a reduce step's running
// value passes through the thread's own LDS slot rather than memory (R = 8
// fp32: 8 B - 256 KiB per rank 3.4-4.1 -> 3.1-3.7 us per call; rows not
// 16-byte aligned, 64 MiB + 4 B per rank, 357 -> 322 us).
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_ring_fused(RingArgs a)
{
    using E = Elem<DT>;
    const uint64_t tiles_per_seg = (a.sub_len + kBlock - 1) / kBlock;
    const uint64_t ntiles = tiles_per_seg * (uint64_t)a.R;

    // with xcd_pack = n only every n-th workgroup works: workgroups are
    // dispatched to the XCDs round-robin, so the working ones share an XCD
    const uint32_t pack = a.xcd_pack > 1 ? (uint32_t)a.xcd_pack : 1u;
    if (blockIdx.x % pack)
        return;
    const uint64_t wg = blockIdx.x / pack, nwg = gridDim.x / pack;
    // each thread's hand-off slot: the running value passes from rank to
    // rank through it (a store, then the next step's load, by this thread)
    __shared__ typename E::A hand[kBlock];
    for (uint64_t t = wg; t < ntiles; t += nwg) {
        int c;
        uint64_t lo, e;
        if (scalar_tile(a, tiles_per_seg, t, &c, &lo, &e))
            fused_tile_scalar<E, OP>(a, c, lo, e, &hand[threadIdx.x]);
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
