// ar_fused.hip -- the fused ring form on the 16-byte vector path, for gfx950
// (MI355X).
//
// The schedule is the ring's (ar_ring.hip, header): R-1 reduce steps, then
// R-1 copy steps around q -> q+m, rank c owning segment c, so an element of
// segment c is the left fold x_{c+m} + x_{c+2m} + ... + x_c ("GPU MODE
// lecture 68 notes", section 05: 2(N-1) steps).
//
// One persistent launch.  The unit of work is a wave tile: one wave64 takes
// kWaveSlots 16-byte slots per lane -- 2 KiB of every rank row for 32-bit
// elements -- of one segment, and carries it through all 2(R-1) steps in
// order.  Every hop is a store by the rank that passes the value on and a
// load by the rank that receives it, at the same address and by the same lane
// (so program order makes the load see the store; an empty asm memory clobber
// keeps the compiler from forwarding the value in registers).  Tiles are
// independent, so there are no flags and no fences.  A reduce step's hop goes
// through LDS (below); a copy step's is the receiver's load of the sender's
// output row, whose lines are still in this XCD's L2.
//
// Why wave tiles: the rows a tile touches are 2R streams through HBM (R
// inputs read, R outputs written back from L2).  With one tile per wave and
// two workgroups per CU, a wave's 2 KiB of a row is contiguous and the chain
// of one tile never waits on another wave; each rank's input is loaded one
// step ahead into the other of two register sets, so its HBM latency overlaps
// the hand-off instead of adding to it.  Ranks advance by adding m (no
// division inside the chain).
//
// Where a reduce step's running value is handed on: in the wave's own region
// of LDS (16 KiB per workgroup), a store and a load by the same lane as
// through L2 but at a fraction of the round trip -- for every reduce-scatter,
// every call that would otherwise stage it in memory (bfloat16, in place) and
// an all-reduce whose rows (2 R N s) total at most 512 MiB (RingArgs::
// hand_lds).  A larger all-reduce with the accumulator type T hands it on in
// the owner's output row, where the final value lands: from 128 MiB per rank
// at R = 8 float32 that was ~7% faster than LDS, up to 32 MiB 7-13% slower,
// level at 64 MiB.  (With LDS: R = 16 bfloat16 buckets, reduce-scatter 117 ->
// 74 us and all-reduce 198 -> 170 us, against a per-wave staging slot in the
// workspace or the lines of two output rows; R = 8 float32 64 MiB per rank,
// reduce-scatter 144 -> 95 us.)  Tiles cut short by a segment's end (the
// checked path) still stage in memory.  A float32 value sits in LDS as two
// runs of 16-byte halves.
//
// Every access goes through a buffer resource that spans exactly the tile it
// addresses: an offset past the tile is dropped by the hardware.
#include "ar_elem.h"
#include "ar_internal.h"
#include "ar_slots.h"

namespace ar {
namespace {

constexpr int kWaves = kBlock / 64;                      // waves per workgroup
constexpr uint32_t kTileSlots = kWaveTileSlots;           // 16-byte slots per wave tile
constexpr int kPolPlain = 0;
constexpr int kPolStream = 2;  // nt: each input element is read once per collective
// sc1 (device scope): the store is written through to memory at once.  The
// reduce-scatter's shard is written once and never read back by the launch,
// and sending it out in issue order, instead of leaving it as dirty lines for
// later evictions, measured ~3% faster on bf16 buckets (the all-reduce's
// final row is the next hop's input and must stay in L2).
constexpr int kPolWriteThrough = 16;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Resource over `bytes` bytes from p; p must be wave-uniform.
__device__ inline rsrc_t tile_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

template <int POL>
__device__ inline u32x4 bload(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL));
}

template <int POL>
__device__ inline void bstore(rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, POL);
}

// Byte offset of slot u of `lane` in a row tile (16-byte slots of T).  A
// lane's accumulator slot (V/4 16-byte halves) keeps half h in its own run
// of the same shape, so each half is a row tile of its own.
__device__ inline uint32_t t_off(int u, uint32_t lane) { return ((uint32_t)u * 64u + lane) * 16u; }

// Where a whole tile's running value is handed on: the wave's own region of
// LDS, half h of slot u of `lane` at h[h][u * 64 + lane] (one run for 32-bit
// T, two for bfloat16's float32 values).  A store by the rank that passes the
// value on and a load by the rank that receives it, by the same lane and in
// order within the wave.
struct Hand {
    u32x4* h[2];
};

template <class E, int V>
__device__ inline void a_load(const Hand& r, uint32_t lane, int u, typename E::A (&o)[V])
{
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const u32x4 q = r.h[h][(uint32_t)u * 64u + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[4 * h + i] = E::from_bits(q[i]);
    }
}

template <class E, int V>
__device__ inline void a_store(const Hand& r, uint32_t lane, int u, const typename E::A (&v)[V])
{
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = E::to_bits(v[4 * h + i]);
        r.h[h][(uint32_t)u * 64u + lane] = q;
    }
}

// The same hand-off through memory: half h of every accumulator slot in the
// run behind h[h] (the owner's output row), each kTileSlots * 16 bytes.
struct HandMem {
    rsrc_t h[2];
};

template <class E, int V>
__device__ inline void a_load(const HandMem& r, uint32_t lane, int u, typename E::A (&o)[V])
{
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const u32x4 q = bload<kPolPlain>(r.h[h], t_off(u, lane));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[4 * h + i] = E::from_bits(q[i]);
    }
}

template <class E, int V>
__device__ inline void a_store(const HandMem& r, uint32_t lane, int u, const typename E::A (&v)[V])
{
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = E::to_bits(v[4 * h + i]);
        bstore<kPolPlain>(r.h[h], t_off(u, lane), q);
    }
}

// The final value of slot u as T (bfloat16: one nearest-even rounding),
// stored with cache policy POL.
template <class E, int V, int POL>
__device__ inline void t_store(rsrc_t r, uint32_t lane, int u, const typename E::A (&v)[V])
{
    u32x4 q;
    if constexpr (sizeof(typename E::T) == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = E::to_bits(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = (uint32_t)E::narrow(v[2 * i]) | ((uint32_t)E::narrow(v[2 * i + 1]) << 16);
    }
    bstore<POL>(r, t_off(u, lane), q);
}

// What one wave tile needs to know.
struct Tile {
    int c;              // segment
    uint64_t lo;        // segment (channel sub-range) start, elements
    uint64_t len;       // its length
    uint64_t first;     // the tile's first slot within the segment
    uint32_t lane;
};

// The tile's place in the rows of one rank-major array, walked around the
// ring: rank r's row is at base + r * row bytes; next() moves to rank r + m
// with an add and a wrap instead of a multiply, so that no chain of scalar
// multiplies sits between one step's store and the next step's load.
struct RowWalk {
    const char* p;    // the current rank's tile
    const char* end;  // base + R * row: one past the last rank
    uint64_t step;    // m * row bytes
    uint64_t wrap;    // R * row bytes
    __device__ void next()
    {
        p += step;
        if (p >= end)
            p -= wrap;
    }
    __device__ rsrc_t rsrc() const { return tile_rsrc(p, kTileSlots * 16u); }
};

// Walk over the tile in `arr` ([R][row] elements of T) starting at rank r.
template <class E, int V>
__device__ inline RowWalk row_walk(const void* arr, uint64_t row, const RingArgs& a, const Tile& t,
                                   int r)
{
    const uint64_t rb = row * sizeof(typename E::T);
    const char* base = static_cast<const char*>(arr) + (t.lo + t.first * V) * sizeof(typename E::T);
    RowWalk w;
    w.p = base + (uint64_t)r * rb;
    w.end = base + (uint64_t)a.R * rb;
    w.step = (uint64_t)a.m * rb;
    w.wrap = (uint64_t)a.R * rb;
    return w;
}

// One reduce step of a whole wave tile.  x holds the received value: on entry
// at step 0 (the predecessor's input), else loaded here from the hand-off slot
// the previous step stored (LOADX).  With PREFETCH the input of the next
// step's rank (the walker `in`, then advanced by m) is loaded into `nxt` after the hand-off
// load, so a wait for the hand-off leaves it in flight; `own` was loaded the
// same way one step earlier.  LAST: the owner's step, written as T with
// cache policy FP.
template <class E, int V, int RED, int FP, bool LOADX, bool PREFETCH, bool LAST, class H>
__device__ inline void wt_step(const RingArgs& a, const Tile& t, typename E::A (&x)[kWaveSlots][V],
                               const u32x4 (&own)[kWaveSlots], u32x4 (&nxt)[kWaveSlots],
                               const H& hand, rsrc_t fin, RowWalk* in)
{
    if constexpr (LOADX) {
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            a_load<E, V>(hand, t.lane, u, x[u]);
    }
    if constexpr (PREFETCH) {
        const rsrc_t q = in->rsrc();
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            nxt[u] = bload<kPolStream>(q, t_off(u, t.lane));
        in->next();
    }
#pragma unroll
    for (int u = 0; u < kWaveSlots; ++u) {
        typename E::A y[V];
        widen_slot<E, V>(own[u], y);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            x[u][i] = combine<E, RED>(x[u][i], y[i]);
            if constexpr (LAST)
                x[u][i] = finalize<E, RED>(x[u][i], (float)a.R);
        }
        if constexpr (LAST)
            t_store<E, V, FP>(fin, t.lane, u, x[u]);
        else
            a_store<E, V>(hand, t.lane, u, x[u]);
    }
    step_boundary();
}

// The R-1 reduce steps of a whole wave tile of segment c.  Step s is rank
// c + (s+2)m; its input was loaded during step s-1 into the other of two
// register sets.
template <class E, int V, int RED, int FP, class H>
__device__ inline void wt_reduce(const RingArgs& a, const Tile& t, const H& hand, rsrc_t fin)
{
    using A = typename E::A;
    const int R = a.R;
    int r1 = t.c + a.m;
    if (r1 >= R)
        r1 -= R;
    RowWalk rn = row_walk<E, V>(a.send, a.send_row, a, t, r1);
    A x[kWaveSlots][V];
    u32x4 b0[kWaveSlots], b1[kWaveSlots];
    {
        const rsrc_t q1 = rn.rsrc();
        rn.next();
        const rsrc_t q2 = rn.rsrc();
        rn.next();  // now the rank whose input step 1 adds
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u) {
            widen_slot<E, V>(bload<kPolStream>(q1, t_off(u, t.lane)), x[u]);
            b0[u] = bload<kPolStream>(q2, t_off(u, t.lane));
        }
    }
    if (R == 2) {
        wt_step<E, V, RED, FP, false, false, true>(a, t, x, b0, b1, hand, fin, &rn);
        return;
    }
    // R >= 3: steps 0 .. R-3 hand off, step R-2 is the owner's
    wt_step<E, V, RED, FP, false, true, false>(a, t, x, b0, b1, hand, fin, &rn);
    int s = 1;  // the next step; its input is in b1
    for (; s + 1 <= R - 3; s += 2) {
        wt_step<E, V, RED, FP, true, true, false>(a, t, x, b1, b0, hand, fin, &rn);
        wt_step<E, V, RED, FP, true, true, false>(a, t, x, b0, b1, hand, fin, &rn);
    }
    if (s == R - 3) {
        wt_step<E, V, RED, FP, true, true, false>(a, t, x, b1, b0, hand, fin, &rn);
        wt_step<E, V, RED, FP, true, false, true>(a, t, x, b0, b1, hand, fin, &rn);
    } else {
        wt_step<E, V, RED, FP, true, false, true>(a, t, x, b1, b0, hand, fin, &rn);
    }
}

// The copy steps of a whole wave tile: rank p's output is read and stored as
// rank p+m's, starting at the owner c (all-gather: after the owner placed its
// own shard).
template <class E, int V, int OP>
__device__ inline void wt_copy(const RingArgs& a, const Tile& t)
{
    RowWalk w = row_walk<E, V>(a.out, a.out_row, a, t, t.c);
    rsrc_t src = w.rsrc();
    if constexpr (OP == kOpAllGather) {
        // send is [R][S]: the owner's shard, at the same offset within it
        const typename E::T* own = static_cast<const typename E::T*>(a.send) +
                                   (uint64_t)t.c * a.send_row + (t.lo - (uint64_t)t.c * a.S) +
                                   t.first * V;
        const rsrc_t s = tile_rsrc(own, kTileSlots * 16u);
        u32x4 v[kWaveSlots];
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            v[u] = bload<kPolStream>(s, t_off(u, t.lane));
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            bstore<kPolPlain>(src, t_off(u, t.lane), v[u]);
        step_boundary();
    }
    for (int s = 0; s <= a.R - 2; ++s) {
        w.next();
        const rsrc_t dst = w.rsrc();
        u32x4 v[kWaveSlots];
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            v[u] = bload<kPolPlain>(src, t_off(u, t.lane));
#pragma unroll
        for (int u = 0; u < kWaveSlots; ++u)
            bstore<kPolPlain>(dst, t_off(u, t.lane), v[u]);
        step_boundary();
        src = dst;
    }
}

// The last tile of a segment when the segment ends inside it: step by step
// with the checked slot helpers.  Lane slots are j0 + u*64; the helpers'
// slots past the tile lie past the segment's end, so they are skipped.  `acc`
// addresses slot j's running value at acc + j*V.
template <class E, int V, int OP>
__device__ inline void wt_ragged(const RingArgs& a, const Tile& t, typename E::A* acc)
{
    using T = typename E::T;
    const int R = a.R, m = a.m;
    const uint64_t j0 = t.first + t.lane;
    const T* send = static_cast<const T*>(a.send);
    T* out = static_cast<T*>(a.out);
    if constexpr (OP != kOpAllGather) {
        int q = t.c + 2 * m;  // rank of step 0, and its predecessor p
        q %= R;
        int p = t.c + m;
        p %= R;
        for (int s = 0; s <= R - 2; ++s) {
            ReducePtrs<E> rp;
            rp.prevT = send + (uint64_t)p * a.send_row + t.lo;
            rp.own = send + (uint64_t)q * a.send_row + t.lo;
            rp.prevA = acc;
            rp.dstA = acc;
            rp.dstT = out + (uint64_t)q * a.out_row +
                      (OP == kOpReduceScatter ? t.lo - (uint64_t)t.c * a.S : t.lo);
            reduce_step_slots<E, V>(rp, s, R, a.redop, t.len, j0, 64);
            step_boundary();
            p = q;
            q += m;
            if (q >= R)
                q -= R;
        }
    }
    if constexpr (OP != kOpReduceScatter) {
        if constexpr (OP == kOpAllGather) {
            const T* src = send + (uint64_t)t.c * a.send_row + (t.lo - (uint64_t)t.c * a.S);
            copy_slots<E, V>(src, out + (uint64_t)t.c * a.out_row + t.lo, t.len, j0, 64);
            step_boundary();
        }
        int p = t.c;
        for (int s = 0; s <= R - 2; ++s) {
            int q = p + m;
            if (q >= R)
                q -= R;
            copy_slots<E, V>(out + (uint64_t)p * a.out_row + t.lo, out + (uint64_t)q * a.out_row + t.lo,
                             t.len, j0, 64);
            step_boundary();
            p = q;
        }
    }
}

// RAGGED: some segment ends inside a tile (the host knows from the sizes);
// without it every tile is whole and the checked path is not compiled in,
// which keeps the kernel's registers (and so its occupancy) to the chain's.
template <int DT, int OP, int RED, bool RAGGED>
__device__ inline void wt_run(const RingArgs& a, uint32_t unit, uint32_t nunits, uint32_t lane)
{
    using E = Elem<DT>;
    using T = typename E::T;
    using A = typename E::A;
    constexpr int V = E::VEC;
    const uint64_t tps = ((a.sub_len + V - 1) / V + kTileSlots - 1) / kTileSlots;  // tiles per segment
    const uint64_t ntiles = tps * (uint64_t)a.R;
    // this wave's staging slot, or the running value in part at c*part_seg + e
    A* stage = a.stage_wave ? static_cast<A*>(a.part) + (uint64_t)unit * a.stage_wave : nullptr;
    // a whole tile hands its running value on through this wave's LDS region
    // where the host asks for it (and wherever it would stage in memory); the
    // staging slot then serves ragged tiles only
    __shared__ u32x4 lds_hand[kWaves][2][kTileSlots];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int c = (int)(unit / tps);
    uint64_t k = unit % tps;
    for (uint64_t t = unit; t < ntiles; t += nunits) {
        Tile tl;
        tl.c = c;
        tl.lane = lane;
        uint64_t hi;
        seg_range(a.N, a.S, c, a.sub_lo, a.sub_len, &tl.lo, &hi);
        tl.len = hi - tl.lo;
        tl.first = k * kTileSlots;
        if (tl.first * V < tl.len) {  // else an empty tile of a short trailing segment
            A* acc = stage ? stage - tl.first * V
                           : static_cast<A*>(a.part) + (uint64_t)c * a.part_seg + tl.lo;
            if ((tl.first + kTileSlots) * V <= tl.len) {
                if constexpr (OP != kOpAllGather) {
                    constexpr int FP = OP == kOpReduceScatter ? kPolWriteThrough : kPolPlain;
                    T* fin = static_cast<T*>(a.out) + (uint64_t)c * a.out_row +
                             (OP == kOpReduceScatter ? tl.lo - (uint64_t)c * a.S : tl.lo) +
                             tl.first * V;
                    if (stage || a.hand_lds) {
                        Hand hand;
                        hand.h[0] = lds_hand[wave][0];
                        hand.h[1] = lds_hand[wave][1];
                        wt_reduce<E, V, RED, FP>(a, tl, hand, tile_rsrc(fin, kTileSlots * 16u));
                    } else {
                        // the owner's output row (the accumulator is T)
                        HandMem hm;
                        constexpr uint32_t half = kTileSlots * 16u;
                        const char* b = reinterpret_cast<const char*>(acc + tl.first * V);
                        hm.h[0] = tile_rsrc(b, half);
                        hm.h[1] = tile_rsrc(b + half, half);
                        wt_reduce<E, V, RED, FP>(a, tl, hm, tile_rsrc(fin, kTileSlots * 16u));
                    }
                }
                if constexpr (OP != kOpReduceScatter)
                    wt_copy<E, V, OP>(a, tl);
            } else if constexpr (RAGGED) {
                wt_ragged<E, V, OP>(a, tl, acc);
            }
        }
        k += nunits;
        if (k >= tps) {
            c += (int)(k / tps);
            k %= tps;
        }
    }
}

// The reduction operator is a template argument (the host picks the
// instantiation), so each kernel holds one operator's code.
template <int DT, int OP, int RED, bool RAGGED>
__global__ __launch_bounds__(kBlock) void k_ring_fused_vec(RingArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nunits = min(gridDim.x * (uint32_t)kWaves, a.max_units);
    if (unit >= nunits)
        return;
    wt_run<DT, OP, RED, RAGGED>(a, unit, nunits, lane);
}

template <int DT, int OP, int RED>
void fused_vec_go(const RingArgs& a, int grid, hipStream_t st)
{
    if (a.ragged)
        hipLaunchKernelGGL((k_ring_fused_vec<DT, OP, RED, true>), dim3(grid), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_ring_fused_vec<DT, OP, RED, false>), dim3(grid), dim3(kBlock), 0, st, a);
}

template <int DT, int OP>
void fused_vec_op(const RingArgs& a, int grid, hipStream_t st)
{
    if constexpr (OP == kOpAllGather) {
        fused_vec_go<DT, OP, AR_SUM>(a, grid, st);  // a copy: no operator
    } else {
        switch (a.redop) {
        case AR_MAX:
            fused_vec_go<DT, OP, AR_MAX>(a, grid, st);
            break;
        case AR_MIN:
            fused_vec_go<DT, OP, AR_MIN>(a, grid, st);
            break;
        case AR_AVG:
            if constexpr (DT != AR_INT32)  // no integer average (refused by the host)
                fused_vec_go<DT, OP, AR_AVG>(a, grid, st);
            break;
        default:
            fused_vec_go<DT, OP, AR_SUM>(a, grid, st);
            break;
        }
    }
}

template <int DT>
hipError_t fused_vec_launch(const RingArgs& a, int grid, hipStream_t st)
{
    if (a.op == kOpAllReduce)
        fused_vec_op<DT, kOpAllReduce>(a, grid, st);
    else if (a.op == kOpReduceScatter)
        fused_vec_op<DT, kOpReduceScatter>(a, grid, st);
    else
        fused_vec_op<DT, kOpAllGather>(a, grid, st);
    return hipGetLastError();
}

template <int DT>
int resident_vec_dt()
{
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_fused_vec<DT, kOpAllReduce, AR_SUM, true>,
                                                     kBlock, 0) != hipSuccess)
        return 0;
    return per_cu * ncu;
}

}  // namespace

hipError_t launch_ring_fused_vec(int dtype, const RingArgs& a, int grid, hipStream_t st)
{
    switch (dtype) {
    case AR_INT32:
        return fused_vec_launch<AR_INT32>(a, grid, st);
    case AR_FLOAT32:
        return fused_vec_launch<AR_FLOAT32>(a, grid, st);
    case AR_BF16:
        return fused_vec_launch<AR_BF16>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

int resident_ring_fused_vec(int dtype)
{
    switch (dtype) {
    case AR_INT32:
        return resident_vec_dt<AR_INT32>();
    case AR_FLOAT32:
        return resident_vec_dt<AR_FLOAT32>();
    case AR_BF16:
        return resident_vec_dt<AR_BF16>();
    }
    return 0;
}

}  // namespace ar
