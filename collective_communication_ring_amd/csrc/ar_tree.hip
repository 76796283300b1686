// ar_tree.hip -- double-binary-tree all-reduce with the LL protocol, for
// gfx950 (MI355X).
//
// Two complementary binary trees run at once, each on different links
// ("NCCL and NVSHMEM -- two GPU communication models, side by side", section
// "double binary tree").  Reading used here: tree A is the in-order binary
// tree on ranks 0..R-1 rooted at 0, tree B is its mirror image (even R) or
// its shift by one (odd R); tree A reduces and broadcasts elements [0, H),
// tree B elements [H, N), H = ceil(N/2).  A node's value is its own input,
// then each child's subtree sum added in ascending rank order; the root's
// sum comes back down unchanged and every rank writes it (narrowed to T).
//
// LL protocol: a value travels as one 8-byte line, 4 bytes of data (the
// accumulator's bits) and 4 bytes of flag, written by one 64-bit atomic store
// ("Demystifying NVSHMEM ..." summary, paragraph on collectives: LL packs data
// and arrival flag into one atomic write).  The consumer polls the line until
// its flag equals this call's epoch; because data and flag arrive together
// there is no fence between them.  On gfx950 the agent-scope atomic store and
// load of the line bypass the non-coherent per-XCD L2 state, so a line written
// on one XCD is seen by a poller on another.
//
// One launch per piece: 2 trees x blocks_per_rank sets of R workgroups (one
// per rank), each set on one XCD (ll_set_of).  Every
// workgroup of the grid must be resident at once (a node spins on its
// children), which the host guarantees by capping the grid at the occupancy
// limit; every wait is also bounded in time (the watchdog) and a timeout sets
// the error word instead of hanging.
//
// Epochs: every group of kTreeGroup lines (one wave's lines of a sub-block, the
// same positions on every rank) has its own epoch word; a launch uses that
// word plus one as the flag of the group's lines, and the root's wave stores
// the new value when it has sent the group's result down.  By then every
// rank's wave of the group has read the old value: each stored an up line
// carrying it, and the root has received them all (directly or through its
// children).  So no launch ever reuses a flag a line may still hold, a
// replayed graph uses fresh flags too, and the launch needs no counter of
// finished workgroups (an atomic round trip at the end of every workgroup).
// Groups are fixed by line position, so launches with different grids share
// them consistently; a group a launch does not touch keeps its epoch, and
// its lines only carry flags up to it.
#include "ar_elem.h"
#include "ar_internal.h"
#include "ar_ll.h"

namespace ar {
namespace {

// The reduction operator is a template argument (the host picks the
// instantiation): on this latency-bound path every branch counts.  K is the
// number of sub-blocks a thread takes per pass: 1 when every workgroup has at
// most one sub-block (small messages: one line per lane, no per-line
// branches), else kTreeEPT.
template <int DT, int RED, int K>
__global__ __launch_bounds__(kBlock) void k_tree_ll(TreeArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    using A = typename E::A;
    const int R = a.R;
    const int bpr = a.blocks_per_rank;
    // set (tree t, block b) of R workgroups, all on one XCD (ll_set_of)
    const uint32_t n = a.xcd_sets > 1 ? (uint32_t)a.xcd_sets : 1u;
    const uint32_t set = ll_set_of(blockIdx.x, n, (uint32_t)R);
    if (set >= 2u * (uint32_t)bpr)
        return;  // past the last set
    const int v = (int)ll_rank_of(blockIdx.x, n, (uint32_t)R);
    const int t = (int)(set / (uint32_t)bpr);
    const int b = (int)(set % (uint32_t)bpr);
    const uint64_t deadline = (uint64_t)wall_clock64() + a.timeout_ticks;
    uint32_t* err = &a.ctrl[kCtrlError];

    // this tree's half of the elements, and this launch's piece of it
    const uint64_t hlo = (t == 0) ? 0 : a.H;
    const uint64_t hlen = (t == 0) ? a.H : a.N - a.H;
    const uint64_t plen = a.piece_lo < hlen ? min(a.piece_len, hlen - a.piece_lo) : 0;
    const uint64_t first = hlo + a.piece_lo;  // element of line 0

    const T* x = static_cast<const T*>(a.send) + (uint64_t)v * a.N + first;
    T* y = static_cast<T*>(a.out) + (uint64_t)v * a.N + first;
    // the node's packed word (one scalar load; see tree_node_word)
    const uint32_t node = a.node[t][v];
    const int parent = (int)(node & 0xffu) - 1;
    const int nchild = (int)((node >> 8) & 0xffu);
    const int child0 = (int)((node >> 16) & 0xffu);
    const int child1 = (int)(node >> 24);
    uint64_t* up_mine = a.up + ((uint64_t)t * R + v) * a.line_stride;
    uint64_t* down_mine = a.down + ((uint64_t)t * R + v) * a.line_stride;
    uint32_t* epochs = a.epochs + (uint64_t)t * a.line_groups;

    const bool publish = (v != a.mute_rank);
    const uint64_t wave_first = threadIdx.x & ~(uint64_t)(kTreeGroup - 1);
    bool timed_out = false;
    // sub-blocks of kBlock lines: sub-block j belongs to workgroup j mod bpr of
    // this (tree, rank); a thread takes K of its workgroup's sub-blocks at once
    // and waits for their lines together
    const uint64_t nsub = (plen + kBlock - 1) / kBlock;
    for (uint64_t j0 = (uint64_t)b; j0 < nsub; j0 += (uint64_t)bpr * K) {
        uint64_t idx[K], grp[K];
        bool ok[K], wave_ok[K];
        A acc[K];
        uint32_t flag[K];
        // Loads are unconditional (a lane past the end reads element 0 of the
        // piece, and a wave past the end group 0's epoch, and never uses
        // them): with conditional loads the compiler cannot count the
        // outstanding memory operations and waits for all of them, stores
        // included, before each later store.
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint64_t base = (j0 + (uint64_t)k * bpr) * kBlock;
            idx[k] = base + threadIdx.x;
            ok[k] = idx[k] < plen;
            wave_ok[k] = base + wave_first < plen;  // the wave has lines in this sub-block
            grp[k] = wave_ok[k] ? (base + wave_first) / kTreeGroup : 0;
            acc[k] = E::widen(x[ok[k] ? idx[k] : 0]);
            flag[k] = __hip_atomic_load(&epochs[grp[k]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        }
        // The inputs and epochs are needed at once (added, or stored up by a
        // leaf).  An explicit wait here tells the compiler that no load is
        // outstanding on any path, so the stores that forward a line later
        // are not each made to wait for the stores before them (vmcnt counts
        // both, in order).
        wait_vmem_all();
        // reduce up: own value, then each child's subtree value in ascending
        // rank order.  The lines of both children are polled together (they
        // arrive at about the same time), so the second child costs no round
        // trip of its own; the adds still take the children in order.
        if (nchild > 0) {
            const uint64_t* up_c0 = a.up + ((uint64_t)t * R + child0) * a.line_stride;
            const uint64_t* up_c1 = a.up + ((uint64_t)t * R + child1) * a.line_stride;
            const uint64_t* ln[2 * K];
            bool want[2 * K];
            uint32_t fl[2 * K];
            uint32_t d[2 * K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                // a line this lane does not wait for is read at offset 0 (valid)
                ln[k] = up_c0 + (ok[k] ? idx[k] : 0);
                ln[K + k] = (nchild > 1 ? up_c1 : up_c0) + (ok[k] ? idx[k] : 0);
                want[k] = ok[k];
                want[K + k] = ok[k] && nchild > 1;
                fl[k] = flag[k];
                fl[K + k] = flag[k];
            }
            if (!ll_wait_all<2 * K>(ln, want, fl, deadline, err, d))
                timed_out = true;
            // own value first, then the children in ascending rank order; a
            // lane past the end combines junk it never stores
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc[k] = combine<E, RED>(acc[k], E::from_bits(d[k]));
            if (nchild > 1) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    acc[k] = combine<E, RED>(acc[k], E::from_bits(d[K + k]));
            }
        }
        if constexpr (RED == AR_AVG) {
            if (parent < 0) {  // the root's sum is final: average it once
#pragma unroll
                for (int k = 0; k < K; ++k)
                    acc[k] = finalize<E, AR_AVG>(acc[k], (float)R);
            }
        }
        if (parent >= 0) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (ok[k] && publish)
                    ll_store(up_mine + idx[k], E::to_bits(acc[k]), flag[k]);
            // broadcast down: the root's value arrives from the parent
            const uint64_t* ln[K];
            uint32_t d[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                ln[k] = down_mine + (ok[k] ? idx[k] : 0);
            if (!ll_wait_all<K>(ln, ok, flag, deadline, err, d))
                timed_out = true;
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc[k] = E::from_bits(d[k]);
        }
        // broadcast down to the children first (they are waiting), then
        // write this rank's output
        for (int ci = 0; ci < nchild; ++ci) {
            uint64_t* down_ch = a.down + ((uint64_t)t * R + (ci == 0 ? child0 : child1)) * a.line_stride;
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (ok[k] && publish)
                    ll_store(down_ch + idx[k], E::to_bits(acc[k]), flag[k]);
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (ok[k])
                y[idx[k]] = E::narrow(acc[k]);
        // the root closes each group it finished: every rank's wave of the
        // group has read its epoch (see the top of this file).  Done even by a
        // muted root, so that a later launch never reuses this flag.
        if (parent < 0 && (threadIdx.x & (kTreeGroup - 1)) == 0) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (wave_ok[k])
                    __hip_atomic_store(&epochs[grp[k]], flag[k], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (timed_out)
        __hip_atomic_fetch_or(err, (uint32_t)kErrTimeout, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT>
int resident_tree_dt()
{
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_tree_ll<DT, AR_SUM, kTreeEPT>, kBlock, 0) !=
        hipSuccess)
        return 0;
    return per_cu * ncu;
}

}  // namespace

namespace {

template <int DT, int K>
void tree_launch_k(const TreeArgs& a, int grid, hipStream_t st)
{
    switch (a.redop) {
    case AR_MAX:
        hipLaunchKernelGGL((k_tree_ll<DT, AR_MAX, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    case AR_MIN:
        hipLaunchKernelGGL((k_tree_ll<DT, AR_MIN, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    case AR_AVG:
        if constexpr (DT != AR_INT32)  // no integer average (refused by the host)
            hipLaunchKernelGGL((k_tree_ll<DT, AR_AVG, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    default:
        hipLaunchKernelGGL((k_tree_ll<DT, AR_SUM, K>), dim3(grid), dim3(kBlock), 0, st, a);
        break;
    }
}

template <int DT>
void tree_launch_dt(const TreeArgs& a, int grid, hipStream_t st)
{
    // the larger tree half's sub-blocks: at most one per workgroup means one
    // line per thread
    const uint64_t half = a.H > a.N - a.H ? a.H : a.N - a.H;
    const uint64_t plen = a.piece_lo < half ? (a.piece_len < half - a.piece_lo ? a.piece_len : half - a.piece_lo) : 0;
    const uint64_t nsub = (plen + kBlock - 1) / kBlock;
    if (nsub <= (uint64_t)a.blocks_per_rank)
        tree_launch_k<DT, 1>(a, grid, st);
    else
        tree_launch_k<DT, kTreeEPT>(a, grid, st);
}

}  // namespace

hipError_t launch_tree_ll(int dtype, const TreeArgs& a, int grid, hipStream_t st)
{
    switch (dtype) {
    case AR_INT32:
        tree_launch_dt<AR_INT32>(a, grid, st);
        break;
    case AR_FLOAT32:
        tree_launch_dt<AR_FLOAT32>(a, grid, st);
        break;
    case AR_BF16:
        tree_launch_dt<AR_BF16>(a, grid, st);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int resident_tree_ll(int dtype)
{
    switch (dtype) {
    case AR_INT32:
        return resident_tree_dt<AR_INT32>();
    case AR_FLOAT32:
        return resident_tree_dt<AR_FLOAT32>();
    case AR_BF16:
        return resident_tree_dt<AR_BF16>();
    }
    return 0;
}

}  // namespace ar
