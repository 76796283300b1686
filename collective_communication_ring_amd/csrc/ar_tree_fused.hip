// ar_tree_fused.hip -- the double binary tree in fused form, for gfx950
// (MI355X): one launch, no LL lines, 32-bit element types.
//
// The trees and their fold are those of the LL tree (ar_tree.hip): elements
// [0, H) go up tree A and back down, [H, N) tree B; a node's value is its own
// input, then each child's subtree value in ascending rank order; the root's
// value (averaged once for AR_AVG) comes back down unchanged ("NCCL and
// NVSHMEM -- two GPU communication models, side by side", section "double
// binary tree").
//
// As the fused ring does, one thread carries its element through every hop,
// and each hop is a store by the sender and a load by the receiver at the
// same address and by the same lane: a node sends up by storing its partial
// in its own output row, its parent loads it from there; going down, a node
// loads its parent's output row and stores its own.  (Those rows hold the
// final value once the broadcast has passed, so the hand-offs add no lines of
// their own.  32-bit T only: a bfloat16 row cannot hold a float32 partial;
// bfloat16 trees take the LL form.)  An empty asm memory clobber after every
// level keeps the compiler from forwarding values in registers.
//
// Each tree is walked level by level: all loads of a level are issued, then
// used, so a hop costs one round trip per level, not per node -- 2(depth)
// round trips in all (6 at R = 8), against the ring's 2(R-1).  Every own
// input is read before the first row is written, so in place works.  The
// kernel is compiled for each R up to kTreeFusedMaxRanks; the host takes the
// LL tree beyond that.
#include "ar_elem.h"
#include "ar_tree_fused.h"

namespace ar {
namespace {

// ---- the trees, at compile time ------------------------------------------
//
// The same trees as the host builds (ar_comm.cpp, build_trees): tree A is the
// in-order binary tree on 0..R-1 rooted at 0 (parent of r with lowest set bit
// b: r-b if bit 2b of r is set, else r+b if that is a rank, else r-b); tree B
// is tree A relabelled r -> R-1-r (even R) or r -> (r+1) mod R (odd R).  The
// kernel is compiled for each R, so a level's rows are constants: no table is
// read while the chain runs, and the own inputs are all loaded at once.
constexpr int shape_a_parent(int R, int r)
{
    if (r == 0)
        return -1;
    const int b = r & -r;
    if (r & (2 * b))
        return r - b;
    if (r + b < R)
        return r + b;
    return r - b;
}

constexpr int shape_parent(int R, int t, int r)
{
    if (t == 0)
        return shape_a_parent(R, r);
    if (R % 2 == 0) {
        const int p = shape_a_parent(R, R - 1 - r);
        return p < 0 ? -1 : R - 1 - p;
    }
    const int p = shape_a_parent(R, (r - 1 + R) % R);
    return p < 0 ? -1 : (p + 1) % R;
}

// Levels of a tree on at most kTreeFusedMaxRanks ranks (depth <= 5 at 16).
constexpr int kTreeMaxLevels = 8;

template <int R>
struct FusedShape {
    int parent[2][R];
    int nch[2][R];
    int ch[2][R][2];
    int bfs[2][R];
    int lvl[2][kTreeMaxLevels + 1];
    int nlev[2];
};

template <int R>
constexpr FusedShape<R> fused_shape()
{
    FusedShape<R> s{};
    for (int t = 0; t < 2; ++t) {
        int root = 0;
        for (int r = 0; r < R; ++r) {
            s.parent[t][r] = shape_parent(R, t, r);
            s.nch[t][r] = 0;
            if (s.parent[t][r] < 0)
                root = r;
        }
        for (int r = 0; r < R; ++r) {  // children in ascending rank order
            const int p = s.parent[t][r];
            if (p >= 0)
                s.ch[t][p][s.nch[t][p]++] = r;
        }
        int n = 0, L = 0, lo = 0;
        s.bfs[t][n++] = root;
        s.lvl[t][0] = 0;
        while (lo < n) {
            const int hi = n;
            s.lvl[t][++L] = hi;
            for (int i = lo; i < hi; ++i)
                for (int k = 0; k < s.nch[t][s.bfs[t][i]]; ++k)
                    s.bfs[t][n++] = s.ch[t][s.bfs[t][i]][k];
            lo = hi;
        }
        s.nlev[t] = L;
    }
    return s;
}

// V consecutive elements of one row: V = 4 (one 16-byte access) where the
// halves and rows are 16-byte aligned, else V = 1.
template <class E, int V>
struct Pack {
    typename E::A v[V];
};

template <class E, int V>
__device__ inline Pack<E, V> load_pack(const typename E::T* p)
{
    Pack<E, V> r;
    if constexpr (V == 1) {
        r.v[0] = E::widen(*p);
    } else {
        static_assert(V == 4 && sizeof(typename E::T) == 4, "16 bytes of 32-bit elements");
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r.v[k] = E::from_bits(u[k]);
    }
    return r;
}

template <class E, int V>
__device__ inline void store_pack(typename E::T* p, const Pack<E, V>& r)
{
    if constexpr (V == 1) {
        *p = E::narrow(r.v[0]);
    } else {
        u32x4 u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            u[k] = E::t_bits(E::narrow(r.v[k]));
        *reinterpret_cast<u32x4*>(p) = u;
    }
}

// The raw T bits of V elements, for the broadcast (no arithmetic).
template <int V>
struct Raw {
    uint32_t v[V];
};

template <class E, int V>
__device__ inline Raw<V> load_raw(const typename E::T* p)
{
    Raw<V> r;
    if constexpr (V == 1) {
        r.v[0] = E::t_bits(*p);
    } else {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r.v[k] = u[k];
    }
    return r;
}

template <class E, int V>
__device__ inline void store_raw(typename E::T* p, const Raw<V>& r)
{
    if constexpr (V == 1) {
        *p = E::t_from_bits(r.v[0]);
    } else {
        u32x4 u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            u[k] = r.v[k];
        *reinterpret_cast<u32x4*>(p) = u;
    }
}

// Elements e .. e+V-1 through the whole tree TT (0: A, 1: B), every row
// index a constant; each of the V elements folds on its own, in the same
// order.
template <class E, int RED, int R, int TT, int V>
__device__ inline void tree_fused_elem(const typename E::T* x, typename E::T* y, uint64_t N,
                                       uint64_t e, float fr)
{
    constexpr FusedShape<R> S = fused_shape<R>();
    Pack<E, V> xin[R];  // own inputs, by breadth-first position, all loaded at once
#pragma unroll
    for (int i = 0; i < R; ++i)
        xin[i] = load_pack<E, V>(x + (uint64_t)S.bfs[TT][i] * N + e);
    // up, deepest level first
#pragma unroll
    for (int L = S.nlev[TT] - 1; L >= 0; --L) {
        Pack<E, V> cv[R][2];
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i) {
            const int v = S.bfs[TT][i];
#pragma unroll
            for (int k = 0; k < S.nch[TT][v]; ++k)
                cv[i][k] = load_pack<E, V>(y + (uint64_t)S.ch[TT][v][k] * N + e);
        }
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i) {
            const int v = S.bfs[TT][i];
            Pack<E, V> acc = xin[i];
#pragma unroll
            for (int k = 0; k < S.nch[TT][v]; ++k)
#pragma unroll
                for (int j = 0; j < V; ++j)
                    acc.v[j] = combine<E, RED>(acc.v[j], cv[i][k].v[j]);
            if (S.parent[TT][v] < 0)
#pragma unroll
                for (int j = 0; j < V; ++j)
                    acc.v[j] = finalize<E, RED>(acc.v[j], fr);
            store_pack<E, V>(y + (uint64_t)v * N + e, acc);
        }
        step_boundary();
    }
    // down, from the root's children
#pragma unroll
    for (int L = 1; L < S.nlev[TT]; ++L) {
        Raw<V> val[R];
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i)
            val[i] = load_raw<E, V>(y + (uint64_t)S.parent[TT][S.bfs[TT][i]] * N + e);
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i)
            store_raw<E, V>(y + (uint64_t)S.bfs[TT][i] * N + e, val[i]);
        step_boundary();
    }
}

template <int DT, int RED, int R, int V>
__global__ __launch_bounds__(kBlock) void k_tree_fused_r(TreeFusedArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const T* x = static_cast<const T*>(a.send);
    T* y = static_cast<T*>(a.out);
    const uint64_t N = a.N;
    const float fr = (float)R;
    const bool tb = (int)blockIdx.x >= a.blocks_a;
    const uint64_t lo = tb ? a.H : 0, hi = tb ? N : a.H;
    const uint64_t b = tb ? blockIdx.x - a.blocks_a : blockIdx.x;
    const uint64_t nb = tb ? gridDim.x - a.blocks_a : a.blocks_a;
    // (with V = 4 the host guarantees that both halves are whole packs)
    for (uint64_t e = lo + (b * kBlock + threadIdx.x) * V; e < hi; e += nb * kBlock * V) {
        if (tb)
            tree_fused_elem<E, RED, R, 1, V>(x, y, N, e, fr);
        else
            tree_fused_elem<E, RED, R, 0, V>(x, y, N, e, fr);
    }
}

template <int DT, int RED, int R>
void tree_fused_launch_r(int r, const TreeFusedArgs& a, int grid, hipStream_t st)
{
    if constexpr (R <= kTreeFusedMaxRanks) {
        if (r != R)
            tree_fused_launch_r<DT, RED, R + 1>(r, a, grid, st);
        else if (a.vec)
            hipLaunchKernelGGL((k_tree_fused_r<DT, RED, R, 4>), dim3(grid), dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((k_tree_fused_r<DT, RED, R, 1>), dim3(grid), dim3(kBlock), 0, st, a);
    }
}

template <int DT>
hipError_t tree_fused_dt(int R, const TreeFusedArgs& a, int grid, hipStream_t st)
{
    switch (a.redop) {
    case AR_MAX:
        tree_fused_launch_r<DT, AR_MAX, 2>(R, a, grid, st);
        break;
    case AR_MIN:
        tree_fused_launch_r<DT, AR_MIN, 2>(R, a, grid, st);
        break;
    case AR_AVG:
        if constexpr (DT == AR_FLOAT32) {
            tree_fused_launch_r<DT, AR_AVG, 2>(R, a, grid, st);
            break;
        } else {
            return hipErrorInvalidValue;  // no integer average (refused on the host)
        }
    default:
        tree_fused_launch_r<DT, AR_SUM, 2>(R, a, grid, st);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_fused(int dtype, int R, const TreeFusedArgs& a, int grid, hipStream_t st)
{
    if (R < 2 || R > kTreeFusedMaxRanks)
        return hipErrorInvalidValue;
    switch (dtype) {
    case AR_INT32:
        return tree_fused_dt<AR_INT32>(R, a, grid, st);
    case AR_FLOAT32:
        return tree_fused_dt<AR_FLOAT32>(R, a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ar
