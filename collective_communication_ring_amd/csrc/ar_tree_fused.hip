// ar_tree_fused.hip -- the double binary tree in fused form, for gfx950
// (MI355X): one launch, no LL lines.
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
// their own.  A bfloat16 row cannot hold a float32 partial, so there an inner
// node's partial travels in two 16-bit halves, in its own row and in its
// first child's.)  An empty asm memory clobber after every level keeps the
// compiler from forwarding values in registers.
//
// Each tree is walked level by level: all loads of a level are issued, then
// used, so a hop costs one round trip per level, not per node -- 2(depth)
// round trips in all (6 at R = 8), against the ring's 2(R-1).  Every own
// input is read before the first row is written, so in place works.  The
// kernel is compiled for each R up to kTreeFusedMaxRanks and for 32 and 64
// (tree_fused_compiled); the host takes the LL tree for other R.
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

// Most levels of a compiled tree (7 at R = 64; a deeper shape would fail to
// compile: constant evaluation checks bounds).
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

// V consecutive elements of one row: one 16-byte access (V = 4 for 32-bit
// T, 8 for bfloat16) where the halves and rows are 16-byte aligned, else
// V = 1.  Packed bfloat16 elements sit two to a 32-bit word, the lower
// element in the low half (little endian).
template <class E, int V>
struct Pack {
    typename E::A v[V];
};

template <class E, int V>
constexpr bool kWide = V * sizeof(typename E::T) == 16;

// V elements of T, widened.
template <class E, int V>
__device__ inline Pack<E, V> load_t(const typename E::T* p)
{
    Pack<E, V> r;
    if constexpr (V == 1) {
        r.v[0] = E::widen(*p);
    } else {
        static_assert(kWide<E, V>, "one 16-byte access");
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if constexpr (sizeof(typename E::T) == 4)
                r.v[k] = E::from_bits(u[k]);
            else
                r.v[k] = E::widen(E::t_from_bits(u[k / 2] >> (16 * (k % 2))));
        }
    }
    return r;
}

// V elements narrowed to T (the final value at the root; for 32-bit T also
// a partial, which T holds exactly).
template <class E, int V>
__device__ inline void store_t(typename E::T* p, const Pack<E, V>& r)
{
    if constexpr (V == 1) {
        *p = E::narrow(r.v[0]);
    } else {
        u32x4 u = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if constexpr (sizeof(typename E::T) == 4)
                u[k] = E::t_bits(E::narrow(r.v[k]));
            else
                u[k / 2] |= E::t_bits(E::narrow(r.v[k])) << (16 * (k % 2));
        }
        *reinterpret_cast<u32x4*>(p) = u;
    }
}

// bfloat16 rows: one 16-bit half (HI: the upper, else the lower) of each
// float32 partial, laid out as V elements of T.
template <class E, int V, bool HI>
__device__ inline void store_half(typename E::T* p, const Pack<E, V>& r)
{
    auto half = [](typename E::A a) -> uint32_t {
        const uint32_t b = E::to_bits(a);
        return HI ? b >> 16 : b & 0xffffu;
    };
    if constexpr (V == 1) {
        *p = E::t_from_bits(half(r.v[0]));
    } else {
        u32x4 u = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < V; ++k)
            u[k / 2] |= half(r.v[k]) << (16 * (k % 2));
        *reinterpret_cast<u32x4*>(p) = u;
    }
}

// A float32 partial from its two halves, in rows hi and lo.
template <class E, int V>
__device__ inline Pack<E, V> load_halves(const typename E::T* hi, const typename E::T* lo)
{
    Pack<E, V> r;
    if constexpr (V == 1) {
        r.v[0] = E::from_bits((E::t_bits(*hi) << 16) | E::t_bits(*lo));
    } else {
        const u32x4 h = *reinterpret_cast<const u32x4*>(hi);
        const u32x4 l = *reinterpret_cast<const u32x4*>(lo);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t sh = 16 * (k % 2);
            r.v[k] = E::from_bits((((h[k / 2] >> sh) & 0xffffu) << 16) | ((l[k / 2] >> sh) & 0xffffu));
        }
    }
    return r;
}

// The raw bits of V elements, for the broadcast (no arithmetic).
template <class E, int V>
struct Raw {
    u32x4 w;
    typename E::T t;
};

template <class E, int V>
__device__ inline Raw<E, V> load_raw(const typename E::T* p)
{
    Raw<E, V> r;
    if constexpr (kWide<E, V>)
        r.w = *reinterpret_cast<const u32x4*>(p);
    else
        r.t = *p;
    return r;
}

template <class E, int V>
__device__ inline void store_raw(typename E::T* p, const Raw<E, V>& r)
{
    if constexpr (kWide<E, V>)
        *reinterpret_cast<u32x4*>(p) = r.w;
    else
        *p = r.t;
}

// Elements e .. e+V-1 through the whole tree TT (0: A, 1: B), every row
// index a constant; each of the V elements folds on its own, in the same
// order.  A node hands its partial to its parent through rows: for 32-bit T
// its own row holds it whole; for bfloat16 a leaf's partial is its own input
// (its row holds it exactly), and an inner node's float32 partial goes in two
// halves -- the upper in its own row, the lower in its first child's row,
// which it has just read and which only the broadcast writes again.
template <class E, int RED, int R, int TT, int V>
__device__ inline void tree_fused_elem(const typename E::T* x, typename E::T* y, uint64_t N,
                                       uint64_t e, float fr)
{
    constexpr bool kHalves = sizeof(typename E::T) == 2;
    constexpr FusedShape<R> S = fused_shape<R>();
    auto row = [&](int v) { return y + (uint64_t)v * N + e; };
    Pack<E, V> xin[R];  // own inputs, by breadth-first position, all loaded at once
#pragma unroll
    for (int i = 0; i < R; ++i)
        xin[i] = load_t<E, V>(x + (uint64_t)S.bfs[TT][i] * N + e);
    // up, deepest level first
#pragma unroll
    for (int L = S.nlev[TT] - 1; L >= 0; --L) {
        Pack<E, V> cv[R][2];
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i) {
            const int v = S.bfs[TT][i];
#pragma unroll
            for (int k = 0; k < S.nch[TT][v]; ++k) {
                const int c = S.ch[TT][v][k];
                if (kHalves && S.nch[TT][c] > 0)
                    cv[i][k] = load_halves<E, V>(row(c), row(S.ch[TT][c][0]));
                else
                    cv[i][k] = load_t<E, V>(row(c));
            }
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
            if (S.parent[TT][v] < 0) {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    acc.v[j] = finalize<E, RED>(acc.v[j], fr);
                store_t<E, V>(row(v), acc);  // the root: the final value
            } else if (!kHalves) {
                store_t<E, V>(row(v), acc);
            } else {
                store_half<E, V, true>(row(v), acc);  // a leaf: its input bits
                if (S.nch[TT][v] > 0)
                    store_half<E, V, false>(row(S.ch[TT][v][0]), acc);
            }
        }
        step_boundary();
    }
    // down, from the root's children
#pragma unroll
    for (int L = 1; L < S.nlev[TT]; ++L) {
        Raw<E, V> val[R];
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i)
            val[i] = load_raw<E, V>(row(S.parent[TT][S.bfs[TT][i]]));
#pragma unroll
        for (int i = S.lvl[TT][L]; i < S.lvl[TT][L + 1]; ++i)
            store_raw<E, V>(row(S.bfs[TT][i]), val[i]);
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
    // (with V > 1 the host guarantees that both halves are whole packs)
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
    if (r == 32 || r == 64) {  // one element per thread (the host never sets vec here)
        if (r == 32)
            hipLaunchKernelGGL((k_tree_fused_r<DT, RED, 32, 1>), dim3(grid), dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((k_tree_fused_r<DT, RED, 64, 1>), dim3(grid), dim3(kBlock), 0, st, a);
        return;
    }
    if constexpr (R <= kTreeFusedMaxRanks) {
        constexpr int kVec = 16 / (int)sizeof(typename Elem<DT>::T);
        if (r != R)
            tree_fused_launch_r<DT, RED, R + 1>(r, a, grid, st);
        else if (a.vec)
            hipLaunchKernelGGL((k_tree_fused_r<DT, RED, R, kVec>), dim3(grid), dim3(kBlock), 0, st,
                               a);
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
        if constexpr (DT != AR_INT32) {
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
    if (!tree_fused_compiled(R) || (a.vec && R > kTreeFusedMaxRanks))
        return hipErrorInvalidValue;
    switch (dtype) {
    case AR_INT32:
        return tree_fused_dt<AR_INT32>(R, a, grid, st);
    case AR_FLOAT32:
        return tree_fused_dt<AR_FLOAT32>(R, a, grid, st);
    case AR_BF16:
        return tree_fused_dt<AR_BF16>(R, a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ar
