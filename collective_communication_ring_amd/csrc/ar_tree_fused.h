// ar_tree_fused.h -- arguments of the fused double binary tree, shared by the
// host (ar_comm.cpp) and the kernel (ar_tree_fused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar_internal.h"

namespace ar {

// The fused tree is compiled for R = 2 .. kTreeFusedMaxRanks and for 32 and
// 64, each R with its trees fixed at compile time; 16-byte packs up to
// kTreeFusedMaxRanks (at 32 and 64 ranks one element per thread).
constexpr int kTreeFusedMaxRanks = 16;
inline bool tree_fused_compiled(int R)
{
    return (R >= 2 && R <= kTreeFusedMaxRanks) || R == 32 || R == 64;
}

// One launch covers the whole collective.  Workgroups [0, blocks_a) take the
// elements [0, H) of tree A, the others [H, N) of tree B, V elements per
// thread (a grid-stride loop on each half): V = 16 bytes of T (4 for 32-bit
// T, 8 for bfloat16) when vec is set, which the host does only for N above
// the grid's threads, a multiple of 2V, with both buffers 16-byte aligned (so
// every half and row starts on 16 bytes and each half is whole packs), else
// V = 1.
struct TreeFusedArgs {
    const void* send;
    void* out;
    uint64_t N;
    uint64_t H;
    int redop;
    int blocks_a;  // workgroups on tree A's half
    int vec;
};

// hipErrorInvalidValue for an unknown dtype, an R not compiled
// (tree_fused_compiled), vec at more than kTreeFusedMaxRanks ranks, or an
// integer AR_AVG.
hipError_t launch_tree_fused(int dtype, int R, const TreeFusedArgs& a, int grid, hipStream_t st);

}  // namespace ar
