// ar_internal.h -- definitions shared by the host side (ar_comm.cpp) and the
// HIP kernels (ar_ring.hip, ar_tree.hip) of libar.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

constexpr int kMaxRanks = 64;

// Words of the control block at the start of the workspace (uint32 each).
enum CtrlWord {
    kCtrlTreeEpoch = 0,  // unused (the tree keeps one epoch per group of lines)
    kCtrlError = 1,      // non-zero: a bounded wait expired (watchdog)
    kCtrlTreeDone = 2,   // unused
    kCtrlPipeDone = 3,   // workgroups of the running pipelined call that finished
    kCtrlRingLLEpoch = 4, // ring-LL: epoch of the last completed launch
    kCtrlRingLLDone = 5,  // ring-LL: workgroups of the running launch that finished
    kCtrlPipeBase = 8,   // uint64 at words 8-9: the value every chunk flag holds between
                         // pipelined calls; a call of n steps raises it by n
    kCtrlWords = 64      // 256 bytes
};

enum ErrorBits : uint32_t {
    kErrTimeout = 1u,
};

enum Op { kOpAllReduce = 0, kOpReduceScatter = 1, kOpAllGather = 2 };

// Double binary tree: per tree, per rank, the parent and up to two children
// (ascending), plus the root.  Built on the host, passed by value.
struct TreeTable {
    int8_t parent[2][kMaxRanks];
    int8_t child[2][kMaxRanks][2];
    int8_t nchild[2][kMaxRanks];
    int8_t root[2];
};

// The same table packed for the kernel, one 32-bit word per (tree, rank):
// bits 0-7 parent + 1 (0 at the root), bits 8-15 the number of children,
// bits 16-23 and 24-31 the children in ascending order.  A word is read with
// one scalar load; a byte table is read with vector loads, whose waits also
// wait for every store issued before them.
__host__ __device__ inline uint32_t tree_node_word(int parent, int nchild, int child0, int child1)
{
    return (uint32_t)(parent + 1) | ((uint32_t)nchild << 8) | ((uint32_t)child0 << 16) |
           ((uint32_t)child1 << 24);
}

// Arguments of one ring collective, shared by every ring launch mode.
//   send : [R][send_row] elements of T
//   part : the hand-off accumulators (A): the running value of element e of
//          segment c sits at part[c * part_seg + e] whichever rank holds it,
//          so each hop overwrites the slot the previous hop wrote
//   out  : [R][out_row] elements of T
// Segment c of the N-element vector is [min(c*S, N), min((c+1)*S, N)).
struct RingArgs {
    const void* send;
    void* part;
    uint64_t part_seg; // 0: one workspace row of N accumulators; out_row: the
                       //   owner's output row (A == T, the final lands there)
    void* out;
    uint32_t* ctrl;   // control block
    uint64_t* flags;  // pipelined ring: one ready flag per (segment, chunk)
    uint64_t N;       // logical elements per rank (all-reduce count; RS input row; AG output row)
    uint64_t S;       // segment length, ceil(N / R)
    uint64_t send_row;
    uint64_t out_row;
    uint64_t unit;    // pipelined ring: elements per flagged chunk (a multiple of the slot)
    uint64_t nunits;  // pipelined ring: chunks per segment, ceil(S / unit)
    uint64_t flag_stride; // pipelined ring: flags per segment in `flags`
    int xcd_pack;     // fused form, scalar path: only workgroups whose id is a multiple of
                      //   this take tiles (the others exit at once), so that they share one XCD
    uint64_t stage_wave; // fused form, vector path: accumulator elements of `part` per wave
                         //   (each wave's own staging slot, reused for every tile it takes:
                         //   whole tiles hand off through LDS, tiles cut short by a segment's
                         //   end through this slot); 0: the running value of element e of
                         //   segment c sits at part[c * part_seg + e]
    uint32_t max_units;  // fused form, vector path: waves that take tiles (the staging holds
                         //   this many); waves of the grid past it exit
    int ragged;          // fused form, vector path: some segment ends inside a wave tile
    int hand_lds;        // fused form, vector path: whole tiles hand the running value on
                         //   through LDS even where a row could take it
    uint64_t sub_lo;  // this channel's sub-range of every segment: [c*S + sub_lo,
    uint64_t sub_len; //   c*S + sub_lo + sub_len), clipped to the segment
    int m;            // this channel's ring stride: rank q receives from q - m
    int R;
    int op;           // Op
    int step;         // step-per-launch mode: the step this launch runs
    int per_rank_wg;  // pipelined ring: workgroups per logical rank
    int mute_rank;    // testing only: rank that skips publishing (-1: none)
    int redop;        // ar_redop_t
    uint64_t timeout_ticks;
};

struct TreeArgs {
    const void* send;
    void* out;
    uint64_t* up;     // [2 trees][R][piece_half] LL lines, child -> parent
    uint64_t* down;   // [2 trees][R][piece_half] LL lines, parent -> child
    uint32_t* epochs; // [2 trees][line_groups]: the flag of the last call that used each
                      //   group of kTreeGroup lines (0: never)
    uint64_t line_groups;
    uint32_t* ctrl;
    uint64_t N;
    uint64_t H;       // tree A's half: [0, H); tree B: [H, N)
    uint64_t piece_lo;   // this launch covers [piece_lo, piece_lo + piece_len) of each half
    uint64_t piece_len;
    uint64_t line_stride; // lines per (tree, rank) in up/down
    int R;
    int blocks_per_rank;  // workgroups per (tree, rank)
    int xcd_sets;         // XCDs the (tree, block) sets of R workgroups are dealt to
    int mute_rank;        // testing only: rank that skips publishing (-1: none)
    int redop;            // ar_redop_t
    uint64_t timeout_ticks;
    uint32_t node[2][kMaxRanks];  // tree_node_word of every (tree, rank)
};

// Ring with the LL protocol: every value a rank passes on travels as an
// 8-byte line lines[q][c][i] (sender q, segment c, offset i within this
// launch's piece of the segment).
struct RingLLArgs {
    const void* send;
    void* out;
    uint64_t* lines;     // [R][R][piece_cap]
    uint32_t* ctrl;
    uint64_t N;
    uint64_t S;
    uint64_t send_row;
    uint64_t out_row;
    uint64_t sub_lo;     // channel sub-range of every segment (see RingArgs)
    uint64_t sub_len;
    uint64_t piece_lo;   // this launch covers offsets [piece_lo, piece_lo + piece_len) of the sub-range
    uint64_t piece_len;
    uint64_t piece_cap;  // lines per (sender, segment)
    int m;               // ring stride
    int R;
    int op;
    int per_rank_wg;
    int xcd_sets;        // XCDs the sets of R workgroups (one per rank) are dealt to
    int mute_rank;
    int redop;
    uint64_t timeout_ticks;
};

// Launchers (ar_ring.hip / ar_tree.hip).  Return hipSuccess or the error.
hipError_t launch_ring_step(int dtype, bool vec, const RingArgs& a, int grid_x, hipStream_t s);
hipError_t launch_ring_placement(int dtype, bool vec, const RingArgs& a, int grid_x, hipStream_t s);
hipError_t launch_ring_fused(int dtype, bool vec, const RingArgs& a, int grid, hipStream_t s);
hipError_t launch_ring_fused_vec(int dtype, const RingArgs& a, int grid, hipStream_t s);
hipError_t launch_ring_pipelined(int dtype, bool vec, const RingArgs& a, int grid, hipStream_t s);
hipError_t launch_tree_ll(int dtype, const TreeArgs& a, int grid, hipStream_t s);
hipError_t launch_ring_ll(int dtype, const RingLLArgs& a, int grid, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);
hipError_t launch_fill_u64(uint64_t* p, uint64_t v, size_t n, hipStream_t s);

// Last HIP error of the utility calls (ar_stream_*, ar_ll_pingpong).
extern thread_local int g_util_hip_error;  // per host thread

// The allocation-free all-reduce's device array (ar_noalloc.hip): 8 MiB per
// GPU, the hand-off staging of 2,048 waves for bfloat16 (4,096 for 32-bit
// types).  noalloc_scratch gives the current device's copy and its size.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Largest number of workgroups of each persistent kernel that can be
// resident at once on the current device (0 on error).
int resident_ring_fused(int dtype, bool vec);
int resident_ring_fused_vec(int dtype);
int resident_ring_pipelined(int dtype, bool vec);
int resident_tree_ll(int dtype);
int resident_ring_ll(int dtype);

#ifndef AR_BLOCK
#define AR_BLOCK 256
#endif
#ifndef AR_UNROLL
#define AR_UNROLL 4
#endif
constexpr int kBlock = AR_BLOCK;   // threads per workgroup (4 wave64 by default)
constexpr int kUnroll = AR_UNROLL; // 16-byte vectors per thread per pass
// Fused form, vector path: a wave tile is 64 lanes x kWaveSlots 16-byte slots
// of one segment in every rank row (2 KiB of a row for 32-bit elements).
constexpr int kWaveSlots = 2;
constexpr uint32_t kWaveTileSlots = 64u * kWaveSlots;
// LL kernels' placement: a launch is made of sets of R workgroups (one per
// rank) that exchange lines only with each other.  Workgroups are dispatched
// to the XCDs round-robin (workgroup x to XCD x mod n), so set j is put on
// XCD j mod n: workgroup x plays rank (x / n) mod R of set x mod n + n *
// ((x / n) / R), and a line then travels between CUs of one XCD (LL
// ping-pong probe: ~0.37 us one way within an XCD, ~0.58 us between XCDs).
// The grid is rounded up to whole rows of n sets; workgroups past the last
// set have no work.
__host__ __device__ inline uint32_t ll_set_of(uint32_t x, uint32_t n, uint32_t R)
{
    return x % n + n * ((x / n) / R);
}
__host__ __device__ inline uint32_t ll_rank_of(uint32_t x, uint32_t n, uint32_t R)
{
    return (x / n) % R;
}
inline int64_t ll_grid_for_sets(int64_t sets, int n, int R)
{
    return (int64_t)n * R * ((sets + n - 1) / n);
}

constexpr int kTreeGroup = 64;   // LL lines per tree epoch (one wave's lines of a sub-block)
constexpr int kTreeEPT = 4;      // LL lines per thread per tree kernel pass
constexpr int kRingLLEPT = 4;    // LL lines per thread per ring-LL pass

}  // namespace ar
