// ar_comm.cpp -- host side of libar: communicator, schedule tables,
// workspace layout, argument checking and dispatch to the HIP kernels.
//
// The communicator mirrors NCCL's host pattern: create once, then enqueue
// collectives on a stream and let the caller synchronize ("NCCL and NVSHMEM
// -- two GPU communication models, side by side", NCCL host code listing;
// "NCCL, NIXL, and Distributed GPU Communication", performance checklist on
// not creating communicators inside loops).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "ar.h"
#include "ar_internal.h"
#include "ar_tree_fused.h"

using namespace ar;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kDefaultChunkBytes = 512 * 1024;
constexpr int64_t kDefaultTimeoutUs = 2000000;      // 2 s bounded waits
// AR_AUTO's cost model: one line T(n) = alpha + n / bw per algorithm and ring
// launch form (n = bytes per rank), indexed by ar_cost_form_t.  Defaults are
// least-squares fits (weighted by 1/T^2) of graph-replayed all-reduces on
// MI355X, R = 8 float32, 8 B - 4 MiB per rank; the fused ring's line is the
// fit of its full 8 B - 1 GiB sweep.  With them the tree takes messages up to
// ~640 KB/rank against the pipelined ring, ~460 KB against ring + LL and
// ~1 MB against the step ring (measured: the tree is faster than each of them
// up to 512 KiB and slower from 1 MiB), and none against the fused ring.
// With AR_PROTO_AUTO the ring goes by LL where its line is below the simple
// form's: up to ~830 KB/rank against the pipelined ring and ~1.7 MB against
// the step ring (so with AR_AUTO: tree up to ~460 KB, then ring + LL, then
// the simple form), and at no size against the fused ring.
struct CostLine {
    double alpha_us;
    double bw_gbps;
};
constexpr CostLine kDefaultCost[AR_COST_FORMS] = {
    {5.9, 35.5},    // tree + LL
    {3.9, 356.0},   // ring, fused
    {21.7, 278.0},  // ring, pipelined (simple protocol: ready flags)
    {28.9, 179.0},  // ring, one launch per step
    {11.6, 63.2},   // ring + LL
    {2.8, 316.0},   // tree, fused
};
constexpr uint64_t kTreeLinesCap = 1u << 16;         // LL lines per (tree, rank) per launch
constexpr uint64_t kMaxChunkBytes = 1ull << 30;      // pipelined ring: largest chunk
// LL flags are 32-bit epochs advanced once per launch (ring + LL: 2e and
// 2e + 1; the tree: a group's epoch + 1): after this many tree and ring-LL
// launches the lines and epochs are cleared again, so no flag wraps around
// to a value that a stale line may still hold.
constexpr uint64_t kLLResetLaunches = 1ull << 30;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elem_size(int dtype) { return dtype == AR_BF16 ? 2 : 4; }

const char* dtype_name(int d)
{
    return d == AR_INT32 ? "int32" : d == AR_FLOAT32 ? "float32" : d == AR_BF16 ? "bf16" : "?";
}
const char* launch_name(int l)
{
    return l == AR_LAUNCH_STEP ? "step" : l == AR_LAUNCH_FUSED ? "fused"
         : l == AR_LAUNCH_PIPELINED ? "pipelined" : "auto";
}

// Tree A: the in-order binary tree on 0..R-1 rooted at 0.  For r >= 1 with
// lowest set bit b: parent r-b if bit 2b of r is set, else r+b if that is a
// rank, else r-b.  Tree B is tree A relabelled r -> R-1-r (even R) or
// r -> (r+1) mod R (odd R), so that the two trees use complementary links
// ("NCCL and NVSHMEM -- two GPU communication models, side by side", section
// "double binary tree").
int tree_a_parent(int R, int r)
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

int tree_parent_of(int R, int tree, int r)
{
    if (tree == 0)
        return tree_a_parent(R, r);
    if (R % 2 == 0) {
        const int p = tree_a_parent(R, R - 1 - r);
        return p < 0 ? -1 : R - 1 - p;
    }
    const int p = tree_a_parent(R, (r - 1 + R) % R);
    return p < 0 ? -1 : (p + 1) % R;
}

void build_trees(int R, TreeTable* tt)
{
    std::memset(tt, 0, sizeof *tt);
    for (int t = 0; t < 2; ++t) {
        for (int r = 0; r < R; ++r) {
            const int p = tree_parent_of(R, t, r);
            tt->parent[t][r] = (int8_t)p;
            if (p < 0)
                tt->root[t] = (int8_t)r;
        }
        // children in ascending rank order
        for (int r = 0; r < R; ++r) {
            const int p = tt->parent[t][r];
            if (p >= 0)
                tt->child[t][p][tt->nchild[t][p]++] = (int8_t)r;
        }
    }
}

int64_t env_int(const char* name, int64_t dflt)
{
    const char* s = std::getenv(name);
    if (!s || !*s)
        return dflt;
    return std::strtoll(s, nullptr, 0);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

struct ar_comm {
    int R = 0;
    size_t cap = 0;  // elements per rank row
    int dtype = AR_FLOAT32;
    int algo = AR_RING;
    int proto = AR_SIMPLE;
    // options
    int64_t chunk_bytes = kDefaultChunkBytes;
    int launch = AR_LAUNCH_AUTO;
    int64_t grid = 0;
    int64_t timeout_us = kDefaultTimeoutUs;
    int64_t debug = 0;
    int64_t tree_max_bytes = -1;  // AR_AUTO: -1 = by the cost model, else a fixed threshold
    CostLine cost[AR_COST_FORMS] = {kDefaultCost[0], kDefaultCost[1], kDefaultCost[2],
                                    kDefaultCost[3], kDefaultCost[4], kDefaultCost[5]};
    int64_t mute_rank = -1;  // testing the watchdog only
    int64_t redop = AR_SUM;
    int64_t channels = 1;
    int strides[kMaxRanks] = {};  // ring stride of each possible channel
    int nstrides = 0;
    // schedule
    TreeTable tt{};
    // workspace layout
    size_t off_part = 0, off_up = 0, off_down = 0, off_flags = 0, ws_need = 0;
    size_t part_bytes = 0;    // the hand-off region at off_part
    size_t off_tree_epochs = 0;
    uint64_t tree_lines = 0;  // lines per (tree, rank)
    uint64_t tree_groups = 0; // epoch words per tree: one per kTreeGroup lines
    uint64_t flag_stride = 0; // pipelined ring: ready flags per segment
    size_t off_rll = 0;       // ring-LL line slots
    uint64_t rll_cap = 0;     // ring-LL: lines per (sender, segment) per launch
    char* ws = nullptr;
    size_t ws_bytes = 0;
    // device facts, read on first use
    bool dev_ready = false;
    int ncu = 0;
    int nxcd = 1;             // XCDs (accelerator complex dies) of the device
    double ticks_per_us = 100.0;
    int resident_fused[3][2] = {};
    int resident_pipe[3][2] = {};
    int resident_tree[3] = {};
    int resident_rll[3] = {};
    // last call
    uint64_t ll_launches = 0;  // tree and ring-LL launches since their lines were cleared
    hipStream_t last_stream = nullptr;
    int last_hip = 0;
};

namespace {

int fail_hip(ar_comm* c, hipError_t e)
{
    c->last_hip = (int)e;
    return AR_ERR_HIP;
}

int device_ready(ar_comm* c)
{
    if (c->dev_ready)
        return AR_SUCCESS;
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&c->ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess)
        return fail_hip(c, e);
    if (khz > 0)
        c->ticks_per_us = khz / 1000.0;
    int nxcd = 0;
    if (hipDeviceGetAttribute(&nxcd, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && nxcd > 0)
        c->nxcd = nxcd;
    else
        (void)hipGetLastError();  // not known: no packing; keep the error from the next launch check
    for (int d = 0; d < 3; ++d) {
        c->resident_fused[d][0] = resident_ring_fused(d, false);
        c->resident_fused[d][1] = resident_ring_fused_vec(d);
        c->resident_pipe[d][0] = resident_ring_pipelined(d, false);
        c->resident_pipe[d][1] = resident_ring_pipelined(d, true);
        c->resident_tree[d] = resident_tree_ll(d);
        c->resident_rll[d] = resident_ring_ll(d);
        if (c->resident_fused[d][0] <= 0 || c->resident_fused[d][1] <= 0 ||
            c->resident_pipe[d][0] <= 0 || c->resident_pipe[d][1] <= 0 || c->resident_tree[d] <= 0 ||
            c->resident_rll[d] <= 0)
            return fail_hip(c, hipErrorInvalidDeviceFunction);
    }
    c->dev_ready = true;
    return AR_SUCCESS;
}

uint64_t timeout_ticks(const ar_comm* c)
{
    return (uint64_t)((double)c->timeout_us * c->ticks_per_us);
}

int resolve_launch(const ar_comm* c)
{
    if (c->launch != AR_LAUNCH_AUTO)
        return c->launch;
    return AR_LAUNCH_FUSED;
}

// The cost-model line of the ring's simple-protocol launch form.
int simple_ring_form(const ar_comm* c)
{
    switch (resolve_launch(c)) {
    case AR_LAUNCH_STEP:
        return AR_COST_RING_STEP;
    case AR_LAUNCH_PIPELINED:
        return AR_COST_RING_PIPELINED;
    default:
        return AR_COST_RING_FUSED;
    }
}

double cost_us(const CostLine& l, double bytes) { return l.alpha_us + bytes / (l.bw_gbps * 1e3); }

// Does a tree call take the fused form (one launch, hops through the nodes'
// output rows) rather than the LL form?  With the fused launch, a protocol
// other than LL and an R the kernel is compiled for (2 .. 16, 32, 64).
bool tree_fused_ok(const ar_comm* c)
{
    return c->proto != AR_LL && resolve_launch(c) == AR_LAUNCH_FUSED && tree_fused_compiled(c->R);
}

// The cost-model line of the tree as this comm would run it.
int tree_cost_form(const ar_comm* c)
{
    return tree_fused_ok(c) ? AR_COST_TREE_FUSED : AR_COST_TREE_LL;
}

// The ring's protocol for `bytes` per rank: the comm's, or with
// AR_PROTO_AUTO, LL where the ring + LL line is strictly below the
// simple-protocol form's.
int ring_proto(const ar_comm* c, double bytes)
{
    if (c->proto != AR_PROTO_AUTO)
        return c->proto;
    return cost_us(c->cost[AR_COST_RING_LL], bytes) <
                   cost_us(c->cost[simple_ring_form(c)], bytes)
               ? AR_LL
               : AR_SIMPLE;
}

// Bytes per rank the cost model weighs for a call over rows of `count`.
double call_bytes(const ar_comm* c, size_t count) { return (double)count * elem_size(c->dtype); }

// AR_AUTO: tree for small messages, ring for large ones, chosen by size
// ("NCCL and NVSHMEM -- two GPU communication models, side by side": the
// tree for latency at small sizes, the ring for bandwidth at large ones, and
// NCCL picks automatically).  The choice is whichever line of the cost model
// is lower at this size: the tree's, or that of the ring as the call would
// run it (its protocol, then its launch form).  A fixed threshold
// (AR_OPT_TREE_MAX_BYTES >= 0) overrides the model.
int resolve_algo(const ar_comm* c, size_t count)
{
    if (c->algo != AR_AUTO)
        return c->algo;
    const double bytes = call_bytes(c, count);
    if (c->tree_max_bytes >= 0)
        return bytes <= (double)c->tree_max_bytes ? AR_TREE : AR_RING;
    const int form = ring_proto(c, bytes) == AR_LL ? AR_COST_RING_LL : simple_ring_form(c);
    return cost_us(c->cost[tree_cost_form(c)], bytes) < cost_us(c->cost[form], bytes) ? AR_TREE
                                                                                        : AR_RING;
}

// The protocol of a call whose algorithm is `algo` (the LL tree moves LL
// lines; the fused tree, like the fused ring, has no protocol of its own and
// reports AR_SIMPLE).
int resolve_proto(const ar_comm* c, size_t count, int algo)
{
    if (algo == AR_TREE)
        return tree_fused_ok(c) ? AR_SIMPLE : AR_LL;
    return ring_proto(c, call_bytes(c, count));
}

// The per-rank sizes n >= 0 (bytes) at which line a is strictly below line
// b, as an integer range [lo, hi] (lo > hi: none; hi = INT64_MAX: no upper
// end).  Two lines meet once at most, so the range is empty, everything, a
// prefix [0, hi] or a suffix [lo, INT64_MAX].  The meeting point is found in
// floating point, then the ends are stepped (a few steps at most) to the
// exact integers at which the same comparison resolve_algo makes changes.
struct Span {
    int64_t lo, hi;
};

Span below(const CostLine& a, const CostLine& b)
{
    constexpr double kBig = 4e15;  // integers are exact in a double far beyond this
    auto lt = [&](int64_t n) { return cost_us(a, (double)n) < cost_us(b, (double)n); };
    const double da = a.alpha_us - b.alpha_us;
    const double ds = 1.0 / (a.bw_gbps * 1e3) - 1.0 / (b.bw_gbps * 1e3);
    if (ds == 0.0)
        return da < 0.0 ? Span{0, INT64_MAX} : Span{1, 0};
    const double x = -da / ds;  // where the lines meet
    if (ds > 0.0) {
        // a rises faster: below b up to the meeting point
        if (x >= kBig)
            return Span{0, INT64_MAX};
        int64_t hi = x <= 0.0 ? 0 : (int64_t)x;
        for (int i = 0; i < 64 && hi > 0 && !lt(hi); ++i)
            --hi;
        for (int i = 0; i < 64 && lt(hi + 1); ++i)
            ++hi;
        return lt(hi) ? Span{0, hi} : Span{1, 0};
    }
    // a rises more slowly: below b from the meeting point on
    if (x >= kBig)
        return Span{1, 0};
    int64_t lo = x <= 0.0 ? 0 : (int64_t)x;
    for (int i = 0; i < 64 && lo > 0 && lt(lo - 1); ++i)
        --lo;
    for (int i = 0; i < 64 && !lt(lo); ++i)
        ++lo;
    return Span{lo, INT64_MAX};
}

Span intersect(Span a, Span b) { return Span{std::max(a.lo, b.lo), std::min(a.hi, b.hi)}; }

// Do the 16-byte vector kernels apply?  Every row start and every segment
// start must be 16-byte aligned in both T and accumulator units, and a
// segment must be at least AR_SCALAR_SEG_BYTES long.  Shorter segments take
// the scalar path (one element per lane) in every ring form: a short
// segment's few loads and stores per step are then single instructions, and
// 16-byte slots only pay once a segment has enough of them (R = 8 fp32,
// fused, graph-replayed: 1-8 KiB per rank 6.0 /
// 6.1 / 5.8 / 5.9 us with the vector path from 128-byte segments, 5.3 / 5.2
// / 5.3 / 5.5 us with this threshold; the step form 30 -> 27.5 us there; a
// 8 KiB threshold was slower at 32 KiB per rank and at R = 4, 16 KiB).
#ifndef AR_SCALAR_SEG_BYTES
#define AR_SCALAR_SEG_BYTES 2048
#endif

bool vector_ok(const ar_comm* c, const void* send, const void* part, const void* out,
               uint64_t N, uint64_t S, uint64_t send_row, uint64_t out_row)
{
    const uint64_t es = (uint64_t)elem_size(c->dtype);
    if (S * es < AR_SCALAR_SEG_BYTES)
        return false;
    return aligned16(send) && aligned16(part) && aligned16(out) && (N * es) % 16 == 0 &&
           (S * es) % 16 == 0 && (send_row * es) % 16 == 0 && (out_row * es) % 16 == 0 &&
           (N * 4) % 16 == 0 && (S * 4) % 16 == 0;
}

// Does the fused form take its 16-byte vector path for a channel whose
// segments are sub_len long?  Its scalar path runs tiles of kBlock elements,
// one per thread, each tile's 2(R-1)-step chain a latency-bound run by lone
// waves; while its tiles number at most two per CU it is the faster one (its
// reduce steps hand off through LDS; R = 8, graph-replayed: fp32 512 KiB per
// rank 4.4-4.5 against 4.7 us, bf16 256 KiB 4.3 against 5.6 us on the vector
// path; at four per CU, fp32 1 MiB, 6.4 against 5.2 us).
bool fused_vector(const ar_comm* c, const void* send, const void* part, const void* out,
                  uint64_t N, uint64_t S, uint64_t send_row, uint64_t out_row, uint64_t sub_len)
{
    if (!vector_ok(c, send, part, out, N, S, send_row, out_row))
        return false;
    const uint64_t tiles = (sub_len + kBlock - 1) / kBlock * (uint64_t)c->R;
    return tiles > 2 * (uint64_t)c->ncu;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int ring_grid_x(const ar_comm* c, uint64_t S, bool vec)
{
    const uint64_t V = vec ? (c->dtype == AR_BF16 ? 8 : 4) : 1;
    const uint64_t slots = (S + V - 1) / V;
    const uint64_t per_wg = (uint64_t)kBlock * kUnroll;
    uint64_t need = (slots + per_wg - 1) / per_wg;
    const int64_t total = c->grid > 0 ? c->grid : (int64_t)c->ncu * 8;
    uint64_t cap = (uint64_t)std::max<int64_t>(1, total / c->R);
    need = std::max<uint64_t>(1, std::min(need, cap));
    return (int)std::min<uint64_t>(need, 65535);
}

// Workgroups per rank (per tree and rank for the tree) of an LL kernel over
// `lines` lines per rank, cut into sub-blocks of kBlock: one line per thread
// while the whole grid stays within one workgroup per CU (the latency-best
// shape), beyond that each thread batches up to `ept` lines (more
// workgroups would only add polling traffic); never above the residency cap.
uint64_t ll_grid_per_rank(uint64_t lines, int groups, int ncu, int ept, int64_t cap)
{
    const uint64_t nsub = (lines + kBlock - 1) / kBlock;
    const uint64_t batched = (nsub + ept - 1) / ept;
    const uint64_t budget = (uint64_t)std::max(1, ncu / groups);
    uint64_t g = std::min<uint64_t>(nsub, std::max<uint64_t>(batched, budget));
    return std::max<uint64_t>(1, std::min<uint64_t>(g, (uint64_t)cap));
}

// Before each tree or ring-LL launch: once kLLResetLaunches of them have run
// since the lines were cleared, clear the tree's lines and group epochs, the
// ring-LL lines and the ring-LL epoch word on the stream, so the launch
// starts again from epoch 1.  The error word and the pipelined ring's 64-bit
// flags are left alone.
hipError_t ll_clear(ar_comm* c, hipStream_t st)
{
    hipError_t e = launch_fill_u64(reinterpret_cast<uint64_t*>(c->ws + c->off_up), 0ull,
                                   (c->off_flags - c->off_up) / sizeof(uint64_t), st);
    if (e == hipSuccess)
        e = launch_fill_u64(reinterpret_cast<uint64_t*>(c->ws + c->off_rll), 0ull,
                            (c->ws_need - c->off_rll) / sizeof(uint64_t), st);
    if (e == hipSuccess)
        e = launch_fill_u32(reinterpret_cast<uint32_t*>(c->ws) + kCtrlRingLLEpoch, 0u, 1, st);
    if (e == hipSuccess)
        c->ll_launches = 0;
    return e;
}

int ll_launch_guard(ar_comm* c, hipStream_t st)
{
    if (c->ll_launches >= kLLResetLaunches) {
        hipError_t e = ll_clear(c, st);
        if (e != hipSuccess)
            return fail_hip(c, e);
    }
    ++c->ll_launches;
    return AR_SUCCESS;
}

// Ring with the LL protocol: one launch per piece of the segments.
int run_ring_ll(ar_comm* c, const RingArgs& r, hipStream_t st)
{
    RingLLArgs a{};
    a.send = r.send;
    a.out = r.out;
    a.lines = reinterpret_cast<uint64_t*>(c->ws + c->off_rll);
    a.ctrl = reinterpret_cast<uint32_t*>(c->ws);
    a.N = r.N;
    a.S = r.S;
    a.send_row = r.send_row;
    a.out_row = r.out_row;
    a.piece_cap = c->rll_cap;
    a.sub_lo = r.sub_lo;
    a.sub_len = r.sub_len;
    a.m = r.m;
    a.R = r.R;
    a.op = r.op;
    a.mute_rank = (int)c->mute_rank;
    a.redop = (int)c->redop;
    a.timeout_ticks = r.timeout_ticks;
    // every workgroup must be resident: at most the occupancy limit, and at
    // most AR_OPT_GRID (a stream held to fewer CUs holds fewer workgroups)
    const int64_t res = c->grid > 0 ? std::min<int64_t>(c->resident_rll[c->dtype], c->grid)
                                    : (int64_t)c->resident_rll[c->dtype];
    const int64_t gmax = res / a.R;
    if (gmax < 1)
        return AR_ERR_UNSUPPORTED;
    int launches = 0;
    for (uint64_t lo = 0; lo < a.sub_len; lo += c->rll_cap) {
        a.piece_lo = lo;
        a.piece_len = std::min<uint64_t>(c->rll_cap, a.sub_len - lo);
        a.per_rank_wg = (int)ll_grid_per_rank(a.piece_len, a.R, c->ncu, kRingLLEPT, gmax);
        // sets of R workgroups on one XCD each, the grid rounded up to whole
        // rows of sets; every workgroup must still be resident
        a.xcd_sets = c->nxcd;
        while (a.per_rank_wg > 1 && ll_grid_for_sets(a.per_rank_wg, a.xcd_sets, a.R) > res)
            --a.per_rank_wg;
        if (ll_grid_for_sets(a.per_rank_wg, a.xcd_sets, a.R) > res)
            a.xcd_sets = 1;
        const int64_t grid = ll_grid_for_sets(a.per_rank_wg, a.xcd_sets, a.R);
        const int rc = ll_launch_guard(c, st);
        if (rc)
            return rc;
        hipError_t e = launch_ring_ll(c->dtype, a, (int)grid, st);
        if (e != hipSuccess)
            return fail_hip(c, e);
        ++launches;
    }
    if (c->debug)
        std::fprintf(stderr, "ar: ring-LL op=%d R=%d N=%llu dtype=%s launches=%d\n", a.op, a.R,
                     (unsigned long long)a.N, dtype_name(c->dtype), launches);
    return AR_SUCCESS;
}

// How one ring call runs beyond its arguments: where the fused form may stage
// hand-offs (a.part, when it is this region), and whether the call must take
// the fused form whatever the comm's options say (the allocation-free entry
// point, which has no flags or lines to offer the other forms).
struct RunOpts {
    const void* stage = nullptr;  // the region a.part points at when staging is allowed
    size_t stage_bytes = 0;
    bool fused_only = false;
    int proto = AR_SIMPLE;        // the call's ring protocol (resolve_proto)
};

int run_ring_channel(ar_comm* c, RingArgs& a, hipStream_t st, const RunOpts& o);

// One ring collective: every channel covers its own sub-range of every
// segment with its own ring stride, launched one after the other.
int run_ring(ar_comm* c, RingArgs& a, hipStream_t st, const RunOpts& o)
{
    const uint64_t K = (uint64_t)c->channels;
    const uint64_t Sk = ((a.S + K - 1) / K + 7) / 8 * 8;
    for (uint64_t k = 0; k < K; ++k) {
        a.m = c->strides[k];
        a.sub_lo = k * Sk;
        if (a.sub_lo >= a.S && k > 0)
            break;  // nothing left for later channels
        // the kernels clip the sub-range to each segment's end; clipping its
        // length to what a full segment holds changes no range, and keeps grids
        // and LL pieces from covering a rounded-up tail
        a.sub_len = std::min<uint64_t>(Sk, a.S - a.sub_lo);
        const int rc = run_ring_channel(c, a, st, o);
        if (rc)
            return rc;
    }
    return AR_SUCCESS;
}

int run_ring_channel(ar_comm* c, RingArgs& a, hipStream_t st, const RunOpts& o)
{
    if (o.proto == AR_LL && !o.fused_only)
        return run_ring_ll(c, a, st);
    a.mute_rank = (int)c->mute_rank;
    a.redop = (int)c->redop;
    const bool vec = vector_ok(c, a.send, a.part, a.out, a.N, a.S, a.send_row, a.out_row);
    const int launch = o.fused_only ? AR_LAUNCH_FUSED : resolve_launch(c);
    hipError_t e = hipSuccess;
    int grid = 0;
    if (launch == AR_LAUNCH_STEP) {
        const int gx = ring_grid_x(c, a.sub_len, vec);
        grid = gx * a.R;
        int nsteps = 0;
        if (a.op == kOpAllGather) {
            e = launch_ring_placement(c->dtype, vec, a, gx, st);
            nsteps = a.R - 1;
        } else {
            nsteps = (a.op == kOpAllReduce) ? 2 * (a.R - 1) : a.R - 1;
        }
        for (int s = 0; s < nsteps && e == hipSuccess; ++s) {
            a.step = s;
            e = launch_ring_step(c->dtype, vec, a, gx, st);
        }
    } else if (launch == AR_LAUNCH_FUSED && vec &&
               fused_vector(c, a.send, a.part, a.out, a.N, a.S, a.send_row, a.out_row, a.sub_len)) {
        // wave tiles of kWaveTileSlots 16-byte slots; two workgroups (8 waves)
        // per CU by default
        const uint64_t V = c->dtype == AR_BF16 ? 8 : 4;
        const uint64_t tps = ((a.sub_len + V - 1) / V + kWaveTileSlots - 1) / kWaveTileSlots;
        const uint64_t units = tps * (uint64_t)a.R;
        const uint64_t waves = (uint64_t)(kBlock / 64);
        const int64_t want = c->grid > 0 ? c->grid : 2 * (int64_t)c->ncu;
        uint64_t g = std::min<uint64_t>((units + waves - 1) / waves, (uint64_t)want);
        // does any segment of this channel end inside a tile? (then the kernel
        // with the checked path for a segment's last tile is launched)
        a.ragged = 0;
        for (int sc = 0; sc < a.R && !a.ragged; ++sc) {
            const uint64_t slo = std::min<uint64_t>((uint64_t)sc * a.S, a.N);
            const uint64_t send_ = std::min<uint64_t>((uint64_t)(sc + 1) * a.S, a.N);
            const uint64_t x0 = std::min<uint64_t>(slo + a.sub_lo, send_);
            const uint64_t x1 = std::min<uint64_t>(slo + a.sub_lo + a.sub_len, send_);
            a.ragged = ((x1 - x0) % (kWaveTileSlots * V)) != 0;
        }
        a.stage_wave = 0;
        a.max_units = 0xffffffffu;
        // reduce steps hand off through LDS for every reduce-scatter and every
        // all-reduce whose rows total at most 512 MiB (measured crossover: LDS
        // 7-13% faster up to 32 MiB per rank at R = 8 float32, level at 64 MiB,
        // ~7% slower from 128 MiB, where the owner's output row takes it)
        a.hand_lds = (a.op == kOpReduceScatter ||
                      2.0 * a.R * (double)a.N * elem_size(c->dtype) <= 512.0 * (1 << 20))
                         ? 1 : 0;
        if (a.op != kOpAllGather && o.stage && a.part == o.stage) {
            // whole tiles hand off through LDS, tiles cut short by a segment's end
            // through each wave's staging slot in the hand-off region: at most as
            // many waves as it holds slots take tiles
            a.stage_wave = (uint64_t)kWaveTileSlots * V;
            const uint64_t slots = o.stage_bytes / (a.stage_wave * 4);
            if (slots < 1)
                return AR_ERR_INTERNAL;
            a.max_units = (uint32_t)std::min<uint64_t>(slots, 0xffffffffu);
            g = std::min<uint64_t>(g, (slots + waves - 1) / waves);
        }
        grid = (int)std::max<uint64_t>(1, std::min<uint64_t>(g, 1u << 20));
        e = launch_ring_fused_vec(c->dtype, a, grid, st);
    } else if (launch == AR_LAUNCH_FUSED) {
        // tiles of kBlock elements, one per thread: a tile's chain of 2(R-1)
        // steps is latency-bound, and one element per thread keeps each step
        // to the fewest instructions.  Up to 8 workgroups per CU, so that a
        // large call on rows that are not 16-byte aligned still has enough
        // chains in flight to stream.
        const uint64_t tiles = (a.sub_len + kBlock - 1) / kBlock * (uint64_t)a.R;
        const int64_t want = c->grid > 0 ? c->grid : 8 * (int64_t)c->ncu;
        grid = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)tiles, want, 1 << 20}));
        // On the scalar path (segments shorter than a cache line, so lines are
        // shared between the tiles of different segments) the tiles stay on one
        // XCD: workgroups go to the XCDs round-robin (workgroup i to XCD i mod
        // n), so the launch has n times the workgroups and only every n-th
        // takes tiles.  Spread over the XCDs each shared line was written from
        // several L2s (R = 8 fp32, 32-512 B/rank: 6.0-7.0 us a call, 5.5 us
        // packed).  The vector path gains nothing and loses at 64-128 KiB/rank,
        // where one XCD's CUs and L2 are too few (6.6 against 5.9 us).
        a.xcd_pack = 1;
        if (c->grid <= 0 && c->nxcd > 1 && tiles * (uint64_t)c->nxcd <= (uint64_t)c->ncu) {
            a.xcd_pack = c->nxcd;
            grid = (int)tiles * c->nxcd;
        }
        e = launch_ring_fused(c->dtype, false, a, grid, st);
    } else if (launch == AR_LAUNCH_PIPELINED) {
        const int res = c->resident_pipe[c->dtype][vec ? 1 : 0];
        int64_t gmax = res / a.R;
        if (c->grid > 0)
            gmax = std::min<int64_t>(gmax, c->grid / a.R);
        if (gmax < 1)
            return AR_ERR_UNSUPPORTED;
        const uint64_t V = vec ? (c->dtype == AR_BF16 ? 8 : 4) : 1;
        const uint64_t tile = (uint64_t)kBlock * kUnroll * V;  // elements per workgroup pass
        const uint64_t es = (uint64_t)elem_size(c->dtype);
        uint64_t unit = c->chunk_bytes > 0 ? (uint64_t)c->chunk_bytes / es : a.sub_len;
        // a chunk's elements and its 4-byte accumulators are each addressed
        // through one buffer resource (byte offsets below 2 GiB): cap both at
        // 1 GiB, i.e. the chunk at kMaxChunkBytes / 4 elements whatever T
        unit = std::min<uint64_t>(unit, kMaxChunkBytes / 4);
        unit = std::max<uint64_t>(tile, unit / tile * tile);
        uint64_t nunits = (a.sub_len + unit - 1) / unit;
        // the chunk is the pipelining unit; cut it finer when a segment has
        // fewer chunks than there are workgroups per rank
        while (nunits < (uint64_t)gmax && unit > tile) {
            unit = std::max<uint64_t>(tile, (unit / 2 + tile - 1) / tile * tile);
            nunits = (a.sub_len + unit - 1) / unit;
        }
        uint64_t G = std::min<uint64_t>(nunits, (uint64_t)gmax);
        G = (nunits + (nunits + G - 1) / G - 1) / ((nunits + G - 1) / G);  // balance chunks per workgroup
        if (nunits > c->flag_stride)
            return AR_ERR_INTERNAL;
        a.flags = reinterpret_cast<uint64_t*>(c->ws + c->off_flags);
        a.flag_stride = c->flag_stride;
        a.unit = unit;
        a.nunits = nunits;
        a.per_rank_wg = (int)G;
        grid = (int)G * a.R;
        e = launch_ring_pipelined(c->dtype, vec, a, grid, st);
    } else {
        return AR_ERR_UNSUPPORTED;
    }
    if (c->debug)
        std::fprintf(stderr,
                     "ar: ring op=%d R=%d N=%llu dtype=%s launch=%s vec=%d grid=%d\n", a.op, a.R,
                     (unsigned long long)a.N, dtype_name(c->dtype), launch_name(launch), (int)vec,
                     grid);
    if (e != hipSuccess)
        return fail_hip(c, e);
    return AR_SUCCESS;
}

int run_tree(ar_comm* c, const void* send, void* recv, uint64_t N, hipStream_t st)
{
    TreeArgs a{};
    a.send = send;
    a.out = recv;
    a.up = reinterpret_cast<uint64_t*>(c->ws + c->off_up);
    a.down = reinterpret_cast<uint64_t*>(c->ws + c->off_down);
    a.epochs = reinterpret_cast<uint32_t*>(c->ws + c->off_tree_epochs);
    a.line_groups = c->tree_groups;
    a.ctrl = reinterpret_cast<uint32_t*>(c->ws);
    a.N = N;
    a.H = (N + 1) / 2;
    a.R = c->R;
    a.line_stride = c->tree_lines;
    a.timeout_ticks = timeout_ticks(c);
    a.mute_rank = (int)c->mute_rank;
    a.redop = (int)c->redop;
    for (int t = 0; t < 2; ++t)
        for (int r = 0; r < c->R; ++r)
            a.node[t][r] = tree_node_word(c->tt.parent[t][r], c->tt.nchild[t][r],
                                          c->tt.child[t][r][0], c->tt.child[t][r][1]);
    // every workgroup must be resident at once: at most res / (2R) per
    // (tree, rank), res being the occupancy limit capped by AR_OPT_GRID; a
    // workgroup loops over its sub-blocks of kBlock lines
    const int64_t res = c->grid > 0 ? std::min<int64_t>(c->resident_tree[c->dtype], c->grid)
                                    : (int64_t)c->resident_tree[c->dtype];
    const int64_t bpr_max = res / (2 * c->R);
    if (bpr_max < 1)
        return AR_ERR_UNSUPPORTED;
    const uint64_t half = a.H;  // the larger half
    const uint64_t piece = std::min<uint64_t>(c->tree_lines, std::max<uint64_t>(half, 1));
    int launches = 0;
    for (uint64_t lo = 0; lo < half; lo += piece) {
        a.piece_lo = lo;
        a.piece_len = piece;
        const uint64_t plen = std::min<uint64_t>(piece, half - lo);
        a.blocks_per_rank = (int)ll_grid_per_rank(plen, 2 * c->R, c->ncu, kTreeEPT, bpr_max);
        // sets of R workgroups on one XCD each (ll_set_of), the grid rounded
        // up to whole rows of sets; every workgroup must still be resident
        a.xcd_sets = c->nxcd;
        while (a.blocks_per_rank > 1 &&
               ll_grid_for_sets(2 * (int64_t)a.blocks_per_rank, a.xcd_sets, c->R) > res)
            --a.blocks_per_rank;
        if (ll_grid_for_sets(2 * (int64_t)a.blocks_per_rank, a.xcd_sets, c->R) > res)
            a.xcd_sets = 1;
        const int grid = (int)ll_grid_for_sets(2 * (int64_t)a.blocks_per_rank, a.xcd_sets, c->R);
        if (grid > res)
            return AR_ERR_INTERNAL;
        const int rc = ll_launch_guard(c, st);
        if (rc)
            return rc;
        hipError_t e = launch_tree_ll(c->dtype, a, grid, st);
        if (e != hipSuccess)
            return fail_hip(c, e);
        ++launches;
    }
    if (c->debug)
        std::fprintf(stderr, "ar: tree-LL R=%d N=%llu dtype=%s piece=%llu launches=%d\n", c->R,
                     (unsigned long long)N, dtype_name(c->dtype), (unsigned long long)piece,
                     launches);
    return AR_SUCCESS;
}

// The fused tree: one launch, tree A's elements on the first workgroups and
// tree B's on the rest, one element per thread (each a grid-stride loop).
int run_tree_fused(ar_comm* c, const void* send, void* recv, uint64_t N, hipStream_t st)
{
    TreeFusedArgs a{};
    a.send = send;
    a.out = recv;
    a.N = N;
    a.H = (N + 1) / 2;
    a.redop = (int)c->redop;
    // up to 4 workgroups per CU in all (or AR_OPT_GRID), shared by the two
    // halves in proportion, at least one for a half that has elements
    const int64_t total = c->grid > 0 ? c->grid : 4 * (int64_t)c->ncu;
    // 16-byte packs (4 or 8 elements) when one element per thread would take
    // more than one pass of the grid, every half and row starts on 16 bytes
    // and R <= kTreeFusedMaxRanks (at 32 and 64 ranks a pack per node would
    // not fit in registers).  (Small calls keep one element per thread: the chain is latency
    // bound there, and more waves carry it sooner.  Large ones move 16 bytes
    // per access, which also keeps their speed when send and recv sit a large
    // power of two apart: one element per thread slowed by ~1.6x there.)
    const uint64_t pack = 16 / elem_size(c->dtype);  // elements in 16 bytes
    a.vec = (c->R <= kTreeFusedMaxRanks && N > (uint64_t)total * kBlock && N % (2 * pack) == 0 &&
             aligned16(send) && aligned16(recv))
                ? 1 : 0;
    // The packed form keeps each non-root output line in L2 from its partial
    // to its final value only while few waves are in flight: by default 2
    // workgroups per CU while the call's rows (2 R N s) fit in half the
    // 256 MB Infinity Cache, else 1 (at 4 waves per CU each XCD's waves hold
    // ~4 MiB of dirty lines, its L2's size, and the partials reached HBM:
    // 1.8x the compulsory writes at R = 8 fp32 64 MiB per rank).
    int64_t grid_total = total;
    if (a.vec && c->grid <= 0) {
        const double rows = 2.0 * c->R * (double)N * elem_size(c->dtype);
        grid_total = (rows <= 128.0 * (1 << 20) ? 2 : 1) * (int64_t)c->ncu;
    }
    const uint64_t per_block = (uint64_t)kBlock * (a.vec ? pack : 1);
    const uint64_t ha = a.H, hb = N - a.H;
    const uint64_t need_a = (ha + per_block - 1) / per_block;
    const uint64_t need_b = (hb + per_block - 1) / per_block;
    const uint64_t cap_a = std::max<uint64_t>(1, (uint64_t)grid_total / 2);
    const uint64_t ga = std::min<uint64_t>(need_a, cap_a);
    const uint64_t gb = hb ? std::min<uint64_t>(need_b,
                                                std::max<uint64_t>(1, (uint64_t)grid_total - ga))
                           : 0;
    a.blocks_a = (int)ga;
    const int grid = (int)(ga + gb);
    hipError_t e = launch_tree_fused(c->dtype, c->R, a, grid, st);
    if (c->debug)
        std::fprintf(stderr, "ar: tree-fused R=%d N=%llu dtype=%s vec=%d grid=%d\n", c->R,
                     (unsigned long long)N, dtype_name(c->dtype), a.vec ? (int)pack : 1, grid);
    if (e != hipSuccess)
        return fail_hip(c, e);
    return AR_SUCCESS;
}

// A call's run options: the workspace's hand-off region, where the
// collectives stage hand-offs, and the ring protocol for rows of `count`.
RunOpts ws_opts(const ar_comm* c, size_t count)
{
    RunOpts o;
    o.stage = c->ws + c->off_part;
    o.stage_bytes = c->part_bytes;
    o.proto = resolve_proto(c, count, AR_RING);
    return o;
}

// Checks shared by the collectives.  A zero-element call is a successful
// no-op whatever its pointers (an empty tensor may have a NULL data pointer);
// it returns AR_SUCCESS through *noop.
int common_checks(ar_comm* c, const void* send, void* recv, size_t n, bool* noop)
{
    *noop = false;
    if (!c)
        return AR_ERR_INVALID_ARG;
    if (!c->ws)
        return AR_ERR_INVALID_USAGE;
    if (n == 0) {
        *noop = true;
        return AR_SUCCESS;
    }
    if (!send || !recv)
        return AR_ERR_INVALID_ARG;
    return device_ready(c);
}

}  // namespace

extern "C" {

int ar_init(ar_comm_t* out, int R, size_t count, ar_dtype_t dtype, ar_algo_t algo,
            ar_proto_t proto)
{
    if (!out)
        return AR_ERR_INVALID_ARG;
    *out = nullptr;
    if (R < 2 || R > kMaxRanks)
        return AR_ERR_INVALID_ARG;
    if (dtype != AR_INT32 && dtype != AR_FLOAT32 && dtype != AR_BF16)
        return AR_ERR_INVALID_ARG;
    if (algo != AR_RING && algo != AR_TREE && algo != AR_AUTO)
        return AR_ERR_INVALID_ARG;
    if (proto != AR_SIMPLE && proto != AR_LL && proto != AR_PROTO_AUTO)
        return AR_ERR_INVALID_ARG;
    if (count > ((size_t)1 << 40))
        return AR_ERR_INVALID_ARG;
    ar_comm* c = new (std::nothrow) ar_comm();
    if (!c)
        return AR_ERR_INTERNAL;
    c->R = R;
    c->cap = count;
    c->dtype = dtype;
    c->algo = algo;
    c->proto = proto;
    c->chunk_bytes = env_int("AR_CHUNK_BYTES", kDefaultChunkBytes);
    c->timeout_us = env_int("AR_TIMEOUT_US", kDefaultTimeoutUs);
    c->debug = env_int("AR_DEBUG", 0);
    const char* l = std::getenv("AR_LAUNCH");
    if (l && !std::strcmp(l, "step"))
        c->launch = AR_LAUNCH_STEP;
    else if (l && !std::strcmp(l, "fused"))
        c->launch = AR_LAUNCH_FUSED;
    else if (l && !std::strcmp(l, "pipelined"))
        c->launch = AR_LAUNCH_PIPELINED;
    build_trees(R, &c->tt);
    // channel strides: 1, R-1, 3, R-3, ... coprime with R, each once
    for (int m = 1; m < R && c->nstrides < kMaxRanks; ++m) {
        for (int cand : {m, R - m}) {
            int a = cand, b = R;
            while (b) {
                const int t = a % b;
                a = b;
                b = t;
            }
            bool seen = false;
            for (int i = 0; i < c->nstrides; ++i)
                seen |= (c->strides[i] == cand);
            if (a == 1 && !seen)
                c->strides[c->nstrides++] = cand;
        }
    }
    c->channels = std::min<int64_t>(std::max<int64_t>(1, env_int("AR_CHANNELS", 1)), c->nstrides);
    // workspace: control block | hand-off accumulators [cap] (A) | tree LL up
    // | down | tree epochs | pipelined flags | ring-LL lines
    const size_t cap1 = count ? count : 1;
    c->tree_lines = std::min<uint64_t>((cap1 + 1) / 2, kTreeLinesCap);
    size_t off = kAlign;  // control block
    c->off_part = off;
    // one accumulator per element (the step and pipelined forms), which also
    // holds one staging slot per wave tile of the fused form: a tile of
    // kWaveTileSlots 16-byte slots of T stages 4 bytes per element, and the
    // tiles of one call number at most cap / (slot elements) + R
    c->part_bytes = align_up(cap1 * 4 + (size_t)R * kWaveTileSlots * 32, kAlign);
    off = align_up(off + c->part_bytes, kAlign);
    c->off_up = off;
    off = align_up(off + 2 * (size_t)R * c->tree_lines * 8, kAlign);
    c->off_down = off;
    off = align_up(off + 2 * (size_t)R * c->tree_lines * 8, kAlign);
    c->off_tree_epochs = off;
    c->tree_groups = (c->tree_lines + kTreeGroup - 1) / kTreeGroup;
    off = align_up(off + 2 * (size_t)c->tree_groups * 4, kAlign);
    c->off_flags = off;
    // one flag per (segment, chunk); a chunk is at least one workgroup pass
    // of the scalar path (kBlock * kUnroll elements)
    c->flag_stride = ((cap1 + R - 1) / R + (size_t)kBlock * kUnroll - 1) / ((size_t)kBlock * kUnroll) + 1;
    off = align_up(off + (size_t)R * c->flag_stride * 8, kAlign);
    // ring-LL: one line per (sender, segment, offset within a launch's piece);
    // pieces keep the region near 16 MiB whatever R
    c->off_rll = off;
    c->rll_cap = std::min<uint64_t>((cap1 + R - 1) / R,
                                    std::max<uint64_t>(64, (uint64_t)(1u << 21) / ((uint64_t)R * R)));
    off = align_up(off + (size_t)R * R * c->rll_cap * 8, kAlign);
    c->ws_need = off;
    *out = c;
    return AR_SUCCESS;
}

int ar_destroy(ar_comm_t c)
{
    delete c;
    return AR_SUCCESS;
}

size_t ar_workspace_bytes(ar_comm_t c) { return c ? c->ws_need : 0; }

int ar_set_workspace(ar_comm_t c, void* dev, size_t bytes, void* stream)
{
    if (!c || !dev || bytes < c->ws_need || ((uintptr_t)dev % kAlign) != 0)
        return AR_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->ws = static_cast<char*>(dev);
    c->ws_bytes = bytes;
    // clear the control block, every LL line and the tree epochs (flags start
    // at 1, so a cleared line never matches)
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(c->ws), 0u, kCtrlWords, st);
    if (e == hipSuccess)
        e = launch_fill_u64(reinterpret_cast<uint64_t*>(c->ws + c->off_up), 0ull,
                            (c->ws_need - c->off_up) / sizeof(uint64_t), st);
    if (e != hipSuccess) {
        c->ws = nullptr;
        return fail_hip(c, e);
    }
    c->ll_launches = 0;
    c->last_stream = st;
    return AR_SUCCESS;
}

int ar_allreduce(ar_comm_t c, const void* send, void* recv, size_t count, void* stream)
{
    if (c && count > c->cap)  // sizes first: checked without a device
        return AR_ERR_INVALID_ARG;
    bool noop = false;
    int rc = common_checks(c, send, recv, count, &noop);
    if (rc || noop)
        return rc;
    const size_t bytes = (size_t)c->R * count * elem_size(c->dtype);
    // in place (send == recv) is allowed: the hand-off goes through the
    // workspace row, and every schedule reads an element of a rank's input
    // before that rank's row is written at the same position (same thread,
    // or ordered by the step hand-off); partial overlap is not
    if (send != recv && overlaps(send, bytes, recv, bytes))
        return AR_ERR_INVALID_USAGE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    if (count == 0)
        return AR_SUCCESS;
    const int algo = resolve_algo(c, count);
    if (algo == AR_TREE)
        return tree_fused_ok(c) ? run_tree_fused(c, send, recv, count, st)
                                : run_tree(c, send, recv, count, st);
    RingArgs a{};
    a.send = send;
    // A segment's running value lives in its owner's output row when the
    // accumulator is the element type (the final value lands in the same
    // place, so no extra row is written), else in the workspace row.  In
    // place, the owner's row still holds its input, read at the last hop.
    if (c->dtype != AR_BF16 && send != recv) {
        a.part = recv;
        a.part_seg = count;
    } else {
        a.part = c->ws + c->off_part;
        a.part_seg = 0;
    }
    a.out = recv;
    a.ctrl = reinterpret_cast<uint32_t*>(c->ws);
    a.N = count;
    a.S = (count + c->R - 1) / c->R;
    a.send_row = count;
    a.out_row = count;
    a.R = c->R;
    a.op = kOpAllReduce;
    a.timeout_ticks = timeout_ticks(c);
    return run_ring(c, a, st, ws_opts(c, count));
}

int ar_allreduce_noalloc(ar_comm_t c, const void* send, void* recv, size_t count, void* stream)
{
    if (!c || count > c->cap)
        return AR_ERR_INVALID_ARG;
    if (count == 0)
        return AR_SUCCESS;
    if (!send || !recv)
        return AR_ERR_INVALID_ARG;
    const size_t bytes = (size_t)c->R * count * elem_size(c->dtype);
    if (send != recv && overlaps(send, bytes, recv, bytes))
        return AR_ERR_INVALID_USAGE;
    int rc = device_ready(c);
    if (rc)
        return rc;
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    hipError_t e = noalloc_scratch(&scratch, &scratch_bytes);
    if (e != hipSuccess)
        return fail_hip(c, e);
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    RingArgs a{};
    a.send = send;
    // as ar_allreduce, with the device array in place of the workspace row
    const bool staged = c->dtype == AR_BF16 || send == recv;
    a.part = staged ? scratch : recv;
    a.part_seg = staged ? 0 : count;
    a.out = recv;
    a.ctrl = nullptr;  // the fused form has no flags, lines or error word
    a.N = count;
    a.S = (count + c->R - 1) / c->R;
    a.send_row = count;
    a.out_row = count;
    a.R = c->R;
    a.op = kOpAllReduce;
    // the vector path stages its cut-short tiles per wave (the launch takes as
    // many waves as the array holds slots); the scalar path hands off through
    // LDS and needs none of it, so every count runs
    RunOpts o;
    o.stage = scratch;
    o.stage_bytes = scratch_bytes;
    o.fused_only = true;
    return run_ring(c, a, st, o);
}

int ar_reduce_scatter(ar_comm_t c, const void* send, void* recv, size_t recvcount, void* stream)
{
    // sizes first (checked without a device), and before multiplying by R so
    // that no count wraps around
    if (c && recvcount > c->cap / (size_t)c->R)
        return AR_ERR_INVALID_ARG;
    bool noop = false;
    int rc = common_checks(c, send, recv, recvcount, &noop);
    if (rc || noop)
        return rc;
    const size_t N = recvcount * (size_t)c->R;
    const size_t es = elem_size(c->dtype);
    if (N && overlaps(send, (size_t)c->R * N * es, recv, N * es))
        return AR_ERR_INVALID_USAGE;
    if (c->algo == AR_TREE)
        return AR_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    if (N == 0)
        return AR_SUCCESS;
    RingArgs a{};
    a.send = send;
    // segment c's running value in rank c's shard row (element e at
    // recv[e], as the shards are contiguous) when A == T, else the workspace
    a.part = (c->dtype != AR_BF16) ? recv : (void*)(c->ws + c->off_part);
    a.part_seg = 0;
    a.out = recv;
    a.ctrl = reinterpret_cast<uint32_t*>(c->ws);
    a.N = N;
    a.S = recvcount;
    a.send_row = N;
    a.out_row = recvcount;
    a.R = c->R;
    a.op = kOpReduceScatter;
    a.timeout_ticks = timeout_ticks(c);
    return run_ring(c, a, st, ws_opts(c, N));
}

int ar_all_gather(ar_comm_t c, const void* send, void* recv, size_t sendcount, void* stream)
{
    if (c && sendcount > c->cap / (size_t)c->R)  // as in ar_reduce_scatter
        return AR_ERR_INVALID_ARG;
    bool noop = false;
    int rc = common_checks(c, send, recv, sendcount, &noop);
    if (rc || noop)
        return rc;
    const size_t N = sendcount * (size_t)c->R;
    const size_t es = elem_size(c->dtype);
    if (N && overlaps(send, N * es, recv, (size_t)c->R * N * es))
        return AR_ERR_INVALID_USAGE;
    if (c->algo == AR_TREE)
        return AR_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    if (N == 0)
        return AR_SUCCESS;
    RingArgs a{};
    a.send = send;
    a.part = c->ws + c->off_part;  // unused by copies; keeps the alignment check uniform
    a.out = recv;
    a.ctrl = reinterpret_cast<uint32_t*>(c->ws);
    a.N = N;
    a.S = sendcount;
    a.send_row = sendcount;
    a.out_row = N;
    a.R = c->R;
    a.op = kOpAllGather;
    a.timeout_ticks = timeout_ticks(c);
    return run_ring(c, a, st, ws_opts(c, N));
}

int ar_check(ar_comm_t c)
{
    if (!c)
        return AR_ERR_INVALID_ARG;
    if (!c->ws)
        return AR_SUCCESS;
    hipError_t e = hipStreamSynchronize(c->last_stream);
    uint32_t word = 0;
    if (e == hipSuccess)
        e = hipMemcpy(&word, c->ws + kCtrlError * sizeof(uint32_t), sizeof word,
                      hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail_hip(c, e);
    if (word == 0)
        return AR_SUCCESS;
    // A bounded wait expired.  The tree's root advances a group's epoch even
    // then, and a workgroup that started after that could have stored lines
    // with the next launch's flag: clear the LL lines and epochs too, so the
    // next calls start from clean state.
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(c->ws) + kCtrlError, 0u, 1, c->last_stream);
    if (e == hipSuccess)
        e = ll_clear(c, c->last_stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(c->last_stream);
    if (e != hipSuccess)
        return fail_hip(c, e);
    return AR_ERR_TIMEOUT;
}

int ar_set_option(ar_comm_t c, int option, int64_t v)
{
    if (!c)
        return AR_ERR_INVALID_ARG;
    switch (option) {
    case AR_OPT_CHUNK_BYTES:
        if (v < 0)
            return AR_ERR_INVALID_ARG;
        c->chunk_bytes = v;
        return AR_SUCCESS;
    case AR_OPT_LAUNCH:
        if (v < AR_LAUNCH_AUTO || v > AR_LAUNCH_PIPELINED)
            return AR_ERR_INVALID_ARG;
        c->launch = (int)v;
        return AR_SUCCESS;
    case AR_OPT_GRID:
        if (v < 0 || v > (1 << 20))
            return AR_ERR_INVALID_ARG;
        c->grid = v;
        return AR_SUCCESS;
    case AR_OPT_TIMEOUT_US:
        if (v <= 0)
            return AR_ERR_INVALID_ARG;
        c->timeout_us = v;
        return AR_SUCCESS;
    case AR_OPT_DEBUG:
        c->debug = v;
        return AR_SUCCESS;
    case AR_OPT_ALGO:
        if (v != AR_RING && v != AR_TREE && v != AR_AUTO)
            return AR_ERR_INVALID_ARG;
        c->algo = (int)v;
        return AR_SUCCESS;
    case AR_OPT_PROTO:
        if (v != AR_SIMPLE && v != AR_LL && v != AR_PROTO_AUTO)
            return AR_ERR_INVALID_ARG;
        c->proto = (int)v;
        return AR_SUCCESS;
    case AR_OPT_TREE_MAX_BYTES:
        if (v < -1)
            return AR_ERR_INVALID_ARG;
        c->tree_max_bytes = v;
        return AR_SUCCESS;
    case AR_OPT_DEBUG_MUTE_RANK:
        if (v < -1 || v >= c->R)
            return AR_ERR_INVALID_ARG;
        c->mute_rank = v;
        return AR_SUCCESS;
    case AR_OPT_REDOP:
        if (v < AR_SUM || v > AR_AVG || (v == AR_AVG && c->dtype == AR_INT32))
            return AR_ERR_INVALID_ARG;
        c->redop = v;
        return AR_SUCCESS;
    case AR_OPT_CHANNELS:
        if (v < 1 || v > c->nstrides)
            return AR_ERR_INVALID_ARG;
        c->channels = v;
        return AR_SUCCESS;
    case AR_OPT_DEBUG_LL_LAUNCHES:
        if (v < 0 || (uint64_t)v > kLLResetLaunches)
            return AR_ERR_INVALID_ARG;
        c->ll_launches = (uint64_t)v;
        return AR_SUCCESS;
    }
    return AR_ERR_INVALID_ARG;
}

int ar_get_option(ar_comm_t c, int option, int64_t* v)
{
    if (!c || !v)
        return AR_ERR_INVALID_ARG;
    switch (option) {
    case AR_OPT_CHUNK_BYTES: *v = c->chunk_bytes; return AR_SUCCESS;
    case AR_OPT_LAUNCH: *v = c->launch; return AR_SUCCESS;
    case AR_OPT_GRID: *v = c->grid; return AR_SUCCESS;
    case AR_OPT_TIMEOUT_US: *v = c->timeout_us; return AR_SUCCESS;
    case AR_OPT_DEBUG: *v = c->debug; return AR_SUCCESS;
    case AR_OPT_ALGO: *v = c->algo; return AR_SUCCESS;
    case AR_OPT_PROTO: *v = c->proto; return AR_SUCCESS;
    case AR_OPT_TREE_MAX_BYTES: *v = c->tree_max_bytes; return AR_SUCCESS;
    case AR_OPT_DEBUG_MUTE_RANK: *v = c->mute_rank; return AR_SUCCESS;
    case AR_OPT_REDOP: *v = c->redop; return AR_SUCCESS;
    case AR_OPT_CHANNELS: *v = c->channels; return AR_SUCCESS;
    case AR_OPT_DEBUG_LL_LAUNCHES: *v = (int64_t)c->ll_launches; return AR_SUCCESS;
    }
    return AR_ERR_INVALID_ARG;
}

int ar_plan(ar_comm_t c, size_t count, int* algo, int* proto, int* launch)
{
    if (!c || !algo || !proto || !launch)
        return AR_ERR_INVALID_ARG;
    *algo = resolve_algo(c, count);
    *proto = resolve_proto(c, count, *algo);
    if (*algo == AR_TREE)
        *launch = tree_fused_ok(c) ? AR_LAUNCH_FUSED : AR_LAUNCH_AUTO;
    else
        *launch = *proto == AR_LL ? AR_LAUNCH_AUTO : resolve_launch(c);
    return AR_SUCCESS;
}

int ar_set_cost(ar_comm_t c, int form, double alpha_us, double bw_gbps)
{
    // written as negations so that a NaN is refused too
    if (!c || form < 0 || form >= AR_COST_FORMS || !(alpha_us >= 0.0) || !(bw_gbps > 0.0) ||
        !(alpha_us < 1e9) || !(bw_gbps < 1e9))
        return AR_ERR_INVALID_ARG;
    c->cost[form] = CostLine{alpha_us, bw_gbps};
    return AR_SUCCESS;
}

int ar_get_cost(ar_comm_t c, int form, double* alpha_us, double* bw_gbps)
{
    if (!c || form < 0 || form >= AR_COST_FORMS || !alpha_us || !bw_gbps)
        return AR_ERR_INVALID_ARG;
    *alpha_us = c->cost[form].alpha_us;
    *bw_gbps = c->cost[form].bw_gbps;
    return AR_SUCCESS;
}

int64_t ar_auto_tree_max_bytes(ar_comm_t c)
{
    if (!c)
        return -1;
    if (c->tree_max_bytes >= 0)
        return c->tree_max_bytes;
    // the sizes at which the tree's line is below the ring's as calls would
    // run it: below the simple form's and, for ring + LL or AR_PROTO_AUTO
    // (the ring then costs the lower of its two lines), below ring + LL's
    const CostLine t = c->cost[tree_cost_form(c)];
    const Span simple = below(t, c->cost[simple_ring_form(c)]);
    const Span ll = below(t, c->cost[AR_COST_RING_LL]);
    const Span s = c->proto == AR_SIMPLE ? simple : c->proto == AR_LL ? ll : intersect(simple, ll);
    if (s.lo > s.hi)
        return 0;  // never by tree
    if (s.lo == 0)
        return s.hi;  // every size up to s.hi by tree (INT64_MAX: every size)
    return -2;  // only sizes from s.lo on by tree
}

int ar_ring_segment(ar_comm_t c, size_t count, int seg, size_t* lo, size_t* hi)
{
    if (!c || !lo || !hi || seg < 0 || seg >= c->R)
        return AR_ERR_INVALID_ARG;
    const size_t S = (count + c->R - 1) / c->R;
    *lo = std::min(count, (size_t)seg * S);
    *hi = std::min(count, (size_t)(seg + 1) * S);
    return AR_SUCCESS;
}

int ar_ring_channel_stride(ar_comm_t c, int k)
{
    if (!c || k < 0 || k >= c->nstrides)
        return -1;
    return c->strides[k];
}

int ar_tree_parent(ar_comm_t c, int tree, int r)
{
    if (!c || tree < 0 || tree > 1 || r < 0 || r >= c->R)
        return -2;
    return c->tt.parent[tree][r];
}

const char* ar_status_string(int s)
{
    switch (s) {
    case AR_SUCCESS: return "success";
    case AR_ERR_INVALID_ARG: return "invalid argument";
    case AR_ERR_INVALID_USAGE: return "invalid usage";
    case AR_ERR_UNSUPPORTED: return "unsupported";
    case AR_ERR_HIP: return "HIP runtime error";
    case AR_ERR_TIMEOUT: return "timeout (a bounded wait expired)";
    case AR_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

int ar_last_hip_error(ar_comm_t c) { return c ? c->last_hip : ar::g_util_hip_error; }

}  // extern "C"
