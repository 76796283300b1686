/*
 * ar.h -- C ABI of libar: ring and double-binary-tree all-reduce (sum),
 * reduce-scatter and all-gather over R logical ranks that all live in one
 * MI355X's HBM.
 *
 * Every rank's buffer is a row of one rank-major device array: rank q's
 * elements start at base + q * row_elems * elem_size.  One call covers all R
 * logical ranks (in a multi-process library each rank would make the call;
 * here the R ranks of one communicator are emulated by one process).
 *
 * Conventions shared by every entry point:
 *  - Pointers named send/recv/dev are DEVICE pointers allocated by the caller
 *    (hipMalloc or torch); the library never frees them.  `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream).
 *  - Collective calls are asynchronous on `stream`, as the NCCL host call
 *    pattern is: enqueue, then the caller synchronizes the stream ("NCCL and
 *    NVSHMEM -- two GPU communication models, side by side", the NCCL host
 *    code listing).  Argument errors are reported synchronously by the return
 *    code and nothing is enqueued.
 *  - One collective in flight per communicator: two calls on the same comm
 *    must be ordered on one stream (a team's internal resources cannot be
 *    shared by two concurrent collectives -- "Demystifying NVSHMEM ..."
 *    summary, paragraph on fence/quiet and teams), and made from one host
 *    thread at a time (a communicator's host state is not locked; different
 *    communicators may be used from different threads).  All ranks of the comm take
 *    part in every call with the same count and dtype ("NCCL, NIXL, and
 *    Distributed GPU Communication", section on communication types).
 *  - Create a communicator once and reuse it; creation is the expensive part
 *    ("NCCL, NIXL, and Distributed GPU Communication", performance checklist:
 *    never create the communicator inside the loop).
 *  - Return value: AR_SUCCESS (0) or one of the ar_status_t codes below.
 *    count == 0 is a successful no-op.
 */
#ifndef AR_H_
#define AR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ar_comm* ar_comm_t;

/* Element type of send/recv.  AR_BF16 elements are 16-bit bfloat16 bit
 * patterns; they are added in float32 and rounded once (nearest-even) by the
 * rank that owns the element. */
typedef enum { AR_INT32 = 0, AR_FLOAT32 = 1, AR_BF16 = 2 } ar_dtype_t;

/* AR_RING: 2(R-1) steps around the ring q -> q+1, R-1 reduce-and-pass steps
 * then R-1 copy-and-pass steps ("GPU MODE lecture 68 notes", section 05,
 * "SHARP -- in-network reduction": the ring takes 2(N-1) steps).
 * AR_TREE: double binary tree -- two complementary binary trees working at
 * once, each reducing and broadcasting half of the elements ("NCCL and
 * NVSHMEM -- two GPU communication models, side by side", section "double
 * binary tree").  It runs in one of two forms with the same fold order (so
 * the same bits): fused -- one launch, each thread carrying an element up
 * and down its tree through the nodes' output rows -- when the launch is
 * fused (AR_LAUNCH_AUTO is), the protocol is not AR_LL and R <= 16, 32 or 64 (a
 * bfloat16 node's float32 partial travels in two 16-bit halves); else with
 * LL lines between the nodes' workgroups.
 * AR_AUTO picks by message size: tree for small messages, ring for large ones
 * (same page: tree for small messages, ring for large, chosen
 * automatically).  The choice compares two lines of a cost model
 * (ar_set_cost): that of the tree in the form the call would run and that of
 * the ring launch form the call would use.  With the defaults (fused forms,
 * R = 8, float32) the tree takes messages up to about 3 MB per rank; a comm
 * of 17 .. 63 ranks other than 32 has only the LL tree, whose line is above
 * the fused ring's: the ring at every size.  With a form in
 * which every step is a hand-off between ranks (AR_LAUNCH_STEP,
 * AR_LAUNCH_PIPELINED, AR_LL) the LL tree takes small messages. */
typedef enum { AR_RING = 0, AR_TREE = 1, AR_AUTO = 2 } ar_algo_t;

/* AR_SIMPLE: bulk data, then a release, then a ready flag (or a kernel
 * boundary between steps).  AR_LL: data and its arrival flag packed in one
 * 8-byte store -- 4 bytes of data, 4 bytes of flag -- that the consumer polls
 * ("Demystifying NVSHMEM ..." summary, paragraph on collectives).
 * AR_PROTO_AUTO: chosen per call from the same cost model as AR_AUTO
 * (ar_set_cost): the ring runs with AR_LL where the ring + LL line is
 * strictly below the line of the comm's simple-protocol launch form at the
 * call's size, else with AR_SIMPLE; the tree takes its fused form where it
 * can (see AR_TREE), else LL lines.  With AR_AUTO the tree is then weighed
 * against that cheaper ring.  The pages
 * pick the algorithm by size ("NCCL and NVSHMEM -- two GPU communication
 * models, side by side", ring vs tree); picking the protocol by the same
 * model is this library's extension.  With the default fused ring the model
 * keeps AR_SIMPLE at every size (its line is below ring + LL's); with
 * AR_LAUNCH_PIPELINED or AR_LAUNCH_STEP mid-size messages go by ring + LL. */
typedef enum { AR_SIMPLE = 0, AR_LL = 1, AR_PROTO_AUTO = 2 } ar_proto_t;

/* Reduction operator (ar_set_option(AR_OPT_REDOP, ...)); the default is the
 * sum.  Ranks reduce with sum, min or max; an average is the sum divided by
 * the number of ranks ("NCCL, NIXL, and Distributed GPU Communication",
 * section "All-reduce").  Max/min fold like the sum, keeping the running
 * value only when it is strictly larger/smaller (with equal values -- +0 and
 * -0 -- or a NaN, the value folded later wins).  AR_AVG divides the reduced
 * sum by R once, in float32 (IEEE division), where it is final (the ring
 * segment's owner, the tree's root); not for AR_INT32. */
typedef enum { AR_SUM = 0, AR_MAX = 1, AR_MIN = 2, AR_AVG = 3 } ar_redop_t;

typedef enum {
    AR_SUCCESS = 0,
    AR_ERR_INVALID_ARG = 1,   /* R out of range, NULL pointer, count above capacity, misaligned */
    AR_ERR_INVALID_USAGE = 2, /* partly overlapping send/recv, missing workspace */
    AR_ERR_UNSUPPORTED = 3,   /* combination not provided (e.g. tree reduce-scatter) */
    AR_ERR_HIP = 4,           /* a HIP runtime call failed; see ar_last_hip_error */
    AR_ERR_TIMEOUT = 5,       /* a kernel's bounded wait expired (watchdog) */
    AR_ERR_INTERNAL = 6
} ar_status_t;

/* How the ring's steps are launched.
 * AR_LAUNCH_STEP: one kernel per ring step covering all R ranks; the kernel
 *   boundary orders the steps.
 * AR_LAUNCH_FUSED: one persistent kernel; each workgroup carries its tiles
 *   of a segment through all 2(R-1) steps in order, every reduce step reading
 *   the running value its predecessor rank stored and storing its own over
 *   it, every copy step reading the predecessor rank's output row.
 * AR_LAUNCH_PIPELINED: one persistent kernel in which each logical rank has
 *   its own workgroups; a chunk passes from rank q-1 to rank q through a
 *   per-chunk ready flag (device-scope write-through stores, then the flag;
 *   the consumer polls the flag, then reads coherently) -- the simple
 *   protocol.
 * AR_LAUNCH_AUTO: the library's choice (the default).
 * A tree call takes its fused form with AR_LAUNCH_FUSED or AR_LAUNCH_AUTO
 * (see AR_TREE), its LL form with the others.
 * The pipelined ring, the ring with AR_LL and the LL tree need every workgroup
 * of a launch resident at once (the library sizes their grids to the
 * device's occupancy, capped by AR_OPT_GRID; on a stream held to fewer CUs
 * the caller sets AR_OPT_GRID, else the waits expire: AR_ERR_TIMEOUT).  Two
 * such launches running at the same time on different streams can each hold
 * part of the device and wait for each other until their bounded waits
 * expire (AR_ERR_TIMEOUT): do not overlap them with each other.  The step
 * and fused forms (ring and tree) have no such waits. */
typedef enum {
    AR_LAUNCH_AUTO = 0,
    AR_LAUNCH_STEP = 1,
    AR_LAUNCH_FUSED = 2,
    AR_LAUNCH_PIPELINED = 3
} ar_launch_t;

/* Tunables for ar_set_option / ar_get_option. */
typedef enum {
    AR_OPT_CHUNK_BYTES = 0,   /* pipelined ring: slice ("chunk") size in bytes of T; 0 = whole
                                 segment; at most 2^28 elements are used (1 GiB of 32-bit T,
                                 512 MiB of bf16, whose float32 partials take 1 GiB); larger
                                 values are cut */
    AR_OPT_LAUNCH = 1,        /* an ar_launch_t */
    AR_OPT_GRID = 2,          /* workgroups per launch; 0 = library default.  For the
                                 pipelined ring, ring + LL and the LL tree, whose workgroups
                                 must all be resident at once, a cap: on a stream held to
                                 some CUs (ar_stream_create_cu_masked) set it to at most the
                                 workgroups those CUs hold (one per CU is always safe); it
                                 must be at least R (2R for the LL tree).  The fused ring and
                                 the fused tree take it as their grid (the fused ring caps it
                                 at the waves its staging holds); their workgroups never wait
                                 for each other */
    AR_OPT_TIMEOUT_US = 3,    /* microseconds before a kernel's bounded wait gives up */
    AR_OPT_DEBUG = 4,         /* 1: print algorithm/protocol/launch per call to stderr */
    AR_OPT_ALGO = 5,          /* an ar_algo_t, overriding the one given to ar_init */
    AR_OPT_PROTO = 6,         /* an ar_proto_t, overriding the one given to ar_init */
    AR_OPT_TREE_MAX_BYTES = 7, /* AR_AUTO: largest per-rank message (bytes) sent by tree;
                                  -1 (default) = chosen by the cost model (ar_set_cost) */
    AR_OPT_DEBUG_MUTE_RANK = 8, /* testing the watchdog only: this logical rank's workgroups
                                   skip publishing (LL lines, ready flags), so its consumers'
                                   bounded waits expire; -1 (default) = none */
    AR_OPT_REDOP = 9,           /* an ar_redop_t for ar_allreduce / ar_reduce_scatter */
    AR_OPT_CHANNELS = 10,       /* ring channels K (default 1): every segment is cut into K
                                   sub-ranges of Sk = ceil(ceil(S/K)/8)*8 elements, and
                                   channel k runs its own ring q -> q + m_k over sub-range k
                                   (strides from ar_ring_channel_stride); the multi-rail /
                                   channels idea ("GPU MODE lecture 68 notes", section 06) */
    AR_OPT_DEBUG_LL_LAUNCHES = 11 /* testing only: LL tree and ring + LL launches counted
                                   since their lines were last cleared (see
                                   ar_set_workspace) */
} ar_option_t;

/* Create a communicator for R logical ranks (2 <= R <= 64) and up to
 * `count` elements per rank for all-reduce (reduce-scatter input / all-gather
 * output rows may be up to `count` long).  Builds the ring step table and
 * the two trees on the host and sizes the workspace; allocates no device
 * memory.  `*out` receives the handle; on error it is set to NULL.
 * Mirrors ncclCommInitRank(&comm, nranks, id, rank). */
int ar_init(ar_comm_t* out, int R, size_t count, ar_dtype_t dtype, ar_algo_t algo,
            ar_proto_t proto);

/* Release the host state of a communicator.  Does not free caller memory.
 * NULL is a no-op.  No page defines this call: it is this library's own
 * boundary design (the handle's lifetime). */
int ar_destroy(ar_comm_t comm);

/* Bytes of device workspace this communicator needs (no page defines this
 * call: it is this library's own boundary design, so that the caller owns
 * every device allocation): one row of `count`
 * 4-byte accumulators for the ring's hand-off (used by bfloat16 and by an
 * in-place all-reduce; otherwise a segment's running value is handed on
 * through its owner's row of recv), LL lines for the tree and the ring-LL
 * path, per-chunk ready flags for the pipelined ring, and a small control
 * block (LL epoch, flag base, error word).  The caller allocates at least
 * this many bytes (any 256-byte aligned device allocation). */
size_t ar_workspace_bytes(ar_comm_t comm);

/* Hand the workspace to the communicator and clear its control block and
 * LL lines (enqueued on `stream`; ordered before any later call on the same
 * stream).  No page defines this call: it is this library's own boundary
 * design; the stream argument lets the clearing be ordered with the caller's
 * own work instead of synchronizing the device.  The memory stays owned by
 * the caller and must outlive every collective issued on this comm.  Returns
 * AR_ERR_INVALID_ARG when `bytes` is smaller than ar_workspace_bytes or
 * `dev` is NULL or misaligned.
 * LL flags are 32-bit epochs that grow by one per launch.  Every 2^30 tree
 * or ring + LL launches the library clears the lines and epochs again, on
 * the call's stream, before the next such launch, so a flag never wraps
 * around to a value a stale line may hold.  The library counts the launches
 * it enqueues; replays of a captured HIP graph advance the epochs without
 * it: a caller that replays a graph holding tree or ring + LL calls more
 * than 2^30 times calls ar_set_workspace again (outside the graph) before
 * that many replays. */
int ar_set_workspace(ar_comm_t comm, void* dev, size_t bytes, void* stream);

/* All-reduce (sum, or the comm's AR_OPT_REDOP).  send and recv are
 * [R][count] rank-major device arrays of the comm's dtype; they may be the
 * same array (in place) but must not otherwise overlap (AR_ERR_INVALID_USAGE).
 * recv's contents are undefined until the call completes (the ring hands
 * running values on through it).
 * On completion every row of recv holds the element-wise reduction over the
 * R rows of send ("NCCL, NIXL, and Distributed GPU Communication", section
 * "All-reduce").  Floating-point sums are added in the order the schedule
 * implies: ring -- a left fold from the owner's successor round to the owner;
 * tree -- each node's own value, then its children's subtree sums in
 * ascending rank order. */
int ar_allreduce(ar_comm_t comm, const void* send, void* recv, size_t count, void* stream);

/* All-reduce that allocates nothing, for callers that cannot allocate device
 * memory when they call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, result and summation
 * order as ar_allreduce with the ring in its fused form.  It always runs the
 * fused ring (the comm's algorithm, protocol and launch options are not
 * consulted) and needs no workspace: ar_set_workspace is not required.
 * Where ar_allreduce stages the float32 running value in the workspace
 * (bfloat16, or send == recv: for wave tiles cut short by a segment's end;
 * whole tiles and the scalar path hand off through LDS), this call uses a
 * device array of 8 MiB that the library holds on every GPU it runs on until
 * the process ends.  The
 * launch then takes at most as many waves as the array holds staging slots
 * (2,048 for bfloat16, 4,096 for 32-bit types), so every count up to the
 * comm's capacity runs, whatever the alignment of the buffers (the scalar
 * path, taken by small counts and rows not 16-byte aligned, uses none of the
 * array).  Nothing in the
 * array needs clearing (a call writes every slot before reading it).  All
 * calls on one GPU share its array: two of them in flight at once on one GPU
 * (on different streams, or from different comms) race and give wrong
 * results; order them on one stream.  Errors: as ar_allreduce, plus
 * AR_ERR_HIP when the array's address cannot be looked up. */
int ar_allreduce_noalloc(ar_comm_t comm, const void* send, void* recv, size_t count,
                         void* stream);

/* Reduce-scatter (sum, or the comm's AR_OPT_REDOP), ring only.  send is
 * [R][R*recvcount], recv is [R][recvcount], not overlapping: row q of recv
 * receives segment q of the reduction ("NCCL, NIXL, and Distributed GPU
 * Communication", section "Reduce-scatter").  The values are bit-identical to
 * the same segment of ar_allreduce's result. */
int ar_reduce_scatter(ar_comm_t comm, const void* send, void* recv, size_t recvcount,
                      void* stream);

/* All-gather, ring only.  send is [R][sendcount], recv is [R][R*sendcount]:
 * every row of recv becomes [send_0, send_1, ..., send_{R-1}] ("NCCL, NIXL,
 * and Distributed GPU Communication", section "All-gather").  A pure copy;
 * reduce-scatter followed by all-gather equals all-reduce bit for bit. */
int ar_all_gather(ar_comm_t comm, const void* send, void* recv, size_t sendcount,
                  void* stream);

/* Synchronize the comm's last stream and report its device error word:
 * AR_ERR_TIMEOUT when a bounded wait expired in an earlier call, else
 * AR_SUCCESS.  Clears the word, and on AR_ERR_TIMEOUT also clears the
 * comm's LL lines and epochs, so that later calls start from clean state.
 * After a timeout the results of every call enqueued since the previous
 * ar_check are not valid; call ar_check before relying on later ones.  No
 * page defines this call: it is this library's own boundary design (the
 * kernels' bounded waits report here). */
int ar_check(ar_comm_t comm);

/* Set / read one tunable (ar_option_t).  Unknown options or out-of-range
 * values give AR_ERR_INVALID_ARG. */
int ar_set_option(ar_comm_t comm, int option, int64_t value);
int ar_get_option(ar_comm_t comm, int option, int64_t* value);

/* Resolved algorithm, protocol and launch that a call with `count` elements
 * per rank would use (values of ar_algo_t, ar_proto_t, ar_launch_t; never
 * AR_AUTO or AR_PROTO_AUTO; the launch is AR_LAUNCH_AUTO for the LL tree
 * and for ring + LL, which have one form each; the fused tree reports
 * AR_SIMPLE and AR_LAUNCH_FUSED).  For reduce-scatter and
 * all-gather the model's size is the full row per rank (R times the shard). */
int ar_plan(ar_comm_t comm, size_t count, int* algo, int* proto, int* launch);

/* The cost model behind AR_AUTO: for each algorithm and ring launch form a
 * line T(n) = alpha_us + n / (bw_gbps * 1e3) microseconds, n = bytes per
 * rank -- the alpha-beta model ("NCCL and NVSHMEM -- two GPU communication
 * models, side by side", cost-model paragraph: alpha is the latency floor,
 * beta the reciprocal bandwidth).  AR_AUTO takes the tree where the line of
 * the tree's form (AR_COST_TREE_FUSED or AR_COST_TREE_LL) is strictly below
 * the line of the ring form the call would use.  The defaults are fits
 * measured on MI355X at R = 8, float32 (the fused tree's set so that its
 * crossing with the fused ring lies where the measured times cross, between
 * 2 and 4 MiB per rank: its time is flat to 512 KiB, which no one line
 * follows); a caller with its own measurements (other R, dtype or machine)
 * sets them here.
 * ar_set_cost: AR_ERR_INVALID_ARG for an unknown form, alpha_us < 0,
 *   bw_gbps <= 0 or a NaN.
 * ar_auto_tree_max_bytes: under the comm's current options, the largest
 *   per-rank message AR_AUTO sends by tree when it sends every message up to
 *   that size by tree and none above (0: none; INT64_MAX: every size); -2
 *   when it sends some larger messages by tree but not the smallest (lines
 *   set to cross the other way), so that no such size exists; -1 for a NULL
 *   comm. */
typedef enum {
    AR_COST_TREE_LL = 0,
    AR_COST_RING_FUSED = 1,
    AR_COST_RING_PIPELINED = 2,
    AR_COST_RING_STEP = 3,
    AR_COST_RING_LL = 4,
    AR_COST_TREE_FUSED = 5,
    AR_COST_FORMS = 6
} ar_cost_form_t;
int ar_set_cost(ar_comm_t comm, int form, double alpha_us, double bw_gbps);
int ar_get_cost(ar_comm_t comm, int form, double* alpha_us, double* bw_gbps);
int64_t ar_auto_tree_max_bytes(ar_comm_t comm);

/* Host-side views of the schedule, for checking and tooling.
 * ar_ring_segment: [*lo, *hi) element range of segment c for a count of
 *   `count` elements; rank c owns it.
 * ar_tree_parent: parent of rank r in tree 0 (A) or tree 1 (B), -1 at the
 *   root; returns -2 for invalid arguments. */
int ar_ring_segment(ar_comm_t comm, size_t count, int c, size_t* lo, size_t* hi);
int ar_tree_parent(ar_comm_t comm, int tree, int r);

/* Ring stride of channel k: the integers in [1, R) coprime with R, ordered
 * 1, R-1, 3, R-3, 5, ... (a stride and its complement are the two directions
 * of one cycle, so the rings are edge-disjoint); -1 past the last one.  The
 * number of strides bounds AR_OPT_CHANNELS. */
int ar_ring_channel_stride(ar_comm_t comm, int k);

/* Measurement utilities (not collectives).  Plain streaming kernels that set
 * the practical HBM ceiling the reduce-copy is compared with, and calibrate
 * byte counters: ar_stream_add computes c[i] = a[i] + b[i] over n float32
 * (two 16-byte loads, one 16-byte store per 4 elements -- the same access
 * mix as one reduce step); ar_stream_copy copies n bytes (n a multiple of
 * 16, pointers 16-byte aligned).  Device pointers; asynchronous on
 * `stream`; AR_ERR_INVALID_ARG for NULL or misaligned arguments. */
int ar_stream_add(const float* a, const float* b, float* c, size_t n, void* stream);
int ar_stream_copy(const void* src, void* dst, size_t nbytes, void* stream);

/* Measurement utility: the fused ring's HBM access pattern without its hops.
 * Copies `rows` rows of `row_bytes` bytes (src and dst rank-major, rows
 * contiguous) tile by tile: a wave loads a 2 KiB tile at one offset from
 * every row, then stores it at that offset of every dst row with plain
 * stores, i.e. the R input rows read and the R output rows written back from
 * L2 that one all-reduce moves.  Its rate is the ceiling of that pattern.
 * row_bytes must be a multiple of 2048 and the pointers 16-byte aligned
 * (AR_ERR_INVALID_ARG otherwise); rows == 0 or row_bytes == 0 is a no-op. */
int ar_stream_rows(const void* src, void* dst, int rows, size_t row_bytes, void* stream);

/* Stream with a CU mask (runtime utility for overlapping a collective with
 * compute, "NCCL, NIXL, and Distributed GPU Communication", performance
 * checklist: overlap communication with computation).  On one GPU the
 * collective and the compute share the CUs; giving each its own CUs keeps
 * them from queueing behind each other.  `mask` has `mask_words` 32-bit
 * words, bit i enabling CU i.  *stream receives a hipStream_t (default
 * priority).  Destroy with ar_stream_destroy. */
int ar_stream_create_cu_masked(void** stream, uint32_t mask_words, const uint32_t* mask);
int ar_stream_destroy(void* stream);

/* LL hop-latency probe (measurement utility): two workgroups pass one 8-byte
 * LL line back and forth `iters` times -- each waits for the other's line
 * with the current round number as flag, then answers.  `lines` is device
 * memory of at least 256 bytes, zeroed by the call.  `xcd_apart` != 0 puts
 * the two workgroups on different XCDs (workgroup ids 0 and 1 under the
 * round-robin dispatch), 0 on the same XCD (ids 0 and 8).  Every wait is
 * bounded by `timeout_us`; `*result_dev` (device uint32) receives 0 on
 * success, 1 on a timeout.  Time the call with events: one-way latency =
 * elapsed / (2 * iters). */
int ar_ll_pingpong(void* lines, uint32_t* result_dev, int iters, int xcd_apart,
                   int64_t timeout_us, void* stream);

/* Message for a status code (static storage).  No page defines this call:
 * it is this library's own boundary design. */
const char* ar_status_string(int status);

/* Last hipError_t seen by this comm (0 if none); with comm == NULL, the last
 * one seen by the calling thread's utility calls (ar_stream_*,
 * ar_ll_pingpong). */
int ar_last_hip_error(ar_comm_t comm);

#ifdef __cplusplus
}
#endif

#endif /* AR_H_ */
