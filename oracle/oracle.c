/*
 * oracle.c -- plain CPU oracle for ring and double-binary-tree all-reduce
 * (sum), reduce-scatter and all-gather over R logical ranks.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference
 * the GPU library is checked against.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the product path never
 * does.  It shares no code, header, table or helper with the GPU library,
 * and includes nothing from it.
 *
 * Reduction operators: sum (the pages' worked examples), max, min, and
 * average (sum / R).
 *
 * The LL protocol changes no value (data and flag share one store; the flag
 * only tells the reader the data arrived), so the oracle has no LL format.
 *
 * Threads: built plain (one thread) and again with OpenMP, where loops over
 * the elements (or ranks) of one step run in parallel; every element is
 * still folded by one thread in the schedule's order, so both builds give
 * the same bits.
 *
 * Parity status: every function here is pinned by CPU tests (closed forms,
 * brute force, hand-computed rounding-order cases, a library conversion
 * routine, and the pages' worked examples); none is "parity unpinned".
 *
 * Buffers are rank-major: row q of R rows holds logical rank q's elements
 * contiguously.  Element types: 0 = int32, 1 = float32, 2 = bfloat16 (stored
 * as uint16 bit patterns).  The accumulator is uint32 wrap-around arithmetic
 * for int32 and IEEE float32 (round-to-nearest-even) for float32 and
 * bfloat16 inputs; a bfloat16 result is rounded once, to nearest-even, by
 * the rank that owns the element.
 *
 * What is computed, and where the pages say so:
 *  - all-reduce: every rank ends with the element-wise sum of all ranks'
 *    inputs ("NCCL, NIXL, and Distributed GPU Communication", section
 *    "All-reduce", the four-GPU g0+g1+g2+g3 example);
 *  - reduce-scatter: rank r receives shard r of that sum (same page,
 *    "Reduce-scatter"); all-gather: every rank receives [x0, x1, ..., x_{k-1}]
 *    (same page, "All-gather"); all-reduce = reduce-scatter + all-gather
 *    (same page, "Reduce-scatter");
 *  - ring: 2(N-1) steps ("GPU MODE lecture 68 notes", section 05, "SHARP --
 *    in-network reduction"), read as R-1 reduce-and-pass steps followed by
 *    R-1 copy-and-pass steps around the ring q -> q+1;
 *  - double binary tree: two complementary binary trees working at once,
 *    each on different links ("NCCL and NVSHMEM -- two GPU communication
 *    models, side by side", section "double binary tree"), read as the
 *    two-tree scheme: tree A is the in-order binary tree on ranks 0..R-1,
 *    tree B its mirror image (even R) or its shift by one (odd R), and each
 *    tree reduces and broadcasts one half of the elements.
 * Floating-point sums depend on the order of the additions, so the oracle
 * replays exactly the order the schedule implies (see each function).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads.  The oracle is built twice: plain (one thread) and with OpenMP,
 * where the loops marked below run in parallel over elements (or ranks)
 * *within* one step.  Every element is still folded by one thread in the
 * schedule's order, so both builds give the same bits. */
int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

enum { ORC_INT32 = 0, ORC_FLOAT32 = 1, ORC_BF16 = 2 };
/* Reduction operators: sum, max, min, and average = sum / R ("NCCL, NIXL,
 * and Distributed GPU Communication", section "All-reduce": ranks reduce with
 * sum/min/max; DDP divides the sum by the world size to average). */
enum { ORC_SUM = 0, ORC_MAX = 1, ORC_MIN = 2, ORC_AVG = 3 };
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ENOMEM = 2 };

/* One accumulator value: uint32 for int32 inputs, float for the others. */
typedef union {
    uint32_t u;
    float f;
} acc_t;

static int mod(int a, int m) { return ((a % m) + m) % m; }

static int elem_size(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

/* ---- bfloat16 -------------------------------------------------------- */

/* float32 -> bfloat16, round to nearest, ties to even.  The top 16 bits are
 * kept; the dropped low 16 bits decide: above half round up, below half
 * round down, exactly half round to the even neighbour.  A carry out of the
 * mantissa moves into the exponent, which is the correct result (and yields
 * infinity above the largest finite bfloat16).  NaN stays NaN (quiet). */
uint16_t orc_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u) != 0u))
        hi += 1u;
    return (uint16_t)hi;
}

/* bfloat16 -> float32 is exact: the 16 bits become the top half. */
float orc_f32_from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void orc_bf16_from_f32_array(const float* in, uint16_t* out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_f32(in[i]);
}

/* ---- element access -------------------------------------------------- */

/* Widen element i of a T-typed buffer into the accumulator type. */
static acc_t widen(int dtype, const void* buf, size_t i)
{
    acc_t a;
    if (dtype == ORC_INT32) {
        int32_t v;
        memcpy(&v, (const char*)buf + 4 * i, 4);
        a.u = (uint32_t)v;
    } else if (dtype == ORC_FLOAT32) {
        memcpy(&a.f, (const char*)buf + 4 * i, 4);
    } else {
        uint16_t h;
        memcpy(&h, (const char*)buf + 2 * i, 2);
        a.f = orc_f32_from_bf16(h);
    }
    return a;
}

/* Narrow an accumulator into element i of a T-typed buffer. */
static void narrow(int dtype, void* buf, size_t i, acc_t a)
{
    if (dtype == ORC_INT32) {
        int32_t v = (int32_t)a.u;
        memcpy((char*)buf + 4 * i, &v, 4);
    } else if (dtype == ORC_FLOAT32) {
        memcpy((char*)buf + 4 * i, &a.f, 4);
    } else {
        uint16_t h = orc_bf16_from_f32(a.f);
        memcpy((char*)buf + 2 * i, &h, 2);
    }
}

/* One addition in the accumulator type: int32 wraps modulo 2^32, floats are
 * IEEE single additions (this file is built without fast-math or FMA
 * contraction, so the compiler may not reassociate or fuse them). */
static acc_t acc_add(int dtype, acc_t a, acc_t b)
{
    acc_t r;
    if (dtype == ORC_INT32)
        r.u = a.u + b.u;
    else
        r.f = a.f + b.f;
    return r;
}

/* One step of the fold: a is what has been accumulated so far, b the next
 * value.  max / min keep a when it is strictly larger / smaller, else take b
 * (so with equal values, e.g. -0 and +0, or a NaN, the newer value wins);
 * sum and average add. */
static acc_t acc_op(int dtype, int op, acc_t a, acc_t b)
{
    if (op == ORC_MAX || op == ORC_MIN) {
        int a_wins;
        if (dtype == ORC_INT32)
            a_wins = op == ORC_MAX ? (int32_t)a.u > (int32_t)b.u : (int32_t)a.u < (int32_t)b.u;
        else
            a_wins = op == ORC_MAX ? a.f > b.f : a.f < b.f;
        return a_wins ? a : b;
    }
    return acc_add(dtype, a, b);
}

/* What the owner does with the fully reduced value before narrowing it:
 * average divides the sum by R once, in float32 (IEEE division). */
static acc_t acc_final(int op, int R, acc_t a)
{
    if (op == ORC_AVG)
        a.f = a.f / (float)R;
    return a;
}

/* ---- ring ------------------------------------------------------------ */

/* Segment c of a rank's N elements: [min(c*S, N), min((c+1)*S, N)) with
 * S = ceil(N/R).  Rank c owns segment c, matching "rank r receives shard r"
 * of reduce-scatter.  Trailing segments may be shorter or empty. */
static size_t seg_lo(size_t N, int R, int c)
{
    size_t S = (N + (size_t)R - 1) / (size_t)R;
    size_t b = (size_t)c * S;
    return b < N ? b : N;
}
static size_t seg_hi(size_t N, int R, int c) { return seg_lo(N, R, c + 1); }

/* Multi-channel rings (reading of the ring plus "channels = rails", "GPU
 * MODE lecture 68 notes" section 06, multi-rail aggregation: one channel per
 * rail).  With K channels every segment is cut into K sub-ranges of
 * Sk = ceil(ceil(S/K)/8)*8 elements; channel k covers sub-range k of every
 * segment, [c*S + k*Sk, c*S + (k+1)*Sk) clipped to the segment, and runs its
 * own ring q -> q + m_k (mod R) with a stride m_k coprime with R.  Rank c
 * still owns segment c.  K = 1, m = 1 is the plain ring. */
static void sub_range(size_t N, int R, int c, size_t Sk, int k, size_t* lo, size_t* hi)
{
    size_t a = seg_lo(N, R, c), b = seg_hi(N, R, c);
    size_t x = a + (size_t)k * Sk, y = x + Sk;
    *lo = x < b ? x : b;
    *hi = y < b ? y : b;
}

/* Ring reduce phase of one channel, replayed step by step.  At step s
 * (0..R-2) every rank q works on segment c = (q - (s+2)m) mod R: it combines
 * the partial its predecessor q-m holds for that segment (at step 0 the
 * predecessor's own input) with its own input.  Before the last step the
 * result is the partial rank q holds; at the last step q == c, the owner,
 * and the result is final.  The owner's final value is written by `emit`.
 * So for e in segment c the fold runs x_{c+m}, x_{c+2m}, ..., x_c. */
typedef void (*emit_fn)(void* ctx, int q, size_t e, acc_t v);

static int ring_reduce_phase(int R, size_t N, int dtype, int op, int m, size_t Sk, int k,
                             const void* send, emit_fn emit, void* ctx)
{
    acc_t* part = NULL; /* part[q*N + e]: the partial rank q holds */
    if (R > 2) {
        part = (acc_t*)malloc(sizeof(acc_t) * (size_t)R * (N ? N : 1));
        if (!part)
            return ORC_ENOMEM;
    }
    for (int s = 0; s <= R - 2; ++s) {
        for (int q = 0; q < R; ++q) {
            int c = mod(q - (s + 2) * m, R);
            int p = mod(q - m, R);
            size_t lo, hi;
            sub_range(N, R, c, Sk, k, &lo, &hi);
#pragma omp parallel for schedule(static)
            for (size_t e = lo; e < hi; ++e) {
                acc_t in = (s == 0) ? widen(dtype, send, (size_t)p * N + e)
                                    : part[(size_t)p * N + e];
                acc_t v = acc_op(dtype, op, in, widen(dtype, send, (size_t)q * N + e));
                if (s < R - 2)
                    part[(size_t)q * N + e] = v;
                else
                    emit(ctx, q, e, acc_final(op, R, v)); /* here q == c */
            }
        }
    }
    free(part);
    return ORC_OK;
}

/* Ring copy phase of one channel: at step s (0..R-2) every rank q copies
 * segment c = (q - (1+s)m) mod R from its predecessor q-m's output into its
 * own.  Rows of y are `row` elements long; segment c of the logical
 * N-element vector sits at the same offset in every row. */
static void ring_gather_phase(int R, size_t N, int dtype, int m, size_t Sk, int k, void* y,
                              size_t row)
{
    int es = elem_size(dtype);
    for (int s = 0; s <= R - 2; ++s) {
        /* within a step rank q writes only its own row, segment c */
#pragma omp parallel for schedule(static)
        for (int q = 0; q < R; ++q) {
            int c = mod(q - (1 + s) * m, R);
            int p = mod(q - m, R);
            size_t lo, hi;
            sub_range(N, R, c, Sk, k, &lo, &hi);
            memcpy((char*)y + ((size_t)q * row + lo) * es,
                   (const char*)y + ((size_t)p * row + lo) * es, (hi - lo) * es);
        }
    }
}

static size_t channel_len(size_t N, int R, int K)
{
    size_t S = (N + (size_t)R - 1) / (size_t)R;
    size_t Sk = (S + (size_t)K - 1) / (size_t)K;
    return (Sk + 7) / 8 * 8;
}

static int check_strides(int R, int K, const int* m)
{
    if (K < 1 || !m)
        return ORC_EINVAL;
    for (int k = 0; k < K; ++k) {
        int a = mod(m[k], R), b = R;
        if (a == 0)
            return ORC_EINVAL;
        while (b) { /* gcd(m, R) must be 1: the ring visits every rank */
            int t = a % b;
            a = b;
            b = t;
        }
        if (a != 1)
            return ORC_EINVAL;
    }
    return ORC_OK;
}

struct emit_ctx {
    int dtype;
    void* out;
    size_t row; /* elements per output row */
    int R;
    size_t N;
};

static void emit_full(void* vctx, int q, size_t e, acc_t v)
{
    struct emit_ctx* x = (struct emit_ctx*)vctx;
    narrow(x->dtype, x->out, (size_t)q * x->row + e, v);
}

static void emit_shard(void* vctx, int q, size_t e, acc_t v)
{
    struct emit_ctx* x = (struct emit_ctx*)vctx;
    narrow(x->dtype, x->out, (size_t)q * x->row + (e - seg_lo(x->N, x->R, q)), v);
}

static int check_args(int R, int dtype, const void* a, const void* b)
{
    if (R < 2 || R > 4096 || dtype < 0 || dtype > 2 || !a || !b)
        return ORC_EINVAL;
    return ORC_OK;
}

static int check_op(int dtype, int op)
{
    if (op < ORC_SUM || op > ORC_AVG)
        return ORC_EINVAL;
    if (op == ORC_AVG && dtype == ORC_INT32)
        return ORC_EINVAL; /* no integer average */
    return ORC_OK;
}

/* All-reduce by ring with K channels (strides m[0..K-1]): per channel, the
 * reduce phase (the owner writes its final sub-segment into its own output
 * row), then the copy phase spreads every sub-segment round that channel's
 * ring.  send and recv are [R][N]. */
int orc_ring_allreduce_ch(int R, size_t N, int dtype, int op, int K, const int* m,
                          const void* send, void* recv)
{
    int rc = check_args(R, dtype, send, recv);
    if (rc || (rc = check_op(dtype, op)) || (rc = check_strides(R, K, m)))
        return rc;
    size_t Sk = channel_len(N, R, K);
    struct emit_ctx ctx = {dtype, recv, N, R, N};
    for (int k = 0; k < K; ++k) {
        rc = ring_reduce_phase(R, N, dtype, op, m[k], Sk, k, send, emit_full, &ctx);
        if (rc)
            return rc;
        ring_gather_phase(R, N, dtype, m[k], Sk, k, recv, N);
    }
    return ORC_OK;
}

int orc_ring_allreduce_op(int R, size_t N, int dtype, int op, const void* send, void* recv)
{
    const int one = 1;
    return orc_ring_allreduce_ch(R, N, dtype, op, 1, &one, send, recv);
}

int orc_ring_allreduce(int R, size_t N, int dtype, const void* send, void* recv)
{
    return orc_ring_allreduce_op(R, N, dtype, ORC_SUM, send, recv);
}

/* Reduce-scatter by ring: the reduce phase only; rank q's output is its own
 * segment q, of length N/R.  send is [R][N], recv is [R][N/R]. */
int orc_ring_reduce_scatter_ch(int R, size_t N, int dtype, int op, int K, const int* m,
                               const void* send, void* recv)
{
    int rc = check_args(R, dtype, send, recv);
    if (rc || (rc = check_op(dtype, op)) || (rc = check_strides(R, K, m)))
        return rc;
    if (N % (size_t)R != 0)
        return ORC_EINVAL;
    size_t Sk = channel_len(N, R, K);
    struct emit_ctx ctx = {dtype, recv, N / (size_t)R, R, N};
    for (int k = 0; k < K; ++k)
        if ((rc = ring_reduce_phase(R, N, dtype, op, m[k], Sk, k, send, emit_shard, &ctx)))
            return rc;
    return ORC_OK;
}

int orc_ring_reduce_scatter_op(int R, size_t N, int dtype, int op, const void* send, void* recv)
{
    const int one = 1;
    return orc_ring_reduce_scatter_ch(R, N, dtype, op, 1, &one, send, recv);
}

int orc_ring_reduce_scatter(int R, size_t N, int dtype, const void* send, void* recv)
{
    return orc_ring_reduce_scatter_op(R, N, dtype, ORC_SUM, send, recv);
}

/* All-gather by ring: rank q first places its own shard at position q of its
 * output, then each channel's copy phase runs.  send is [R][n], recv is
 * [R][R*n]. */
int orc_ring_all_gather_ch(int R, size_t n, int dtype, int K, const int* m, const void* send,
                           void* recv)
{
    int rc = check_args(R, dtype, send, recv);
    if (rc || (rc = check_strides(R, K, m)))
        return rc;
    int es = elem_size(dtype);
    size_t N = n * (size_t)R;
    for (int q = 0; q < R; ++q)
        memcpy((char*)recv + ((size_t)q * N + (size_t)q * n) * es,
               (const char*)send + (size_t)q * n * es, n * es);
    size_t Sk = channel_len(N, R, K);
    for (int k = 0; k < K; ++k)
        ring_gather_phase(R, N, dtype, m[k], Sk, k, recv, N);
    return ORC_OK;
}

int orc_ring_all_gather(int R, size_t n, int dtype, const void* send, void* recv)
{
    const int one = 1;
    return orc_ring_all_gather_ch(R, n, dtype, 1, &one, send, recv);
}

/* ---- double binary tree ---------------------------------------------- */

/* Tree A: the in-order binary tree on 0..R-1 rooted at 0.  For r >= 1 with
 * lowest set bit b, r's parent is r-b when bit 2b of r is set, else r+b when
 * that is a rank, else r-b.  Rank 0's only child is the largest power of two
 * below R; odd ranks are leaves. */
static int tree_a_parent(int R, int r)
{
    if (r == 0)
        return -1;
    int b = r & -r;
    if (r & (2 * b))
        return r - b;
    if (r + b < R)
        return r + b;
    return r - b;
}

/* Parent of rank r in tree 0 (A) or tree 1 (B); -1 for the root.  Tree B is
 * tree A relabelled by r -> R-1-r (even R) or r -> (r+1) mod R (odd R). */
int orc_tree_parent(int R, int tree, int r)
{
    if (R < 2 || r < 0 || r >= R || tree < 0 || tree > 1)
        return -2;
    if (tree == 0)
        return tree_a_parent(R, r);
    if (R % 2 == 0) {
        int p = tree_a_parent(R, R - 1 - r);
        return p < 0 ? -1 : R - 1 - p;
    }
    int p = tree_a_parent(R, mod(r - 1, R));
    return p < 0 ? -1 : mod(p + 1, R);
}

/* Subtree reduction of v for element e: own input first, then each child's
 * subtree value in ascending rank order. */
static acc_t tree_fold(int R, const int* parent, int dtype, int op, const void* send,
                       size_t N, int v, size_t e)
{
    acc_t p = widen(dtype, send, (size_t)v * N + e);
    for (int ch = 0; ch < R; ++ch)
        if (parent[ch] == v)
            p = acc_op(dtype, op, p, tree_fold(R, parent, dtype, op, send, N, ch, e));
    return p;
}

/* All-reduce by double binary tree: elements [0, H) go up tree A and back
 * down, elements [H, N) go through tree B, H = ceil(N/2).  Every rank's
 * output is the root's sum narrowed to T (the broadcast down is a copy). */
int orc_tree_allreduce_op(int R, size_t N, int dtype, int op, const void* send, void* recv)
{
    int rc = check_args(R, dtype, send, recv);
    if (rc || (rc = check_op(dtype, op)))
        return rc;
    int* parent = (int*)malloc(sizeof(int) * 2 * (size_t)R);
    if (!parent)
        return ORC_ENOMEM;
    int root[2] = {-1, -1};
    for (int t = 0; t < 2; ++t)
        for (int r = 0; r < R; ++r) {
            parent[t * R + r] = orc_tree_parent(R, t, r);
            if (parent[t * R + r] == -1)
                root[t] = r;
        }
    size_t H = (N + 1) / 2;
#pragma omp parallel for schedule(static)
    for (size_t e = 0; e < N; ++e) {
        int t = e < H ? 0 : 1;
        acc_t v = acc_final(op, R, tree_fold(R, parent + t * R, dtype, op, send, N, root[t], e));
        for (int q = 0; q < R; ++q)
            narrow(dtype, recv, (size_t)q * N + e, v);
    }
    free(parent);
    return ORC_OK;
}

int orc_tree_allreduce(int R, size_t N, int dtype, const void* send, void* recv)
{
    return orc_tree_allreduce_op(R, N, dtype, ORC_SUM, send, recv);
}

/* ---- plain definition, in double ------------------------------------- */

/* out[e] = sum over ranks of x_r[e], added in float64 in rank order.  For
 * R <= 4096 float32 inputs this is the exact sum to far better than the
 * 1e-6 relative tolerance it is used with (and exact for int32). */
int orc_exact_sum(int R, size_t N, int dtype, const void* send, double* out)
{
    int rc = check_args(R, dtype, send, out);
    if (rc)
        return rc;
#pragma omp parallel for schedule(static)
    for (size_t e = 0; e < N; ++e) {
        double s = 0.0;
        for (int r = 0; r < R; ++r) {
            acc_t a = widen(dtype, send, (size_t)r * N + e);
            s += dtype == ORC_INT32 ? (double)(int32_t)a.u : (double)a.f;
        }
        out[e] = s;
    }
    return ORC_OK;
}
