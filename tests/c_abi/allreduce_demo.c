/* allreduce_demo.c -- uses libar through its C ABI only (include/ar.h and
 * the HIP runtime API, no Python, no PyTorch): allocates the device buffers
 * and the workspace itself, runs int32 ring and tree all-reduces, a
 * reduce-scatter and an all-gather, and checks every result against the
 * integer sum computed on the host.  Prints "ok" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ar.h"

#define R 8
#define N (R * 4096 + 40)

static int fail(const char* what, int rc)
{
    fprintf(stderr, "%s failed: %d (%s)\n", what, rc, ar_status_string(rc));
    return 1;
}

static int check_sum(const int32_t* got, const int32_t* x, size_t n, size_t row)
{
    for (size_t i = 0; i < n; ++i) {
        int64_t s = 0;
        for (int q = 0; q < R; ++q)
            s += x[(size_t)q * row + i];
        for (int q = 0; q < R; ++q)
            if (got[(size_t)q * n + i] != (int32_t)s) {
                fprintf(stderr, "mismatch at rank %d element %zu\n", q, i);
                return 1;
            }
    }
    return 0;
}

int main(void)
{
    const size_t bytes = (size_t)R * N * sizeof(int32_t);
    int32_t* x = malloc(bytes);
    int32_t* y = malloc(bytes);
    if (!x || !y)
        return 1;
    for (int q = 0; q < R; ++q)
        for (size_t i = 0; i < N; ++i)
            x[(size_t)q * N + i] = (int32_t)((q * 131 + (int64_t)i * 7) % 2001) - 1000;

    void *send, *recv, *ws;
    ar_comm_t comm;
    int rc = ar_init(&comm, R, N, AR_INT32, AR_RING, AR_SIMPLE);
    if (rc)
        return fail("ar_init", rc);
    const size_t wsb = ar_workspace_bytes(comm);
    if (hipMalloc(&send, bytes) != hipSuccess || hipMalloc(&recv, bytes) != hipSuccess ||
        hipMalloc(&ws, wsb) != hipSuccess)
        return fail("hipMalloc", -1);
    if (hipMemcpy(send, x, bytes, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy", -1);
    if ((rc = ar_set_workspace(comm, ws, wsb, NULL)))
        return fail("ar_set_workspace", rc);

    /* the ring in every launch form, then the tree with the LL protocol */
    const int launches[] = {AR_LAUNCH_FUSED, AR_LAUNCH_STEP, AR_LAUNCH_PIPELINED};
    for (int k = 0; k < 4; ++k) {
        if (k < 3) {
            rc = ar_set_option(comm, AR_OPT_LAUNCH, launches[k]);
        } else {
            rc = ar_set_option(comm, AR_OPT_ALGO, AR_TREE);
            if (!rc)
                rc = ar_set_option(comm, AR_OPT_PROTO, AR_LL);
        }
        if (rc)
            return fail("ar_set_option", rc);
        if (hipMemset(recv, 0xff, bytes) != hipSuccess)
            return fail("hipMemset", -1);
        if ((rc = ar_allreduce(comm, send, recv, N, NULL)))
            return fail("ar_allreduce", rc);
        if ((rc = ar_check(comm)))
            return fail("ar_check", rc);
        if (hipMemcpy(y, recv, bytes, hipMemcpyDeviceToHost) != hipSuccess)
            return fail("hipMemcpy", -1);
        if (check_sum(y, x, N, N))
            return fail("all-reduce result", k);
    }

    /* ring reduce-scatter of R*n elements, then all-gather of the shards */
    if ((rc = ar_set_option(comm, AR_OPT_ALGO, AR_RING)) ||
        (rc = ar_set_option(comm, AR_OPT_PROTO, AR_SIMPLE)) ||
        (rc = ar_set_option(comm, AR_OPT_LAUNCH, AR_LAUNCH_AUTO)))
        return fail("ar_set_option", rc);
    const size_t n = N / R;
    void* shard;
    if (hipMalloc(&shard, (size_t)R * n * sizeof(int32_t)) != hipSuccess)
        return fail("hipMalloc", -1);
    if ((rc = ar_reduce_scatter(comm, send, shard, n, NULL)))
        return fail("ar_reduce_scatter", rc);
    if ((rc = ar_all_gather(comm, shard, recv, n, NULL)))
        return fail("ar_all_gather", rc);
    if ((rc = ar_check(comm)))
        return fail("ar_check", rc);
    if (hipMemcpy(y, recv, (size_t)R * R * n * sizeof(int32_t), hipMemcpyDeviceToHost) !=
        hipSuccess)
        return fail("hipMemcpy", -1);
    if (check_sum(y, x, R * n, N))
        return fail("reduce-scatter + all-gather result", 0);

    ar_destroy(comm);
    hipFree(shard);
    hipFree(ws);
    hipFree(recv);
    hipFree(send);
    free(x);
    free(y);
    printf("ok\n");
    return 0;
}
