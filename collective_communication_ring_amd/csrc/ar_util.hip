// ar_util.hip -- plain streaming kernels used as measurement references:
// c = a + b over float32 (the access mix of one reduce step) and a byte
// copy (the access mix of one copy step, and a known-size kernel for
// calibrating byte counters).  Both load and store with non-temporal hints:
// nothing they touch is reused, and that is the fastest way to stream on
// gfx950 (a 512 MiB copy: ~6.1 TB/s, against ~5.6 TB/s with plain accesses).
#include <algorithm>

#include "ar_elem.h"
#include "ar_internal.h"

namespace ar {
namespace {

__global__ __launch_bounds__(kBlock) void k_stream_add(const u32x4* __restrict__ a,
                                                       const u32x4* __restrict__ b,
                                                       u32x4* __restrict__ c, uint64_t nvec)
{
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * kUnroll;
    for (uint64_t j0 = (uint64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; j0 < nvec;
         j0 += stride) {
        u32x4 x[kUnroll], y[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * kBlock;
            if (j < nvec) {
                x[u] = __builtin_nontemporal_load(a + j);
                y[u] = __builtin_nontemporal_load(b + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * kBlock;
            if (j < nvec) {
                u32x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    r[i] = __float_as_uint(__uint_as_float(x[u][i]) + __uint_as_float(y[u][i]));
                __builtin_nontemporal_store(r, c + j);
            }
        }
    }
}

__global__ void k_stream_add_tail(const float* a, const float* b, float* c, uint64_t from,
                                  uint64_t n)
{
    const uint64_t i = from + threadIdx.x;
    if (i < n)
        c[i] = a[i] + b[i];
}

__global__ __launch_bounds__(kBlock) void k_stream_copy(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, uint64_t nvec)
{
    const uint64_t stride = (uint64_t)gridDim.x * kBlock * kUnroll;
    for (uint64_t j0 = (uint64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; j0 < nvec;
         j0 += stride) {
        u32x4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * kBlock;
            if (j < nvec)
                r[u] = __builtin_nontemporal_load(src + j);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t j = j0 + (uint64_t)u * kBlock;
            if (j < nvec)
                __builtin_nontemporal_store(r[u], dst + j);
        }
    }
}

int stream_grid(uint64_t nvec)
{
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 256;
    const uint64_t per = (uint64_t)kBlock * kUnroll;
    uint64_t need = (nvec + per - 1) / per;
    const uint64_t cap = (uint64_t)ncu * 8;
    return (int)std::max<uint64_t>(1, std::min(need, cap));
}

}  // namespace
}  // namespace ar

extern "C" int ar_stream_add(const float* a, const float* b, float* c, size_t n, void* stream)
{
    using namespace ar;
    if (!a || !b || !c || ((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u)
        return n == 0 ? AR_SUCCESS : AR_ERR_INVALID_ARG;
    if (n == 0)
        return AR_SUCCESS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t nvec = n / 4;
    if (nvec)
        hipLaunchKernelGGL(k_stream_add, dim3(stream_grid(nvec)), dim3(kBlock), 0, st,
                           reinterpret_cast<const u32x4*>(a), reinterpret_cast<const u32x4*>(b),
                           reinterpret_cast<u32x4*>(c), nvec);
    if (n % 4)
        hipLaunchKernelGGL(k_stream_add_tail, dim3(1), dim3(4), 0, st, a, b, c, nvec * 4,
                           (uint64_t)n);
    return hipGetLastError() == hipSuccess ? AR_SUCCESS : AR_ERR_HIP;
}

extern "C" int ar_stream_copy(const void* src, void* dst, size_t nbytes, void* stream)
{
    using namespace ar;
    if (nbytes == 0)
        return AR_SUCCESS;
    if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst | nbytes) & 15u))
        return AR_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t nvec = nbytes / 16;
    hipLaunchKernelGGL(k_stream_copy, dim3(stream_grid(nvec)), dim3(kBlock), 0, st,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), nvec);
    return hipGetLastError() == hipSuccess ? AR_SUCCESS : AR_ERR_HIP;
}

// ---- the fused ring's row pattern without its hops -----------------------------

namespace ar {
namespace {

// `rows` rows of row_vec 16-byte vectors, copied src -> dst tile by tile in
// the fused ring's access shape: a wave takes a tile of kWaveSlots slots per
// lane at one offset, loads it from every row (non-temporal, as the ring
// loads its inputs), then stores it at the same offset of every dst row with
// plain stores (written back from L2, as the ring's outputs are).  Rows go
// in groups of 8 (loads of a group in flight together).  The host checks
// that row_vec is a whole number of tiles.
__global__ __launch_bounds__(kBlock) void k_stream_rows(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int rows,
                                                        uint64_t row_vec)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t unit = (uint64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    const uint64_t nunits = (uint64_t)gridDim.x * (kBlock / 64);
    const uint64_t ntiles = row_vec / kWaveTileSlots;
    for (uint64_t t = unit; t < ntiles; t += nunits) {
        const uint64_t base = t * kWaveTileSlots + lane;
        for (int r0 = 0; r0 < rows; r0 += 8) {
            const int nr = rows - r0 < 8 ? rows - r0 : 8;
            u32x4 v[8][kWaveSlots];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < nr)
#pragma unroll
                    for (int u = 0; u < kWaveSlots; ++u)
                        v[i][u] = __builtin_nontemporal_load(src + (uint64_t)(r0 + i) * row_vec +
                                                             base + u * 64);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < nr)
#pragma unroll
                    for (int u = 0; u < kWaveSlots; ++u)
                        dst[(uint64_t)(r0 + i) * row_vec + base + u * 64] = v[i][u];
        }
    }
}

}  // namespace
}  // namespace ar

extern "C" int ar_stream_rows(const void* src, void* dst, int rows, size_t row_bytes, void* stream)
{
    using namespace ar;
    const size_t tile = (size_t)kWaveTileSlots * 16;
    if (rows <= 0 || row_bytes == 0)
        return rows < 0 ? AR_ERR_INVALID_ARG : AR_SUCCESS;
    if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst) & 15u) || row_bytes % tile)
        return AR_ERR_INVALID_ARG;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 256;
    const uint64_t tiles = row_bytes / tile;
    const uint64_t waves = kBlock / 64;
    const uint64_t grid = std::max<uint64_t>(1, std::min<uint64_t>((tiles + waves - 1) / waves,
                                                                    2 * (uint64_t)ncu));
    hipLaunchKernelGGL(k_stream_rows, dim3((unsigned)grid), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(src),
                       reinterpret_cast<u32x4*>(dst), rows, (uint64_t)(row_bytes / 16));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        g_util_hip_error = (int)e;
    return e == hipSuccess ? AR_SUCCESS : AR_ERR_HIP;
}

// ---- LL hop-latency probe ---------------------------------------------------

namespace ar {
namespace {

// Workgroups "a" and "b" (by position in the grid) bounce one LL line: a
// writes round r into line 0 and waits for round r in line 1; b waits for
// line 0 then answers in line 1.  Idle workgroups of the grid (used only to
// place a and b on the wanted XCDs) exit at once.
__global__ void k_ll_pingpong(uint64_t* lines, uint32_t* result, int iters, int wa, int wb,
                              uint64_t timeout_ticks)
{
    const int me = blockIdx.x;
    if ((me != wa && me != wb) || threadIdx.x != 0)
        return;
    const uint64_t deadline = (uint64_t)wall_clock64() + timeout_ticks;
    uint64_t* mine = lines + (me == wa ? 0 : 16);
    const uint64_t* theirs = lines + (me == wa ? 16 : 0);
    for (uint32_t r = 1; r <= (uint32_t)iters; ++r) {
        if (me == wa)
            __hip_atomic_store(mine, ((uint64_t)r << 32) | r, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t spin = 0;; ++spin) {
            const uint64_t v = __hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(v >> 32) == r)
                break;
            if ((spin & 255u) == 255u && (uint64_t)wall_clock64() > deadline) {
                __hip_atomic_store(result, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
        if (me == wb)
            __hip_atomic_store(mine, ((uint64_t)r << 32) | r, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace
}  // namespace ar

extern "C" int ar_ll_pingpong(void* lines, uint32_t* result_dev, int iters, int xcd_apart,
                              int64_t timeout_us, void* stream)
{
    using namespace ar;
    if (!lines || !result_dev || iters < 1 || timeout_us <= 0 || ((uintptr_t)lines & 255u))
        return AR_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return AR_ERR_HIP;
    const uint64_t ticks = (uint64_t)timeout_us * (uint64_t)(khz > 0 ? khz : 100000) / 1000u;
    hipError_t e = launch_fill_u64(static_cast<uint64_t*>(lines), 0ull, 32, st);
    if (e == hipSuccess)
        e = launch_fill_u32(result_dev, 0u, 1, st);
    if (e != hipSuccess)
        return AR_ERR_HIP;
    const int wb = xcd_apart ? 1 : 8;  // round-robin dispatch: id mod 8 is the XCD
    hipLaunchKernelGGL(k_ll_pingpong, dim3(wb + 1), dim3(64), 0, st,
                       static_cast<uint64_t*>(lines), result_dev, iters, 0, wb, ticks);
    return hipGetLastError() == hipSuccess ? AR_SUCCESS : AR_ERR_HIP;
}

// ---- CU-masked streams -------------------------------------------------------

namespace ar {
thread_local int g_util_hip_error = 0;  // last HIP error of this thread's utility calls
}

extern "C" int ar_stream_create_cu_masked(void** stream, uint32_t mask_words, const uint32_t* mask)
{
    if (!stream || !mask || mask_words == 0)
        return AR_ERR_INVALID_ARG;
    *stream = nullptr;
    hipStream_t st = nullptr;
    const hipError_t e = hipExtStreamCreateWithCUMask(&st, mask_words, mask);
    if (e != hipSuccess) {
        ar::g_util_hip_error = (int)e;
        return AR_ERR_HIP;
    }
    *stream = st;
    return AR_SUCCESS;
}

extern "C" int ar_stream_destroy(void* stream)
{
    if (!stream)
        return AR_SUCCESS;
    return hipStreamDestroy(static_cast<hipStream_t>(stream)) == hipSuccess ? AR_SUCCESS : AR_ERR_HIP;
}
