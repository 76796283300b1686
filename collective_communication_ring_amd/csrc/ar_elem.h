// ar_elem.h -- element types and 16-byte vector access for the libar kernels.
//
// T is the element type of the user's buffers, A the accumulator type:
//   int32   : T = int32,  A = uint32 (wrap-around adds)
//   float32 : T = float,  A = float  (IEEE single adds, round to nearest even)
//   bfloat16: T = uint16 bit pattern, A = float; the owner rounds once to
//             nearest-even when it writes the final value.
// A "slot" is V consecutive elements: V = 16 bytes of T on the vector path
// (4 for int32/float32, 8 for bfloat16), V = 1 on the unaligned fallback.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct Elem;

template <>
struct Elem<AR_INT32> {
    using T = int32_t;
    using A = uint32_t;
    static constexpr int VEC = 4;
    __device__ static A widen(T v) { return (A)v; }
    __device__ static T narrow(A a) { return (T)a; }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static A from_bits(uint32_t u) { return u; }
    __device__ static uint32_t to_bits(A a) { return a; }
    __device__ static uint32_t t_bits(T v) { return (uint32_t)v; }
    __device__ static T t_from_bits(uint32_t u) { return (T)u; }
};

template <>
struct Elem<AR_FLOAT32> {
    using T = float;
    using A = float;
    static constexpr int VEC = 4;
    __device__ static A widen(T v) { return v; }
    __device__ static T narrow(A a) { return a; }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static A from_bits(uint32_t u) { return __uint_as_float(u); }
    __device__ static uint32_t to_bits(A a) { return __float_as_uint(a); }
    __device__ static uint32_t t_bits(T v) { return __float_as_uint(v); }
    __device__ static T t_from_bits(uint32_t u) { return __uint_as_float(u); }
};

template <>
struct Elem<AR_BF16> {
    using T = uint16_t;
    using A = float;
    static constexpr int VEC = 8;
    __device__ static A widen(T v) { return __uint_as_float((uint32_t)v << 16); }
    // Round to nearest, ties to even: adding 0x7fff plus the lowest kept bit
    // carries into the kept half exactly when the dropped half is above one
    // half, or equal to one half with an odd kept half.  NaN stays quiet NaN.
    __device__ static T narrow(A a)
    {
        uint32_t u = __float_as_uint(a);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            return (T)((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (T)(u >> 16);
    }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static A from_bits(uint32_t u) { return __uint_as_float(u); }
    __device__ static uint32_t to_bits(A a) { return __float_as_uint(a); }
    __device__ static uint32_t t_bits(T v) { return (uint32_t)v; }
    __device__ static T t_from_bits(uint32_t u) { return (T)(u & 0xffffu); }
};

// ---- reduction operators ------------------------------------------------

// One step of the fold, a = running value, b = next value.  Sum and average
// add; max / min keep a only when it is strictly larger / smaller.  The
// integer compare is signed (the accumulator holds int32 bits).
template <class E, int RED>
__device__ inline typename E::A combine(typename E::A a, typename E::A b)
{
    if constexpr (RED == AR_MAX || RED == AR_MIN) {
        bool a_wins;
        if constexpr (sizeof(typename E::T) == 4 && !__is_same(typename E::A, float))
            a_wins = RED == AR_MAX ? (int32_t)a > (int32_t)b : (int32_t)a < (int32_t)b;
        else
            a_wins = RED == AR_MAX ? a > b : a < b;
        return a_wins ? a : b;
    } else {
        return E::add(a, b);
    }
}

// The value the owner (or the tree's root) keeps: an average divides the
// sum by R once (IEEE division, correctly rounded).
template <class E, int RED>
__device__ inline typename E::A finalize(typename E::A a, float R)
{
    if constexpr (RED == AR_AVG)
        return a / R;
    else
        return a;
}

// ---- slot loads and stores ----------------------------------------------

// 16-byte load of user input (a T row of send).  Every input element is read
// exactly once per collective, so the load is marked non-temporal: it should
// not displace the partial sums that the next step re-reads from L2.
__device__ inline u32x4 load16(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The V accumulator values of a 16-byte slot of T held as raw bits.
template <class E, int V>
__device__ inline void widen_slot(const u32x4& r, typename E::A (&o)[V])
{
    if constexpr (sizeof(typename E::T) == 4) {
        static_assert(V == 4, "16-byte slot of 32-bit elements");
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = E::from_bits(r[i]);
    } else {
        static_assert(V == 8, "16-byte slot of 16-bit elements");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = E::widen((typename E::T)(r[i] & 0xffffu));
            o[2 * i + 1] = E::widen((typename E::T)(r[i] >> 16));
        }
    }
}

template <class E, int V>
__device__ inline void load_t(const typename E::T* p, typename E::A (&o)[V])
{
    if constexpr (V == 1)
        o[0] = E::widen(p[0]);
    else
        widen_slot<E, V>(load16(p), o);
}

template <class E, int V>
__device__ inline void store_t(typename E::T* p, const typename E::A (&v)[V])
{
    if constexpr (V == 1) {
        p[0] = E::narrow(v[0]);
    } else if constexpr (sizeof(typename E::T) == 4) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = E::to_bits(v[i]);
        *reinterpret_cast<u32x4*>(p) = r;
    } else {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = (uint32_t)E::narrow(v[2 * i]) | ((uint32_t)E::narrow(v[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4*>(p) = r;
    }
}

// Accumulator slots are V * 4 bytes: one 16-byte access for V = 4, two for
// V = 8.
template <class E, int V>
__device__ inline void load_a(const typename E::A* p, typename E::A (&o)[V])
{
    if constexpr (V == 1) {
        o[0] = p[0];
    } else {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            u32x4 r = reinterpret_cast<const u32x4*>(p)[h];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[4 * h + i] = E::from_bits(r[i]);
        }
    }
}

template <class E, int V>
__device__ inline void store_a(typename E::A* p, const typename E::A (&v)[V])
{
    if constexpr (V == 1) {
        p[0] = v[0];
    } else {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = E::to_bits(v[4 * h + i]);
            reinterpret_cast<u32x4*>(p)[h] = r;
        }
    }
}

// Keeps the compiler from carrying a value stored by one ring step into the
// next step's load of the same address: every step must read the buffer of
// the rank it receives from.  Emits no instruction.
__device__ inline void step_boundary() { __asm__ __volatile__("" ::: "memory"); }

__device__ inline int mod_r(int a, int R) { return ((a % R) + R) % R; }

__device__ inline uint64_t seg_lo(uint64_t N, uint64_t S, int c)
{
    uint64_t b = (uint64_t)c * S;
    return b < N ? b : N;
}

// The part of segment c a channel covers: [c*S + sub_lo, c*S + sub_lo +
// sub_len) clipped to the segment [c*S, min((c+1)*S, N)).
__device__ inline void seg_range(uint64_t N, uint64_t S, int c, uint64_t sub_lo, uint64_t sub_len,
                                 uint64_t* lo, uint64_t* hi)
{
    const uint64_t end = seg_lo(N, S, c + 1);
    const uint64_t a = seg_lo(N, S, c) + sub_lo;
    const uint64_t b = a + sub_len;
    *lo = a < end ? a : end;
    *hi = b < end ? b : end;
}

}  // namespace ar
