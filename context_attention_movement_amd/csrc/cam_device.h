// cam_device.h -- device-side helpers for the gfx950 kernels: access-width
// vector types, run-time invariant division, payload conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cam_internal.h"

namespace cam {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Register type of one W-byte access.
template <int W> struct VecOf;
template <> struct VecOf<16> { typedef u32x4 type; };
template <> struct VecOf<8> { typedef u32x2 type; };
template <> struct VecOf<4> { typedef uint32_t type; };
template <> struct VecOf<2> { typedef uint16_t type; };

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    return uint32_t((uint64_t(__umulhi(n, f.m)) + n) >> f.l);
}

// ---------------------------------------------------------------------------
// Packed-THD piece arithmetic.  Sequence i of length L is cut into P pieces,
// piece p = positions [floor(p*L/P), floor((p+1)*L/P)).
// ---------------------------------------------------------------------------

// floor(p*L/P): one multiply-high while p*L fits 32 bits (L < 2^26 at P <= 64),
// a 64-bit division beyond.
__device__ __forceinline__ uint32_t piece_start(uint32_t p, uint32_t L, const FastDiv& divP)
{
    const uint64_t n = uint64_t(p) * L;
    if (n <= 0xFFFFFFFFull)
        return fdiv(uint32_t(n), divP);
    return uint32_t(n / divP.d);
}

// The rank whose piece holds position k (0 <= k < L): the largest p with
// piece_start(p) <= k, i.e. floor(((k+1)*P - 1)/L).  An fp32 estimate of that
// quotient is within one of it; two exact integer checks settle it.
__device__ __forceinline__ uint32_t piece_owner(uint32_t k, uint32_t L, const FastDiv& divP)
{
    const uint32_t P = divP.d;
    const float est = (float(k) * float(P) + float(P - 1)) / float(L);
    uint32_t p = est <= 0.0f ? 0u : uint32_t(est);
    if (p > P - 1)
        p = P - 1;
    if (p + 1 < P && piece_start(p + 1, L, divP) <= k)
        ++p;
    if (p > 0 && piece_start(p, L, divP) > k)
        --p;
    return p;
}

// Largest i < nseq with cu[i] <= t (cu non-decreasing, cu[0] = 0).
__device__ __forceinline__ int32_t seq_of_token(const int32_t* cu, int32_t nseq, uint32_t t)
{
    int32_t lo = 0, hi = nseq;
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (int64_t(cu[mid]) <= int64_t(t))
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// The same search done by a whole wave for one token (every lane passes the
// same t, all 64 lanes active): each step the lanes probe 64 evenly spaced
// entries of the bracket and a ballot keeps the last one at or before t, so a
// table in global memory costs ceil(log64 n) dependent loads, not log2 n.
__device__ __forceinline__ int32_t wave_seq_of_token(const int32_t* cu, int32_t nseq, uint32_t t)
{
    const int64_t lane = int64_t(threadIdx.x & 63u);
    int64_t lo = 0, hi = nseq;
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + 63) >> 6;
        const int64_t i = lo + lane * step;
        const bool le = i < hi && int64_t(cu[i]) <= int64_t(t);
        const uint64_t m = __ballot(le);
        if (!m)  // cu[lo] > t: a malformed table; stay in range
            break;
        lo += int64_t(63 - __builtin_clzll(m)) * step;
        hi = hi < lo + step ? hi : lo + step;
    }
    return int32_t(lo);
}

// The search for a token known to lie in sequence b or later (cu[b] <= t):
// gallop forward from b, then bisect -- one load when t is in sequence b,
// which is the common case for the consecutive tokens of a tile.
__device__ __forceinline__ int32_t seq_of_token_from(const int32_t* cu, int32_t nseq, int32_t b, uint32_t t)
{
    int64_t lo = b, span = 1;
    while (lo + span < nseq && int64_t(cu[lo + span]) <= int64_t(t)) {
        lo += span;
        span <<= 1;
    }
    int64_t hi = lo + span < nseq ? lo + span : nseq;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (int64_t(cu[mid]) <= int64_t(t))
            lo = mid;
        else
            hi = mid;
    }
    return int32_t(lo);
}


// Keep a batch of independent loads together: no instruction is scheduled
// across this point, so every load above it is issued before anything below
// it may wait for one (the register-saving interleave of loads with their
// consumers would leave one request in flight per lane).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Cache policy of the streaming accesses.  Every byte these kernels move is
// touched exactly once, so each access may carry the non-temporal hint (no
// reuse expected).  Which side profits depends on the access pattern and was
// chosen per kernel by measurement; a policy is two bits: 1 = non-temporal
// loads, 2 = non-temporal stores.
template <int W, bool NT>
__device__ __forceinline__ typename VecOf<W>::type ld_at(const void* p)
{
    const typename VecOf<W>::type* q = reinterpret_cast<const typename VecOf<W>::type*>(p);
    if (NT)
        return __builtin_nontemporal_load(q);
    return *q;
}

template <int W, bool NT>
__device__ __forceinline__ void st_at(void* p, typename VecOf<W>::type v)
{
    typename VecOf<W>::type* q = reinterpret_cast<typename VecOf<W>::type*>(p);
    if (NT)
        __builtin_nontemporal_store(v, q);
    else
        *q = v;
}

template <int W, bool NT>
__device__ __forceinline__ typename VecOf<W>::type ld(const void* base, uint64_t vec_index)
{
    return ld_at<W, NT>(static_cast<const char*>(base) + vec_index * W);
}

template <int W, bool NT>
__device__ __forceinline__ void st(void* base, uint64_t vec_index, typename VecOf<W>::type v)
{
    st_at<W, NT>(static_cast<char*>(base) + vec_index * W, v);
}

// bf16 <-> fp32.  bf16 is the upper half of an fp32 word; narrowing rounds to
// nearest, ties to even, and keeps NaN a (quiet) NaN.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float fp16_lo(uint32_t w)
{
    return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFFu)));
}
__device__ __forceinline__ float fp16_hi(uint32_t w)
{
    return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
}
__device__ __forceinline__ uint32_t f32_to_fp16_bits(float f)
{
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}

// XCD-aware tile order.  Workgroup b of a grid of nb runs on XCD b % 8 (the
// dispatcher deals workgroups to the eight XCDs in turn).  xcd_first(b, nb)
// renumbers the grid so that the workgroups of one XCD take one contiguous
// range of first tiles: XCD x owns [start(x), start(x) + count(x)) with
// count(x) = nb/8 (+1 for x < nb%8).  It is a bijection of [0, nb).
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_first(uint32_t b, uint32_t nb)
{
    const uint32_t x = b % kXcds, j = b / kXcds;
    const uint32_t q = nb / kXcds, rem = nb % kXcds;
    return x * q + (x < rem ? x : rem) + j;
}

// Launch `fn` over min(n_tiles, kMaxGrid) workgroups of kThreads on `stream`;
// kernels walk their tiles with a grid stride.
template <typename Args>
inline cam_status launch(const void* fn, const Args& a, uint64_t n_tiles, void* stream,
                         const char* what, uint64_t lds_bytes = 0, uint32_t threads = kThreads)
{
    if (n_tiles == 0)
        return CAM_OK;
    const uint32_t grid = uint32_t(n_tiles < kMaxGrid ? n_tiles : kMaxGrid);
    note_launch(grid, threads, lds_bytes);
    Args copy = a;
    void* args[] = {&copy};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(threads), args, size_t(lds_bytes),
                                   reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return set_error(CAM_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return CAM_OK;
}

}  // namespace cam
