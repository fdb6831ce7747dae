// Device helpers shared by the gfx950 kernels of libep.so (internal header).
//
// Wave64 throughout: a "wave" is 64 lanes; ballots and lane masks are 64-bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int ep_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ep_u32x2 __attribute__((ext_vector_type(2)));

#define EP_WAVE 64

namespace ep {

// Device status bits (mirror the public EP_DEV_* values).
constexpr int kDevBadExpert = 1;
constexpr int kDevCapacity = 2;
constexpr int kDevRecvOverflow = 4;

// Layout kernels: a pair's in-tile rank is packed with its expert id as
// (e << kRankBits) | rank until the slot pass replaces it.
constexpr int kRankBits = 12;
constexpr int kMaxChunksPerWave = 4;   // 64-pair chunks per wave in one tile

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_read(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float lane_read_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Lanes strictly below this one.
__device__ __forceinline__ uint64_t lanes_below() {
    const int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// bf16 <-> fp32.  Widening is exact (bf16 is the top half of binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even binary32 -> bf16 by integer rounding of the top 16
// bits: add 0x7FFF plus the lowest kept bit, truncate.  NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP e4m3fn, round to nearest even, from binary32 bits.
//  |f| >  464 (or NaN/inf): NaN code S.1111.111 (no finite neighbour);
//  |f| <  2^-6: subnormal, code = rint(|f| * 2^9) (0..8; 8 is the smallest
//               normal 0x08), exact power-of-two scaling then RNE;
//  otherwise:   drop 20 mantissa bits with RNE on the integer pattern; the
//               exponent rebias (127 -> 7) is a subtraction of 120 << 3 from
//               the top 12 bits.  A mantissa carry moves into the exponent.
__device__ __forceinline__ uint32_t e4m3_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t s = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x43E80000u) {
        code = 0x7Fu;
    } else if (a < 0x3C800000u) {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    }
    return s | code;
}

__device__ __forceinline__ float amax8(ep_u32x4 v) {
    float m = fabsf(bf16_lo(v.x));
    m = fmaxf(m, fabsf(bf16_hi(v.x)));
    m = fmaxf(m, fabsf(bf16_lo(v.y)));
    m = fmaxf(m, fabsf(bf16_hi(v.y)));
    m = fmaxf(m, fabsf(bf16_lo(v.z)));
    m = fmaxf(m, fabsf(bf16_hi(v.z)));
    m = fmaxf(m, fabsf(bf16_lo(v.w)));
    m = fmaxf(m, fabsf(bf16_hi(v.w)));
    return m;
}

// 8 bf16 values / s -> 8 e4m3 codes packed little-endian in two dwords.
__device__ __forceinline__ ep_u32x2 encode8(ep_u32x4 v, float s) {
    uint32_t c0 = e4m3_rne(bf16_lo(v.x) / s) | (e4m3_rne(bf16_hi(v.x) / s) << 8) |
                  (e4m3_rne(bf16_lo(v.y) / s) << 16) | (e4m3_rne(bf16_hi(v.y) / s) << 24);
    uint32_t c1 = e4m3_rne(bf16_lo(v.z) / s) | (e4m3_rne(bf16_hi(v.z) / s) << 8) |
                  (e4m3_rne(bf16_lo(v.w) / s) << 16) | (e4m3_rne(bf16_hi(v.w) / s) << 24);
    ep_u32x2 r;
    r.x = c0;
    r.y = c1;
    return r;
}

// max over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Smallest power of two >= s, for positive normal s: a value with mantissa
// bits set moves to the next exponent with a clear mantissa.
__device__ __forceinline__ float pow2_ceil(float s) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x7FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
    return __uint_as_float(u);
}

// UE8M0 encoding of a power of two: its biased 8-bit exponent.
__device__ __forceinline__ uint32_t ue8m0_of(float p) { return (__float_as_uint(p) >> 23) & 0xFFu; }

__device__ __forceinline__ float scale_of(float amax) {
    const float ap = amax > 1e-4f ? amax : 1e-4f;
    return ap / 448.0f;
}

#ifndef EP_USE_NT_STORE
#define EP_USE_NT_STORE 1
#endif
#ifndef EP_USE_NT_LOAD
#define EP_USE_NT_LOAD 1
#endif

// Streaming accesses: rows are touched once per call, so they are issued with
// the non-temporal hint and do not displace the routing tables in L2.
template <typename T>
__device__ __forceinline__ void store_nt(T *p, T v) {
    if (EP_USE_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <typename T>
__device__ __forceinline__ T load_nt(const T *p) {
    if (EP_USE_NT_LOAD) return __builtin_nontemporal_load(p);
    return *p;
}

}  // namespace ep
