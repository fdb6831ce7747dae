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

#ifndef EP_CAST_DIV
#define EP_CAST_DIV 1   // 1: reciprocal + two residual corrections; 0: plain '/' per element
#endif

// x / s rounded to nearest even, given y = RN(1/s) (one correctly rounded
// division per scale group).  Markstein's refinement (P. Markstein, IBM J.
// Res. Dev. 34(1), 1990): with y = RN(1/s) and q within one ulp of x/s, the
// residual r = x - s*q is exact in one FMA and RN(q + r*y) = RN(x/s).  q =
// x*y can be just over one ulp off, so one correction makes it faithful and
// a second gives the rounded quotient.  Exactness needs the residual to be a
// normal fp32 number: with s >= 1e-4/448 that holds for every |x/s| >= 2^-12,
// and every smaller quotient has e4m3 code +-0 whatever its low bits.  The
// sign is x's (s > 0), which also keeps -0.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
#if EP_CAST_DIV
    float q = x * y;
    float r = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(r, y, q);
    r = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(r, y, q);
    return __builtin_copysignf(q, x);
#else
    (void)y;
    return x / s;
#endif
}

#ifndef EP_CAST_HWCVT
#define EP_CAST_HWCVT 1   // 1: gfx950's packed fp32 -> e4m3 conversion; 0: e4m3_rne
#endif

// Four quotients -> four e4m3 codes, little-endian in one dword.  The
// hardware conversion rounds to nearest even like e4m3_rne; the quotients
// here never exceed 448 * (1 + 2^-23), so its overflow handling is not met.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
#if EP_CAST_HWCVT
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
#else
    return e4m3_rne(a) | (e4m3_rne(b) << 8) | (e4m3_rne(c) << 16) | (e4m3_rne(d) << 24);
#endif
}

// 8 bf16 values / s -> 8 e4m3 codes packed little-endian in two dwords,
// given y = RN(1/s).
__device__ __forceinline__ ep_u32x2 encode8_y(ep_u32x4 v, float s, float y) {
    ep_u32x2 r;
    r.x = pack4_e4m3(div_rn(bf16_lo(v.x), s, y), div_rn(bf16_hi(v.x), s, y),
                     div_rn(bf16_lo(v.y), s, y), div_rn(bf16_hi(v.y), s, y));
    r.y = pack4_e4m3(div_rn(bf16_lo(v.z), s, y), div_rn(bf16_hi(v.z), s, y),
                     div_rn(bf16_lo(v.w), s, y), div_rn(bf16_hi(v.w), s, y));
    return r;
}

__device__ __forceinline__ ep_u32x2 encode8(ep_u32x4 v, float s) {
    return encode8_y(v, s, 1.0f / s);
}

#ifndef EP_GROUP_MAX_DPP
#define EP_GROUP_MAX_DPP 1
#endif

// v from the lane given by a DPP control code (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max over aligned groups of `width` lanes (width a power of two <= 64).
// Up to 16 lanes (one DPP row) the exchanges are DPP moves at ALU rate:
// lane ^ 1 and lane ^ 2 by quad permutes, then the mirror inside each half
// row and inside the row, which pair every lane with one of the other
// half; wider groups go through ds_bpermute.
__device__ __forceinline__ float group_max(float v, int width) {
#if EP_GROUP_MAX_DPP
    if (width <= 16) {
        if (width >= 2) v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
        if (width >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
        if (width >= 8) v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
        if (width >= 16) v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
        return v;
    }
#endif
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
