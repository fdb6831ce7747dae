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

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive scan in place over a[0..n) in LDS by one wave (each lane owns a
// contiguous run of ceil(n/64) entries); returns the total to that wave.
// The caller synchronises the block afterwards.
__device__ __forceinline__ int wave_exclusive_scan(int32_t *a, int n) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) >> 6;
    const int beg = min(n, lane * per);
    const int end = min(n, beg + per);
    int local = 0;
    for (int i = beg; i < end; ++i) local += a[i];
    int x = local;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    int excl = x - local;
    for (int i = beg; i < end; ++i) {
        const int c = a[i];
        a[i] = excl;
        excl += c;
    }
    return __shfl(x, 63);
}

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

// x / s rounded to nearest even, given y = RN(1/s) (one correctly rounded
// reciprocal per scale group).  Markstein's refinement (P. Markstein, IBM J.
// Res. Dev. 34(1), 1990): q = RN(x*y), the residual r = x - s*q is exact in
// one FMA, and RN(q + r*y) is the correctly rounded quotient when q is
// close enough.  For the cast's operands, x a bf16 value and s =
// RN(max(amax, 1e-4)/448) with amax the largest |x| of the group, one
// correction gives RN(x/s) for every pair: both significands take 128 values
// (129 for s), all pairs are checked exhaustively against IEEE division
// with exact rational arithmetic, and the steps scale with the operands'
// exponents while they stay normal.  Quotients below 2^-12, where the
// residual could leave the normal range, have e4m3 code +-0 whatever their
// low bits.  The sign is x's (s > 0), which also keeps -0.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
    float q = x * y;
    const float r = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(r, y, q);
    return __builtin_copysignf(q, x);
}

// Four quotients -> four e4m3 codes, little-endian in one dword, by gfx950's
// packed fp32 -> OCP e4m3 conversion, which rounds to nearest even (checked
// against the definition over every finite bf16 pattern under several
// scales).  The quotients never exceed 448 * (1 + 2^-23), so its overflow
// handling is not met.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// 8 bf16 values / s -> 8 e4m3 codes packed little-endian in two dwords,
// given y = RN(1/s).  EXACT: s is a power of two, so y is exact and so is
// x * y (its sign is x's, -0 included): no correction is needed.
template <bool EXACT>
__device__ __forceinline__ ep_u32x2 encode8_y(ep_u32x4 v, float s, float y) {
    auto q = [&](float x) { return EXACT ? x * y : div_rn(x, s, y); };
    ep_u32x2 r;
    r.x = pack4_e4m3(q(bf16_lo(v.x)), q(bf16_hi(v.x)), q(bf16_lo(v.y)), q(bf16_hi(v.y)));
    r.y = pack4_e4m3(q(bf16_lo(v.z)), q(bf16_hi(v.z)), q(bf16_lo(v.w)), q(bf16_hi(v.w)));
    return r;
}

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
    if (width <= 16) {
        if (width >= 2) v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
        if (width >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
        if (width >= 8) v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
        if (width >= 16) v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
        return v;
    }
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

// s = RN(max(amax, 1e-4) / 448) as a multiply by RN(1/448) and one exact
// residual correction (the refinement of div_rn): the dividend takes 129
// significands (those of bf16 values, and 1e-4f's), all checked
// exhaustively against IEEE division.
__device__ __forceinline__ float scale_of(float amax) {
    const float ap = amax > 1e-4f ? amax : 1e-4f;
    const float c = 1.0f / 448.0f;   // RN(1/448), folded at compile time
    const float q = ap * c;
    return __builtin_fmaf(__builtin_fmaf(-q, 448.0f, ap), c, q);
}

// Streaming accesses: rows are touched once per call, so they are issued with
// the non-temporal hint and do not displace the routing tables in L2.
template <typename T>
__device__ __forceinline__ void store_nt(T *p, T v) {
    __builtin_nontemporal_store(v, p);
}

template <typename T>
__device__ __forceinline__ T load_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}

}  // namespace ep
