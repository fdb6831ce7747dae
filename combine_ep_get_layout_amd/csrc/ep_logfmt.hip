// 10-bit logarithmic combine payload: encode, decode, and the combine that
// reads the payload directly.
//
// "DeepEP test target API reference", sec. 3.4: low_latency_combine can send
// the expert outputs back in a 10-bit log format (use_logfmt) instead of
// bf16.  The page gives only the width; the format here:
//   - 128-channel groups of one row, each with a 16-bit reference;
//   - the log of a bf16 magnitude is its 15 magnitude bits taken as a
//     fixed-point base-2 logarithm (exponent field, then the mantissa as the
//     fraction: Mitchell's piecewise-linear log2), rounded half to even to
//     five fraction bits and held at 0x1FDF, the largest finite value;
//   - reference = the group's largest log; code = sign bit (bit 9) over the
//     index log - reference + 511 (bits 0..8): the largest magnitude is 511,
//     index 0 is zero (zeros, logs of 0, and values 511 or more log units
//     under the reference), signed as the input;
//   - a group holding an infinity or NaN gets the reference 0xFFFF and all
//     codes 0, and decodes to NaN;
//   - decoding is exact: the bf16 magnitude bits are (reference - 511 +
//     index) << 2, so every decoded value is a bf16 number and the combine
//     over the payload is the bf16 combine of the decoded rows.
//
// Packed row (stride ep_logfmt_row_bytes(H), a multiple of 128 bytes so
// that every row starts on a cache line): H bytes of
// code bits 0..7 in channel order; H/16 little-endian words, word v holding
// the high bits of channels 16v..16v+15: channel 16v+2p+e (p = 0..7, e = 0,1)
// has its code's bit 8 in bit 7-p+16e and its sign in bit 15-p+16e; H/128
// references (uint16); the tail up to the stride is neither written nor read.
//
// Kernel shape: a wave covers 1024 channels of a row, a lane 16 of them (one
// 16-byte vector of low bytes, one high word); a group is 8 lanes, aligned.
// Decoding works on channel pairs (2p, 2p+1) as packed 16-bit halves: one
// byte permute puts the two low bytes in the halves, the high word shifted
// left by p+1 has both bit-8s at bits 8 and 24 (and, shifted by p, the
// pair's signs sit at bits 15 and 31), one packed multiply-add makes
// (index + reference - 511) << 2, the bf16 magnitude bits, and a packed
// min / multiply clears the halves whose index is 0.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kChanPerLane = 16;
constexpr int kChanPerWave = kChanPerLane * 64;
constexpr uint32_t kMaxLog = 0x1FDF;
constexpr uint32_t kPoison = 0xFFFF;
constexpr int kRowsInFlight = 4;
// Sparse encode (a layout whose pairs fill at most a quarter of the rows):
// waves per 64-row block, and rows loaded together by one wave.  Four and
// four measured best at the decode shape (1,024 of 32,768 rows: 9 us,
// against 23 us for a wave per row); on dense batches this launch is slower
// than a wave per row (154 against 133 us at prefill), hence the two.
constexpr int kEncodeRows = 4;
constexpr int kEncodeSplit = 4;

struct LogfmtK {
    const uint8_t *src;     // bf16 rows (encode) or payload rows (decode)
    uint8_t *dst;           // payload rows (encode) or bf16 rows (decode)
    const int32_t *row_src; // encode: rows with row_src[r] < 0 are skipped (or NULL)
    int64_t rows;
    int hidden;
    int stride;             // payload row bytes
    int wpr;                // waves per row
};

// Packed 16-bit integer operations (two halves per register).  Written out
// because the compiler turns a multiply by min(x, 1) into per-half compares
// and selects, and x * 4 + y into a shift and an add.
__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_mul_lo_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_mul_lo_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_max_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
// a - b per half, held at 0 (unsigned saturation).
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_lshr_u16(uint32_t a, uint32_t n2) {
    uint32_t d;
    asm("v_pk_lshrrev_b16 %0, %1, %2" : "=v"(d) : "v"(n2), "v"(a));
    return d;
}

// max over aligned groups of 8 lanes, by DPP moves (all lanes active).
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    return v;
}

// Encoding works on the same channel pairs: the magnitude bits u of a pair
// are one register (u = x & 0x7FFF7FFF); the group's reference comes from
// the largest u (the log is monotone in u, and u >= 0x7F80 is an infinity
// or NaN); per pair, l = min((u + 1 + bit 2 of u) >> 2, 0x1FDF) is the
// rounded log of both halves (no carry crosses a half: u <= 0x7F7F there),
// l + 511 where l >= 1, then a saturating subtract of the reference gives
// both indices, 0 where flushed or zero.
// One row's 16 channels of this lane, loaded as x: codes and high bits
// stored; the lane with (lane & 7) == 0 stores its group's reference.
// Every lane of the wave calls it (the group max exchanges across lanes).
__device__ __forceinline__ void encode_lane(const LogfmtK &a, int64_t r, int v, int lane,
                                            bool live, const ep_u32x4 *x) {
    uint32_t w[8], u[8];
    uint32_t umax2 = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {                 // pair p: channels 2p, 2p+1
        w[p] = x[p >> 2][p & 3];
        u[p] = w[p] & 0x7FFF7FFFu;
        umax2 = pk_max_u16(umax2, u[p]);
    }
    uint32_t umax = max(umax2 & 0xFFFFu, umax2 >> 16);
    umax = group8_max(umax);                      // groups never straddle a wave
    if (!live) return;
    const uint32_t top =
        umax >= 0x7F80u ? kPoison : min((umax + 1u + ((umax >> 2) & 1u)) >> 2, kMaxLog);
    uint32_t lo[4] = {0u, 0u, 0u, 0u};
    uint32_t hi = 0;
    if (top != kPoison) {
        const uint32_t top2 = top | (top << 16);
        uint32_t idx[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const uint32_t s = u[p] + 0x00010001u + ((u[p] >> 2) & 0x00010001u);
            const uint32_t l = pk_min_u16(pk_lshr_u16(s, 0x00020002u), 0x1FDF1FDFu);
            const uint32_t t = pk_mad_u16(pk_min_u16(l, 0x00010001u), 0x01FF01FFu, l);
            idx[p] = pk_sub_sat_u16(t, top2);
            hi |= ((idx[p] >> (p + 1)) & (0x01000100u >> (p + 1))) |
                  ((w[p] >> p) & (0x80008000u >> p));
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) lo[d] = __builtin_amdgcn_perm(idx[2 * d + 1], idx[2 * d], 0x06040200u);
    }
    uint8_t *row = a.dst + r * (int64_t)a.stride;
    ((ep_u32x4 *)row)[v] = ep_u32x4{lo[0], lo[1], lo[2], lo[3]};
    ((uint32_t *)(row + a.hidden))[v] = hi;
    if ((lane & 7) == 0) ((uint16_t *)(row + a.hidden + a.hidden / 4))[v >> 3] = (uint16_t)top;
}

// One wave per 1,024 channels of a row; a row without a pair (row_src < 0)
// is skipped.  The launch for batches where most rows are encoded.
__global__ void __launch_bounds__(kBlock) logfmt_encode_kernel(LogfmtK a) {
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int64_t r = gw / a.wpr;
    const int ci = gw - (int)r * a.wpr;
    if (r >= a.rows) return;
    if (a.row_src && a.row_src[r] < 0) return;
    const int v = ci * 64 + lane;
    const bool live = v * kChanPerLane < a.hidden;
    ep_u32x4 x[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (live) {
        const ep_u32x4 *src = (const ep_u32x4 *)(a.src + r * (int64_t)a.hidden * 2) + 2 * v;
        x[0] = load_nt(src);
        x[1] = load_nt(src + 1);
    }
    encode_lane(a, r, v, lane, live, x);
}

// kEncodeSplit waves take 1,024 channels of a block of 64 consecutive rows:
// one lane per row checks whether the row is to be encoded (inside the
// batch, and holding a pair when row_src is given), a ballot collects them,
// and wave s of the block encodes the collected rows whose rank is s modulo
// kEncodeSplit, kEncodeRows at a time with their loads issued together.  A
// sparse batch (a fixed-capacity region at decode size, 3% of its rows
// used) then costs one check per 64 rows per wave instead of a wave per
// row, and a dense one still spreads its rows over many waves.
__global__ void __launch_bounds__(kBlock) logfmt_encode_sparse_kernel(LogfmtK a) {
    constexpr int U = kEncodeRows;
    constexpr int S = kEncodeSplit;
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int64_t rb = gw / (a.wpr * S);
    const int rest = gw - (int)rb * a.wpr * S;
    const int ci = rest / S;
    const int part = rest - ci * S;
    const int64_t r0 = rb * 64;
    if (r0 >= a.rows) return;
    const int64_t rl = r0 + lane;
    const bool want = rl < a.rows && (!a.row_src || a.row_src[rl] >= 0);
    uint64_t all = __ballot(want);
    uint64_t todo = 0;
    for (int rank = 0; all; ++rank) {             // wave-uniform
        const uint64_t bit = all & (0ull - all);
        all ^= bit;
        if (rank % S == part) todo |= bit;
    }
    const int v = ci * 64 + lane;                 // 16-channel block of the row
    const bool live = v * kChanPerLane < a.hidden;
    while (todo) {
        int off[U];
        ep_u32x4 x[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            off[u] = -1;
            x[u][0] = x[u][1] = ep_u32x4{0u, 0u, 0u, 0u};
            if (todo) {
                off[u] = __builtin_ctzll(todo);
                todo &= todo - 1;
                if (live) {
                    const ep_u32x4 *s =
                        (const ep_u32x4 *)(a.src + (r0 + off[u]) * (int64_t)a.hidden * 2) + 2 * v;
                    x[u][0] = load_nt(s);
                    x[u][1] = load_nt(s + 1);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (off[u] >= 0) encode_lane(a, r0 + off[u], v, lane, live, x[u]);
    }
}

// (reference - 511) * 4 in both 16-bit halves.
__device__ __forceinline__ uint32_t base4x2_of(uint32_t ref) {
    const uint32_t b = ((ref - 511u) << 2) & 0xFFFFu;
    return b | (b << 16);
}

// The bf16 pairs of a lane's 16 channels: out[p] holds channels 2p (low
// half) and 2p+1 (high half).
__device__ __forceinline__ void decode_pairs(const ep_u32x4 &lo, uint32_t hi, uint32_t base4x2,
                                             uint32_t out[8]) {
    uint32_t sp = hi;                               // hi << p
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t sn = hi << (p + 1);
        const uint32_t bytes =
            __builtin_amdgcn_perm(0u, lo[p >> 1], (p & 1) ? 0x0C030C02u : 0x0C010C00u);
        const uint32_t f = (sn & 0x01000100u) | bytes;          // two 9-bit indices
        const uint32_t m = pk_mad_u16(f, 0x00040004u, base4x2);  // (f + base) << 2
        out[p] = pk_mul_lo_u16(m, pk_min_u16(f, 0x00010001u)) | (sp & 0x80008000u);
        sp = sn;
    }
}

__global__ void __launch_bounds__(kBlock) logfmt_decode_kernel(LogfmtK a) {
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int64_t r = gw / a.wpr;
    const int ci = gw - (int)r * a.wpr;
    if (r >= a.rows) return;
    const int v = ci * 64 + lane;
    if (v * kChanPerLane >= a.hidden) return;
    const uint8_t *row = a.src + r * (int64_t)a.stride;
    const ep_u32x4 lo = load_nt((const ep_u32x4 *)row + v);
    const uint32_t hi = load_nt((const uint32_t *)(row + a.hidden) + v);
    const uint32_t ref = load_nt((const uint16_t *)(row + a.hidden + a.hidden / 4) + (v >> 3));
    uint32_t o[8];
    decode_pairs(lo, hi, base4x2_of(ref), o);
    if (ref == kPoison) {
#pragma unroll
        for (int p = 0; p < 8; ++p) o[p] = 0x7FC07FC0u;
    }
    ep_u32x4 *d = (ep_u32x4 *)(a.dst + r * (int64_t)a.hidden * 2) + 2 * v;
    store_nt(d, ep_u32x4{o[0], o[1], o[2], o[3]});
    store_nt(d + 1, ep_u32x4{o[4], o[5], o[6], o[7]});
}

struct CombineLK {
    const uint8_t *y;       // payload rows
    int64_t y_rows;
    int stride;
    const float *w;
    const uint8_t *b0;
    const uint8_t *b1;
    const int32_t *dst;
    int32_t *status;
    const float *recv_w;
    float *combined_w;
    uint8_t *out;
    int T, K, hidden, wpr;
};

__device__ __forceinline__ void add_bf16x16(float *acc, const uint8_t *row, int v) {
    const ep_u32x4 *s = (const ep_u32x4 *)row + 2 * v;
    const ep_u32x4 p = load_nt(s), q = load_nt(s + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[2 * j] = acc[2 * j] + bf16_lo(p[j]);
        acc[2 * j + 1] = acc[2 * j + 1] + bf16_hi(p[j]);
        acc[8 + 2 * j] = acc[8 + 2 * j] + bf16_lo(q[j]);
        acc[8 + 2 * j + 1] = acc[8 + 2 * j + 1] + bf16_hi(q[j]);
    }
}

// Same reduction as combine_kernel: acc = 0; += bias0; += bias1; then
// fmaf(w[t,k], y, acc) over kept pairs in ascending k; bf16 result.  A
// marked group's weight becomes NaN, which makes its 128 channels NaN.
__global__ void __launch_bounds__(kBlock) combine_logfmt_kernel(CombineLK a) {
    constexpr int U = kRowsInFlight;
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = gw / a.wpr;
    const int ci = gw - t * a.wpr;
    if (t >= a.T) return;
    const int v = ci * 64 + lane;
    const bool live = v * kChanPerLane < a.hidden;
    const int refs_at = a.hidden + a.hidden / 4;

    float acc[kChanPerLane];
#pragma unroll
    for (int j = 0; j < kChanPerLane; ++j) acc[j] = 0.0f;
    if (live && a.b0) add_bf16x16(acc, a.b0 + (int64_t)t * a.hidden * 2, v);
    if (live && a.b1) add_bf16x16(acc, a.b1 + (int64_t)t * a.hidden * 2, v);

    for (int kb = 0; kb < a.K; kb += 64) {
        int my_slot = -1;
        float my_w = 1.0f;
        if (kb + lane < a.K) {
            my_slot = a.dst[(int64_t)t * a.K + kb + lane];
            if (a.w) my_w = a.w[(int64_t)t * a.K + kb + lane];
        }
        if ((int64_t)my_slot >= a.y_rows) {
            atomicOr(a.status, kDevRecvOverflow);
            my_slot = -1;
        }
        if (ci == 0 && a.combined_w && kb + lane < a.K)
            a.combined_w[(int64_t)t * a.K + kb + lane] = my_slot >= 0 ? a.recv_w[my_slot] : 0.0f;
        const int kn = min(64, a.K - kb);
        for (int k0 = 0; k0 < kn; k0 += U) {
            ep_u32x4 lo[U];
            uint32_t hi[U], ref[U];
            int slot[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                slot[u] = k0 + u < kn ? lane_read(my_slot, k0 + u) : -1;
                lo[u] = ep_u32x4{0u, 0u, 0u, 0u};
                hi[u] = 0u;
                ref[u] = 0u;
                if (slot[u] >= 0 && live) {
                    const uint8_t *row = a.y + (int64_t)slot[u] * a.stride;
                    lo[u] = load_nt((const ep_u32x4 *)row + v);
                    hi[u] = load_nt((const uint32_t *)(row + a.hidden) + v);
                    ref[u] = load_nt((const uint16_t *)(row + refs_at) + (v >> 3));
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (slot[u] < 0) continue;
                float wk = lane_read_f(my_w, k0 + u);
                if (ref[u] == kPoison) wk = __uint_as_float(0x7FC00000u);
                uint32_t pr[8];
                decode_pairs(lo[u], hi[u], base4x2_of(ref[u]), pr);
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    acc[2 * p] = __builtin_fmaf(wk, bf16_lo(pr[p]), acc[2 * p]);
                    acc[2 * p + 1] = __builtin_fmaf(wk, bf16_hi(pr[p]), acc[2 * p + 1]);
                }
            }
        }
    }
    if (!live) return;
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = bf16_rne(acc[2 * j]) | (bf16_rne(acc[2 * j + 1]) << 16);
    ep_u32x4 *d = (ep_u32x4 *)(a.out + (int64_t)t * a.hidden * 2) + 2 * v;
    store_nt(d, ep_u32x4{o[0], o[1], o[2], o[3]});
    store_nt(d + 1, ep_u32x4{o[4], o[5], o[6], o[7]});
}

int64_t grid_of(int64_t rows, int wpr) {
    return (rows * wpr + kWavesPerBlock - 1) / kWavesPerBlock;
}

}  // namespace

int64_t logfmt_row_bytes(int hidden) {
    const int64_t used = (int64_t)hidden + hidden / 4 + 2 * (hidden / 128);
    return (used + 127) / 128 * 128;
}

hipError_t launch_logfmt(const void *src, void *dst, int64_t rows, int hidden, bool encode,
                         const int32_t *row_src, int64_t max_used_rows, hipStream_t stream) {
    LogfmtK k = {};
    k.src = (const uint8_t *)src;
    k.dst = (uint8_t *)dst;
    k.row_src = row_src;
    k.rows = rows;
    k.hidden = hidden;
    k.stride = (int)logfmt_row_bytes(hidden);
    k.wpr = (hidden + kChanPerWave - 1) / kChanPerWave;
    const bool sparse = encode && row_src && max_used_rows * 4 <= rows;
    const int64_t units = sparse ? (rows + 63) / 64 * kEncodeSplit : rows;
    const int64_t grid = grid_of(units, k.wpr);
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFF || units * k.wpr > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (sparse)
        hipLaunchKernelGGL(logfmt_encode_sparse_kernel, dim3((unsigned)grid), dim3(kBlock), 0,
                           stream, k);
    else if (encode)
        hipLaunchKernelGGL(logfmt_encode_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, k);
    else
        hipLaunchKernelGGL(logfmt_decode_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, k);
    return hipGetLastError();
}

hipError_t launch_combine_logfmt(const CombineArgs &c, hipStream_t stream) {
    CombineLK k = {};
    k.y = (const uint8_t *)c.y;
    k.y_rows = c.y_rows;
    k.stride = (int)logfmt_row_bytes(c.hidden);
    k.w = c.w;
    k.b0 = (const uint8_t *)c.bias0;
    k.b1 = (const uint8_t *)c.bias1;
    k.dst = c.dst;
    k.status = c.status;
    k.recv_w = c.recv_w;
    k.combined_w = c.combined_w;
    k.out = (uint8_t *)c.out;
    k.T = c.T;
    k.K = c.K;
    k.hidden = c.hidden;
    k.wpr = (c.hidden + kChanPerWave - 1) / kChanPerWave;
    const int64_t grid = grid_of(k.T, k.wpr);
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFF || (int64_t)k.T * k.wpr > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_logfmt_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, k);
    return hipGetLastError();
}

}  // namespace ep
