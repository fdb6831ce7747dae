// Dispatch: permute token rows into the expert-ordered receive buffer, with
// the fp8 e4m3 variants, plus the standalone per-(token, group) fp8 cast.
//
// What is computed ("DeepEP test target API reference", sec. 2.1: recv_x has
// the input's type, fp8 input travels as (codes, scales), do_zero_padding;
// sec. 4.2: per-token cast, scale = amax / 448, codes = x / scale as
// float8_e4m3fn, here with one scale per group of G channels):
//   recv[dst[t,k]] = row(x[t])       for every pair with dst >= 0,
// with padding rows zeroed on request and recv weights 0 on padding.
//
// Kernel shape (gfx950, wave64).  A wave owns one chunk of VPL x 64 16-byte
// vectors of a token row (VPL = 14: the whole 7168-channel bf16 row): it
// loads the chunk once into registers with non-temporal loads (x is read
// exactly once) and stores it to each of the token's K destination rows with
// 16-byte stores.  Rows are moved as integer vectors, never as floats.  The
// copy modes run on a grid of resident waves, each streaming its share of
// the tokens with the next token's chunk in flight while the current one is
// stored.  In the cast modes the chunk is converted in registers: per-group
// amax by DPP exchanges, fp32 scale, the correctly rounded quotient from one
// reciprocal per group, e4m3 round-to-nearest-even, 8 codes per lane per
// vector.  Padding rows are handled by extra workgroups of the same launch
// (one slice of one expert's padding each).
#include <atomic>

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

struct DispatchK {
    const uint8_t *x;
    const uint8_t *x_scales;  // [T, ng] scales of fp8 x: fp32, or UE8M0 bytes
    const float *w;
    const int32_t *dst;       // NULL: identity (cast only), slot = t, K = 1
    const int32_t *counts;
    const int32_t *offsets;
    int32_t *status;
    uint8_t *recv;
    uint8_t *recv_scales;     // [rows, ng] scales of fp8 rows: fp32, or UE8M0 bytes
    float *recv_w;
    int64_t recv_rows;
    int T, K, E, C;
    int nd;                   // destinations per token: K (expanded) or P (partitioned)
    const int64_t *idx;       // partitioned: routing [T, K]
    int64_t *recv_idx;        // partitioned: [rows, K] local expert ids, or NULL
    float *recv_wk;           // partitioned: [rows, K] weights, or NULL
    int m;                    // partitioned: experts per partition (0: expanded)
    int meta_vec;             // partitioned: metadata rows 16-byte aligned (K % 4 == 0)
    int meta_rows;            // partitioned: metadata by row workgroups after the token ones
    const int32_t *part_src;      // partitioned: token of each receive row
    const int32_t *part_offset;   // partitioned: [P+1] first row of each partition
    int P;
    int nvec;                 // 16-byte vectors per input row
    int in_row_bytes;
    int out_row_bytes;
    int ng;                   // scales per row (fp8 modes)
    int scale_fmt;            // 0: fp32 amax/448; 1: fp32 power of two; 2: UE8M0 byte
    int group_lanes;          // cast: lanes per scale group; 0 = one scale per row
    int group_shift;          // cast: log2(group_lanes) (a power of two)
    uint32_t wpr_magic;       // floor(2^32 / wpr)
    int wpr;                  // waves per row
    int n_tok_blocks;
    int n_groups;             // streaming kernel: token-group slots (waves / wpr)
    int pad_slices;           // padding workgroups per expert (0 = none)
    int zero_padding;
    // A layout whose count kernel just ran (the dispatch derives its
    // slots): every workgroup turns the tile rows into prefixes, totals and
    // expert offsets in LDS; each pair's slot is offset[e] + prefix[tile][e]
    // + its tile rank; dst_slot and src_of_slot are written as slots are
    // found, and workgroup 0 publishes counts, offsets and totals.
    const int32_t *packed;    // [T*K], NULL: slots from dst
    const int32_t *rows;      // [tiles, W] per-tile counts
    int W;
    int tile_tokens;
    int num_tiles;
    int A, NG;                // (P, the partitions, is shared with the partitioned dispatch)
    int32_t *dst_out;
    int32_t *src_out;
    int64_t max_rows;
    int32_t *count_out;
    int32_t *offset_out;
    int32_t *part_out;
    int32_t *group_out;
    int32_t *cum_stats;
    uint32_t *queue;          // token queue: one counter per XCD, kQueueStride apart (or NULL)
    int lds_bytes;            // dynamic LDS per workgroup (host side)
    uint32_t pattern;         // kModeStores: the word every stored row holds
};

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kQueueStride = 64;   // uint32 between two queue counters (256 bytes)

// Launch geometry, fixed from measurements at the prefill shape:
constexpr int kRowVplLimit = 16;      // 16-byte vectors per lane: up to a 16 KB row per wave
constexpr int kTokensPerGroup = 2;    // consecutive tokens per group in the copy modes
                                      // (1 within noise; 4: 8% slower)
constexpr int kPadRowsPerSlice = 4;   // padding rows per workgroup when zeroing
constexpr int kResidentWavesPerCu = 12;      // copy modes: resident grid (156 VGPRs, three per SIMD)
constexpr int kResidentWavesPerCuPart = 8;   // partitioned instances (179 VGPRs, two per SIMD)
constexpr int kQueueWavesPerCu = 4;          // copy modes with the token queue
constexpr int64_t kQueueMinTokens = 16384;   // fewer tokens: the strided resident grid instead

// Receive-row stores are plain: non-temporal stores measured 3-8% slower
// for the scattered 14 KB receive rows.
template <typename T>
__device__ __forceinline__ void row_store(T *p, T v) {
    *p = v;
}

// Dynamic LDS of a dispatch workgroup that derives its layout: [tiles][W]
// exclusive prefixes of the tile rows, [W] totals, [E+1] expert offsets.
__device__ __forceinline__ int32_t *fresh_lds() {
    extern __shared__ __align__(16) int32_t ep_fresh_lds[];
    return ep_fresh_lds;
}
__device__ __forceinline__ const int32_t *fresh_tot(const DispatchK &a) {
    return fresh_lds() + a.num_tiles * a.W;
}
__device__ __forceinline__ const int32_t *fresh_off(const DispatchK &a) {
    return fresh_tot(a) + a.W;
}

constexpr int kFreshRegs = 9;   // tile-row vectors per thread loaded before the first row

// The layout's values this workgroup needs, rebuilt in LDS (what the slots
// phase of the layout computes): the tile rows are loaded (kFreshRegs 16-byte
// vectors per thread into registers first, then `first_rows` issues the
// caller's first row loads so they are in flight meanwhile), each column
// becomes exclusive prefixes over the tiles, the last ones the totals, and
// align(total, A) is scanned into offsets (e*C with a fixed capacity).
// Workgroup 0 then publishes counts, offsets, partition and group totals,
// cumulative stats and its status bits.  Every thread of the workgroup
// calls this.
template <typename F>
__device__ void fresh_setup(const DispatchK &a, F &&first_rows) {
    int32_t *lds = fresh_lds();
    const int tid = threadIdx.x, n = a.num_tiles, W = a.W, E = a.E, Q = W >> 2;
    const int nq = n * Q;
    ep_u32x4 *pre4 = (ep_u32x4 *)lds;
    const ep_u32x4 *rows4 = (const ep_u32x4 *)a.rows;
    ep_u32x4 st[kFreshRegs];
#pragma unroll
    for (int i = 0; i < kFreshRegs; ++i) {
        const int j = tid + i * kBlock;
        st[i] = j < nq ? rows4[j] : ep_u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
    first_rows();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kFreshRegs; ++i) {
        const int j = tid + i * kBlock;
        if (j < nq) pre4[j] = st[i];
    }
    for (int j = tid + kFreshRegs * kBlock; j < nq; j += kBlock) pre4[j] = rows4[j];
    lds_barrier();
    int32_t *tot = lds + n * W;
    int32_t *off = tot + W;
    for (int q = tid; q < Q; q += kBlock) {
        ep_u32x4 run = {0u, 0u, 0u, 0u};
        for (int r = 0; r < n; ++r) {
            const ep_u32x4 v = pre4[r * Q + q];
            pre4[r * Q + q] = run;
            run += v;
        }
        ((ep_u32x4 *)tot)[q] = run;
    }
    lds_barrier();
    if (a.C == 0) {
        for (int e = tid; e < E; e += kBlock) off[e] = (tot[e] + a.A - 1) / a.A * a.A;
        lds_barrier();
        if (tid < 64) {
            const int total = wave_exclusive_scan(off, E);
            if (tid == 0) off[E] = total;
        }
    } else {
        for (int e = tid; e <= E; e += kBlock) off[e] = e * a.C;
    }
    lds_barrier();
    if (blockIdx.x != 0) return;
    int fl = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int c = tot[e];
        a.count_out[e] = c;
        a.offset_out[e] = off[e];
        if (a.cum_stats) a.cum_stats[e] += c;
        if (a.C > 0 && c > a.C) fl |= kDevCapacity;
    }
    for (int q = tid; q < a.P; q += kBlock) a.part_out[q] = tot[E + q];
    if (a.group_out)
        for (int g = tid; g < a.NG; g += kBlock) a.group_out[g] = tot[E + a.P + g];
    if (tid == 0) {
        a.offset_out[E] = off[E];
        if ((int64_t)off[E] > a.max_rows) fl |= kDevRecvOverflow;
        if (tot[E + a.P + a.NG] > 0) fl |= kDevBadExpert;
    }
    if (fl) atomicOr(a.status, fl);
}

// Slot of pair k of token t: the layout's dst entry or, for a layout derived
// here, offset[e] + prefix[tile of t][e] + tile rank (-1 for no expert and
// past a fixed capacity), exactly what the layout's slots phase writes.
__device__ __forceinline__ int pair_slot(const DispatchK &a, int t, int k) {
    if (!a.packed) return a.dst[(int64_t)t * a.nd + k];
    const int v = a.packed[(int64_t)t * a.K + k];
    if (v < 0) return -1;
    const int e = v >> kRankBits;
    const int j = fresh_lds()[(t / a.tile_tokens) * a.W + e] + (v & ((1 << kRankBits) - 1));
    if (a.C > 0 && j >= a.C) return -1;
    return fresh_off(a)[e] + j;
}

// The layout's own outputs for a pair whose slot was derived here.
__device__ __forceinline__ void record_slot(const DispatchK &a, int t, int k, int slot) {
    const int64_t p = (int64_t)t * a.K + k;
    a.dst_out[p] = slot;
    if (slot >= 0 && (int64_t)slot < a.max_rows) a.src_out[slot] = (int32_t)p;
}

// Scale element size and stores (fp32, or one UE8M0 byte per group).
__device__ __forceinline__ int scale_bytes(const DispatchK &a) { return a.scale_fmt == 2 ? 1 : 4; }

__device__ __forceinline__ void store_scale(const DispatchK &a, int64_t slot, int j, float s) {
    if (a.scale_fmt == 2) a.recv_scales[slot * a.ng + j] = (uint8_t)ue8m0_of(s);
    else ((float *)a.recv_scales)[slot * a.ng + j] = s;
}

// fp8 copy: the token's scale row to the receive row, by lanes.
__device__ __forceinline__ void copy_scales(const DispatchK &a, int t, int64_t slot, int lane) {
    if (a.scale_fmt == 2) {
        const uint8_t *ss = a.x_scales + (int64_t)t * a.ng;
        uint8_t *sd = a.recv_scales + slot * a.ng;
        for (int j = lane; j < a.ng; j += 64) sd[j] = ss[j];
    } else {
        const float *ss = (const float *)a.x_scales + (int64_t)t * a.ng;
        float *sd = (float *)a.recv_scales + slot * a.ng;
        for (int j = lane; j < a.ng; j += 64) sd[j] = ss[j];
    }
}

// Scale of one group from its amax, in the call's format (fp32 values; the
// UE8M0 byte is taken from the power of two when stored).
__device__ __forceinline__ float group_scale(const DispatchK &a, float amax) {
    const float s = scale_of(amax);
    return a.scale_fmt == 0 ? s : pow2_ceil(s);
}

// 8 codes of one vector: with a power-of-two scale the quotient is one
// exact multiply, else the corrected one.
__device__ __forceinline__ ep_u32x2 encode8(const DispatchK &a, ep_u32x4 v, float s, float y) {
    return a.scale_fmt != 0 ? encode8_y<true>(v, s, y) : encode8_y<false>(v, s, y);
}

// gw / wpr for a wave-uniform gw < 2^31: a multiply-high by
// floor(2^32 / wpr) (computed on the host) gives the quotient or one less.
__device__ __forceinline__ int div_wpr(const DispatchK &a, int gw) {
    int q = (int)__umulhi((uint32_t)gw, a.wpr_magic);
    if ((q + 1) * a.wpr <= gw) ++q;
    return q;
}

// Cast of a whole row held by one wave, with one scale per row (groups
// narrower than the row go through the pairs kernels): the row's amax, its
// scale, then 8 codes per lane per vector.  Returns the scale.
template <int VPL>
__device__ __forceinline__ float cast_row(const DispatchK &a, const ep_u32x4 (&v)[VPL],
                                          ep_u32x2 (&q)[VPL]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) m = fmaxf(m, amax8(v[i]));
    const float s = group_scale(a, group_max(m, 64));
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < VPL; ++i) q[i] = encode8(a, v[i], s, y);
    return s;
}

// Codes and the scale of one cast row into receive row `slot`.
template <int VPL>
__device__ __forceinline__ void store_cast_row(const DispatchK &a, int64_t slot, int lane, float s,
                                               const ep_u32x2 (&q)[VPL]) {
    ep_u32x2 *dstrow = (ep_u32x2 *)(a.recv + slot * a.out_row_bytes);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int vi = i * 64 + lane;
        if (vi < a.nvec) row_store(dstrow + vi, q[i]);
    }
    if (lane == 0) store_scale(a, slot, 0, s);
}

// Partitioned metadata of row (t, q) (slot; -1: this lane has no row) for
// pairs [kb, kb + kn) of the token, whose expert ids and weights are held
// one pair per lane (e: -1 for none or invalid; wv): every pair's
// partition-local id when it belongs to q, else -1, and its weight, else 0.
// Broadcast by readlane; each destination lane writes its row four pairs at
// a time with 16-byte stores when the rows are aligned for them (meta_vec).
__device__ __forceinline__ void write_meta(const DispatchK &a, int q, int slot, int kb, int kn,
                                           int e, float wv) {
    const int64_t row = (int64_t)slot * a.K + kb;
    for (int k = 0; k < kn; k += 4) {
        int loc[4];
        float wt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ej = k + j < kn ? lane_read(e, k + j) : -1;
            const float wj = k + j < kn ? lane_read_f(wv, k + j) : 0.0f;
            const bool mine = ej >= 0 && ej / a.m == q;
            loc[j] = mine ? ej - q * a.m : -1;
            wt[j] = mine ? wj : 0.0f;
        }
        if (slot < 0) continue;
        if (a.meta_vec && k + 4 <= kn) {
            if (a.recv_idx) {
                ep_u32x4 *p = (ep_u32x4 *)(a.recv_idx + row + k);
                p[0] = ep_u32x4{(uint32_t)loc[0], (uint32_t)(loc[0] >> 31), (uint32_t)loc[1],
                                (uint32_t)(loc[1] >> 31)};
                p[1] = ep_u32x4{(uint32_t)loc[2], (uint32_t)(loc[2] >> 31), (uint32_t)loc[3],
                                (uint32_t)(loc[3] >> 31)};
            }
            if (a.recv_wk)
                *(ep_u32x4 *)(a.recv_wk + row + k) =
                    ep_u32x4{__float_as_uint(wt[0]), __float_as_uint(wt[1]), __float_as_uint(wt[2]),
                             __float_as_uint(wt[3])};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (k + j >= kn) break;
                if (a.recv_idx) a.recv_idx[row + k + j] = loc[j];
                if (a.recv_wk) a.recv_wk[row + k + j] = wt[j];
            }
        }
    }
}

// Token t's expert id and weight for pair kb + lane (partitioned mode).
__device__ __forceinline__ void load_pair(const DispatchK &a, int t, int kb, int lane, int &e, float &wv) {
    e = -1;
    wv = 0.0f;
    if (kb + lane < a.K) {
        const int64_t v = a.idx[(int64_t)t * a.K + kb + lane];
        e = (v >= 0 && v < a.E) ? (int)v : -1;
        wv = a.w ? a.w[(int64_t)t * a.K + kb + lane] : 1.0f;
    }
}

// Partitioned metadata in receive order: thread r of these workgroups writes
// row r (< Rp) for its token part_src[r] and partition q (the last one whose
// first row is <= r), so consecutive threads write consecutive rows.
__device__ __forceinline__ void meta_rows(const DispatchK &a, int mb) {
    const int64_t r = (int64_t)mb * kBlock + threadIdx.x;
    const int rp = a.part_offset[a.P];
    if (r >= rp || r >= a.recv_rows) return;
    const int t = a.part_src[r];
    int lo = 0, hi = a.P - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.part_offset[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int q = lo, K = a.K;
    const int64_t *ids = a.idx + (int64_t)t * K;
    const float *ws = a.w ? a.w + (int64_t)t * K : nullptr;
    for (int k = 0; k < K; k += 4) {
        int loc[4];
        float wt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            loc[j] = -1;
            wt[j] = 0.0f;
            if (k + j < K) {
                const int64_t e = ids[k + j];
                if (e >= 0 && e < a.E && e / a.m == q) {
                    loc[j] = (int)(e - (int64_t)q * a.m);
                    wt[j] = ws ? ws[k + j] : 1.0f;
                }
            }
        }
        if (a.meta_vec && k + 4 <= K) {
            if (a.recv_idx) {
                ep_u32x4 *p = (ep_u32x4 *)(a.recv_idx + r * K + k);
                p[0] = ep_u32x4{(uint32_t)loc[0], (uint32_t)(loc[0] >> 31), (uint32_t)loc[1],
                                (uint32_t)(loc[1] >> 31)};
                p[1] = ep_u32x4{(uint32_t)loc[2], (uint32_t)(loc[2] >> 31), (uint32_t)loc[3],
                                (uint32_t)(loc[3] >> 31)};
            }
            if (a.recv_wk)
                *(ep_u32x4 *)(a.recv_wk + r * K + k) =
                    ep_u32x4{__float_as_uint(wt[0]), __float_as_uint(wt[1]), __float_as_uint(wt[2]),
                             __float_as_uint(wt[3])};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (k + j >= K) break;
                if (a.recv_idx) a.recv_idx[r * K + k + j] = loc[j];
                if (a.recv_wk) a.recv_wk[r * K + k + j] = wt[j];
            }
        }
    }
}

// Per-destination bookkeeping, called by every lane of the wave with its
// destination q (slot -1 when the lane has none): the expanded layout
// records the pair's weight in its row, the partitioned layout (PART, its
// own kernel instances, so the expanded ones carry none of this code and
// keep their register count) the row's metadata, reading the routing here.
template <bool PART>
__device__ __forceinline__ void record_dest(const DispatchK &a, int t, int q, int slot, float w) {
    if (!PART) {
        if (slot >= 0 && a.recv_w) a.recv_w[slot] = w;
        return;
    }
    if (a.meta_rows) return;   // written in receive order by the row workgroups
    for (int kb = 0; kb < a.K; kb += 64) {
        int e;
        float wv;
        load_pair(a, t, kb, __lane_id(), e, wv);
        write_meta(a, q, slot, kb, min(64, a.K - kb), e, wv);
    }
}

__device__ __forceinline__ void pad_rows(const DispatchK &a, int pb) {
    if (a.pad_slices == 0) return;
    const int e = pb / a.pad_slices;
    const int sl = pb - e * a.pad_slices;
    if (e >= a.E) return;
    const int32_t *counts = a.packed ? fresh_tot(a) : a.counts;
    const int32_t *offsets = a.packed ? fresh_off(a) : a.offsets;
    const int c = counts[e];
    const int used = a.C > 0 ? min(c, a.C) : c;
    const int64_t beg = (int64_t)offsets[e] + used;
    int64_t end = a.C > 0 ? (int64_t)offsets[e] + a.C : (int64_t)offsets[e + 1];
    if (a.packed) {
        // the layout's padding slots
        const int64_t lend = end < a.max_rows ? end : a.max_rows;
        for (int64_t r = beg + sl * kBlock + threadIdx.x; r < lend; r += (int64_t)a.pad_slices * kBlock)
            a.src_out[r] = -1;
    }
    if (end > a.recv_rows) end = a.recv_rows;
    if (!a.zero_padding) {
        // weights only: one thread per padding row
        if (a.recv_w)
            for (int64_t r = beg + sl * kBlock + threadIdx.x; r < end; r += (int64_t)a.pad_slices * kBlock)
                a.recv_w[r] = 0.0f;
        return;
    }
    const int nv_out = a.out_row_bytes >> 4;
    const ep_u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t r = beg + sl; r < end; r += a.pad_slices) {
        ep_u32x4 *row = (ep_u32x4 *)(a.recv + r * (int64_t)a.out_row_bytes);
        for (int v = threadIdx.x; v < nv_out; v += kBlock) row_store(row + v, z);
        if (a.recv_scales)
            for (int j = threadIdx.x; j < a.ng * scale_bytes(a); j += kBlock)
                a.recv_scales[r * a.ng * scale_bytes(a) + j] = 0;
        if (a.recv_w && threadIdx.x == 0) a.recv_w[r] = 0.0f;
    }
}

template <int VPL, int MODE, bool PART>
__global__ void __launch_bounds__(kBlock) dispatch_kernel(DispatchK a) {
    if ((int)blockIdx.x >= a.n_tok_blocks) {
        if (PART && a.meta_rows) meta_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        else pad_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        return;
    }
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = gw / a.wpr;
    const int ci = gw - t * a.wpr;
    if (t >= a.T) return;
    const int K = a.dst ? a.nd : 1;
    const int v0 = ci * VPL * 64;

    // Load this wave's chunk of the row once.
    ep_u32x4 v[VPL];
    const ep_u32x4 *src = (const ep_u32x4 *)(a.x + (int64_t)t * a.in_row_bytes);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int vi = v0 + i * 64 + lane;
        if (vi < a.nvec) v[i] = load_nt(src + vi);
        else v[i] = ep_u32x4{0u, 0u, 0u, 0u};
    }

    // Per-pair destinations and weights, one pair per lane (K <= 64 per pass).
    for (int kb = 0; kb < K; kb += 64) {
        int my_slot = -1;
        float my_w = 1.0f;
        if (kb + lane < K) {
            my_slot = a.dst ? a.dst[(int64_t)t * a.nd + kb + lane] : t;
            if (a.w && a.m == 0) my_w = a.w[(int64_t)t * a.K + kb + lane];
        }
        if ((int64_t)my_slot >= a.recv_rows) {
            if (a.status) atomicOr(a.status, kDevRecvOverflow);
            my_slot = -1;
        }
        if (ci == 0) record_dest<PART>(a, t, kb + lane, my_slot, my_w);
        const int kn = min(64, K - kb);

        if (MODE == kModeCast) {
            ep_u32x2 q[VPL];
            const float s = cast_row<VPL>(a, v, q);
            for (int k = 0; k < kn; ++k) {
                const int slot = lane_read(my_slot, k);
                if (slot >= 0) store_cast_row<VPL>(a, slot, lane, s, q);
            }
        } else {
            for (int k = 0; k < kn; ++k) {
                const int slot = lane_read(my_slot, k);
                if (slot < 0) continue;
                ep_u32x4 *dstrow = (ep_u32x4 *)(a.recv + (int64_t)slot * a.out_row_bytes);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int vi = v0 + i * 64 + lane;
                    if (vi < a.nvec) row_store(dstrow + vi, v[i]);
                }
                if (MODE == kModeCopyFp8 && ci == 0) copy_scales(a, t, slot, lane);
            }
        }
    }
}

// fp8 copy: the token's scale row held in registers across its destinations
// (element j in lane j % 64, slot j / 64; rows of up to 64 * kScaleRegs
// scales), loaded together with the row so no destination waits on a load.
// As raw bits: a 32-bit float, or one UE8M0 byte.
constexpr int kScaleRegs = 4;

__device__ __forceinline__ bool scales_in_regs(const DispatchK &a) {
    return a.ng <= 64 * kScaleRegs;
}

__device__ __forceinline__ void load_scales(const DispatchK &a, int t, int lane,
                                            uint32_t (&sc)[kScaleRegs]) {
#pragma unroll
    for (int i = 0; i < kScaleRegs; ++i) {
        const int j = i * 64 + lane;
        sc[i] = 0u;
        if (j < a.ng)
            sc[i] = a.scale_fmt == 2 ? (uint32_t)a.x_scales[(int64_t)t * a.ng + j]
                                     : ((const uint32_t *)a.x_scales)[(int64_t)t * a.ng + j];
    }
}

__device__ __forceinline__ void store_scales(const DispatchK &a, int64_t slot, int lane,
                                             const uint32_t (&sc)[kScaleRegs]) {
#pragma unroll
    for (int i = 0; i < kScaleRegs; ++i) {
        const int j = i * 64 + lane;
        if (j < a.ng) {
            if (a.scale_fmt == 2) a.recv_scales[slot * a.ng + j] = (uint8_t)sc[i];
            else ((uint32_t *)a.recv_scales)[slot * a.ng + j] = sc[i];
        }
    }
}

// All destinations of token t for one row chunk (copy modes); sc holds the
// token's scale row for the fp8 copy when scales_in_regs.
template <int VPL, int MODE, bool PART>
__device__ __forceinline__ void store_token(const DispatchK &a, int t, int ci, int v0, int lane,
                                            const ep_u32x4 (&v)[VPL],
                                            const uint32_t (&sc)[kScaleRegs]) {
    for (int kb = 0; kb < a.nd; kb += 64) {
        int my_slot = -1;
        float my_w = 1.0f;
        if (kb + lane < a.nd) {
            my_slot = pair_slot(a, t, kb + lane);
            if (a.packed && ci == 0) record_slot(a, t, kb + lane, my_slot);
            if (a.w && a.m == 0) my_w = a.w[(int64_t)t * a.K + kb + lane];
        }
        if ((int64_t)my_slot >= a.recv_rows) {
            atomicOr(a.status, kDevRecvOverflow);
            my_slot = -1;
        }
        if (ci == 0) record_dest<PART>(a, t, kb + lane, my_slot, my_w);
        const int kn = min(64, a.nd - kb);
        for (int k = 0; k < kn; ++k) {
            const int slot = lane_read(my_slot, k);
            if (slot < 0) continue;
            ep_u32x4 *dstrow = (ep_u32x4 *)(a.recv + (int64_t)slot * a.out_row_bytes);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int vi = v0 + i * 64 + lane;
                if (vi < a.nvec) row_store(dstrow + vi, v[i]);
            }
            if (MODE == kModeCopyFp8 && ci == 0) {
                if (scales_in_regs(a)) store_scales(a, slot, lane, sc);
                else copy_scales(a, t, slot, lane);
            }
        }
    }
}

template <int VPL>
__device__ __forceinline__ void load_chunk(const DispatchK &a, int t, int v0, int lane, ep_u32x4 (&v)[VPL]) {
    const ep_u32x4 *src = (const ep_u32x4 *)(a.x + (int64_t)t * a.in_row_bytes);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int vi = v0 + i * 64 + lane;
        v[i] = vi < a.nvec ? load_nt(src + vi) : ep_u32x4{0u, 0u, 0u, 0u};
    }
}

// Copy modes on a grid of resident waves: wave (g, ci) streams the tokens of
// groups g, g + n_groups, g + 2 n_groups, ... (TPW consecutive tokens each),
// always holding the next token's chunk in flight while it stores the
// current one, so reads and writes stay interleaved for the whole launch.
template <int VPL, int MODE, int TPW, bool PART>
__global__ void __launch_bounds__(kBlock) dispatch_stream_kernel(DispatchK a) {
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int g = gw / a.wpr;
    const int ci = gw - g * a.wpr;
    const int v0 = ci * VPL * 64;
    const int64_t stride = (int64_t)a.n_groups * TPW;
    // j-th token of this wave
    auto tok = [&](int j) -> int64_t { return (int64_t)g * TPW + (j / TPW) * stride + (j % TPW); };
    int64_t t = tok(0);
    const bool mine = (int)blockIdx.x < a.n_tok_blocks && g < a.n_groups && t < a.T;
    ep_u32x4 v0b[VPL], v1b[VPL];
    uint32_t s0b[kScaleRegs] = {}, s1b[kScaleRegs] = {};
    const bool regs = MODE == kModeCopyFp8 && ci == 0 && scales_in_regs(a);
    // kModeStores: the row is a register pattern (the stores without the reads)
    auto load = [&](int tt, ep_u32x4 (&v)[VPL]) {
        if (MODE == kModeStores) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) v[i] = ep_u32x4{a.pattern, a.pattern, a.pattern, a.pattern};
        } else {
            load_chunk<VPL>(a, tt, v0, lane, v);
        }
    };
    auto first = [&] {
        if (mine) {
            load((int)t, v0b);
            if (regs) load_scales(a, (int)t, lane, s0b);
        }
    };
    if (a.packed) fresh_setup(a, first);
    else first();
    if ((int)blockIdx.x >= a.n_tok_blocks) {
        if (PART && a.meta_rows) meta_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        else pad_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        return;
    }
    if (!mine) return;
    for (int j = 0;; j += 2) {
        int64_t tn = tok(j + 1);
        if (tn < a.T) {
            load((int)tn, v1b);
            if (regs) load_scales(a, (int)tn, lane, s1b);
        }
        store_token<VPL, MODE, PART>(a, (int)t, ci, v0, lane, v0b, s0b);
        if (tn >= a.T) break;
        t = tn;
        tn = tok(j + 2);
        if (tn < a.T) {
            load((int)tn, v0b);
            if (regs) load_scales(a, (int)tn, lane, s0b);
        }
        store_token<VPL, MODE, PART>(a, (int)t, ci, v0, lane, v1b, s1b);
        if (tn >= a.T) break;
        t = tn;
    }
}

// Token queue of the copy modes (a layout whose count kernel just ran, whole
// rows per wave).  The tokens are split into kXcds contiguous ranges, one per
// XCD, each with a counter in the workspace that the layout's count launch,
// just before on the same stream, set to zero.  A wave takes one token at a time from the counter of the XCD it
// runs on (a one-lane global atomic, the next ticket in flight while the
// current token's rows are stored) and, once that range is used up, from the
// other XCDs' counters in turn, so an XCD that finishes early takes tokens
// from a slower one instead of idling.  Every wave stops after at most
// kXcds empty tickets.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & (kXcds - 1);   // HW_REG_XCC_ID
}

// Ticket from queue qx: its counter's old value (one lane's atomic, broadcast).
__device__ __forceinline__ uint32_t queue_ticket(const DispatchK &a, int qx) {
    uint32_t v = 0;
    if (__lane_id() == 0) v = atomicAdd(a.queue + qx * kQueueStride, 1u);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// The token a ticket of queue qx names, or, past that range, the next token
// from the following queues (taken now, one ticket each); -1 when all are
// used up.  qx and tries advance as ranges run out.
__device__ __forceinline__ int queue_token(const DispatchK &a, uint32_t v, int &qx, int &tries) {
    for (;;) {
        const int64_t lo = (int64_t)qx * a.T / kXcds, hi = (int64_t)(qx + 1) * a.T / kXcds;
        if (lo + (int64_t)v < hi) return (int)(lo + v);
        if (++tries >= kXcds) return -1;
        qx = (qx + 1) & (kXcds - 1);
        v = queue_ticket(a, qx);
    }
}

template <int VPL, int MODE>
__global__ void __launch_bounds__(kBlock) dispatch_queue_kernel(DispatchK a) {
    if (a.packed) fresh_setup(a, [] {});
    if ((int)blockIdx.x >= a.n_tok_blocks) {
        pad_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        return;
    }
    const int lane = __lane_id();
    int qx = xcc_id(), tries = 0;
    int t = queue_token(a, queue_ticket(a, qx), qx, tries);
    if (t < 0) return;
    ep_u32x4 v0b[VPL], v1b[VPL];
    uint32_t s0b[kScaleRegs] = {}, s1b[kScaleRegs] = {};
    const bool regs = MODE == kModeCopyFp8 && scales_in_regs(a);
    load_chunk<VPL>(a, t, 0, lane, v0b);
    if (regs) load_scales(a, t, lane, s0b);
    uint32_t pend = queue_ticket(a, qx);
    for (;;) {
        int tn = queue_token(a, pend, qx, tries);
        if (tn >= 0) {
            load_chunk<VPL>(a, tn, 0, lane, v1b);
            if (regs) load_scales(a, tn, lane, s1b);
            pend = queue_ticket(a, qx);
        }
        store_token<VPL, MODE, false>(a, t, 0, 0, lane, v0b, s0b);
        if (tn < 0) break;
        t = tn;
        tn = queue_token(a, pend, qx, tries);
        if (tn >= 0) {
            load_chunk<VPL>(a, tn, 0, lane, v0b);
            if (regs) load_scales(a, tn, lane, s0b);
            pend = queue_ticket(a, qx);
        }
        store_token<VPL, MODE, false>(a, t, 0, 0, lane, v1b, s1b);
        if (tn < 0) break;
        t = tn;
    }
}

// Zero fill of a fixed-capacity receive region before its token rows are
// written.  Each lane stores one 16-byte vector, so every wave writes one
// kilobyte and consecutive waves write consecutive kilobytes: with no loads
// ahead of the stores this is the fastest write pattern measured on the part.
// The workgroups after the row ones clear the scale rows and the weights.
__global__ void __launch_bounds__(kBlock) zero_fill_kernel(ep_u32x4 *rows, int64_t n16,
                                                           int64_t row_blocks, uint8_t *scales,
                                                           int64_t scale_bytes, float *w,
                                                           int64_t nw) {
    const int64_t b = blockIdx.x;
    if (b < row_blocks) {
        const int64_t v = b * kBlock + threadIdx.x;
        if (v < n16) row_store(rows + v, ep_u32x4{0u, 0u, 0u, 0u});
        return;
    }
    const int64_t nt = ((int64_t)gridDim.x - row_blocks) * kBlock;
    const int64_t i0 = (b - row_blocks) * kBlock + threadIdx.x;
    if (scales) {
        if (((uintptr_t)scales & 3u) == 0 && (scale_bytes & 3) == 0) {
            uint32_t *s4 = (uint32_t *)scales;
            for (int64_t i = i0; i < scale_bytes / 4; i += nt) s4[i] = 0u;
        } else {
            for (int64_t i = i0; i < scale_bytes; i += nt) scales[i] = 0;
        }
    }
    if (w)
        for (int64_t i = i0; i < nw; i += nt) w[i] = 0.0f;
}

hipError_t launch_zero_fill(const DispatchK &k, int64_t rows, hipStream_t stream) {
    const int64_t n16 = rows * (k.out_row_bytes / 16);
    const int64_t row_blocks = (n16 + kBlock - 1) / kBlock;
    const int64_t sb = k.recv_scales ? rows * k.ng * (k.scale_fmt == 2 ? 1 : 4) : 0;
    const int64_t nw = k.recv_w ? rows : 0;
    const int64_t tail_items = (sb / 4 > nw ? sb / 4 : nw);
    int64_t tail = (tail_items + kBlock * 8 - 1) / (kBlock * 8);
    if (tail > 1024) tail = 1024;
    const int64_t grid = row_blocks + tail;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       (ep_u32x4 *)k.recv, n16, row_blocks, k.recv_scales, sb, k.recv_w, nw);
    return hipGetLastError();
}

// Cast without a layout, groups narrower than the row.  Lane l of a wave
// holds the adjacent vectors 2l and 2l+1 of its 128-vector chunk: 16
// channels of one group, so a lane derives one scale and one reciprocal for
// its 16 values (not one per vector), and its 16 codes leave in one 16-byte
// store (the wave writes 1 KB contiguous).  nvec is even (H % 16 == 0) and a
// multiple of the vectors per group, so a group is wholly inside the row or
// wholly past its end.
__global__ void __launch_bounds__(kBlock) cast_pairs_kernel(DispatchK a) {
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = div_wpr(a, gw);
    const int c = gw - t * a.wpr;
    if (t >= a.T) return;
    const int vi = c * 128 + 2 * lane;
    const bool on = vi < a.nvec;
    const ep_u32x4 *src = (const ep_u32x4 *)(a.x + (int64_t)t * a.in_row_bytes);
    ep_u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (on) {
        v0 = load_nt(src + vi);
        v1 = load_nt(src + vi + 1);
    }
    const int gl = a.group_lanes >> 1;    // lanes per group here: G / 16
    const float s = group_scale(a, group_max(fmaxf(amax8(v0), amax8(v1)), gl));
    const float y = 1.0f / s;
    const ep_u32x2 e0 = encode8(a, v0, s, y), e1 = encode8(a, v1, s, y);
    if (on) {
        row_store((ep_u32x4 *)(a.recv + (int64_t)t * a.out_row_bytes) + (vi >> 1),
                  ep_u32x4{e0.x, e0.y, e1.x, e1.y});
        if ((vi & (a.group_lanes - 1)) == 0) store_scale(a, t, vi >> a.group_shift, s);
    }
}

// Fused cast + dispatch with the lane layout of cast_pairs_kernel: each
// lane's 16 codes go to every destination row with one 16-byte store, and
// its scale (first lane of each group) with them.  Padding or metadata
// workgroups follow the token ones, as in dispatch_kernel.
template <bool PART>
__global__ void __launch_bounds__(kBlock) dispatch_cast_pairs_kernel(DispatchK a) {
    if ((int)blockIdx.x >= a.n_tok_blocks) {
        if (PART && a.meta_rows) meta_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        else pad_rows(a, (int)blockIdx.x - a.n_tok_blocks);
        return;
    }
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = div_wpr(a, gw);
    const int ci = gw - t * a.wpr;
    if (t >= a.T) return;
    const int vi = ci * 128 + 2 * lane;
    const bool on = vi < a.nvec;
    const ep_u32x4 *src = (const ep_u32x4 *)(a.x + (int64_t)t * a.in_row_bytes);
    ep_u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (on) {
        v0 = load_nt(src + vi);
        v1 = load_nt(src + vi + 1);
    }
    const float s = group_scale(a, group_max(fmaxf(amax8(v0), amax8(v1)), a.group_lanes >> 1));
    const float y = 1.0f / s;
    const ep_u32x2 e0 = encode8(a, v0, s, y), e1 = encode8(a, v1, s, y);
    const ep_u32x4 q = {e0.x, e0.y, e1.x, e1.y};
    const bool scale_lane = on && (vi & (a.group_lanes - 1)) == 0;
    for (int kb = 0; kb < a.nd; kb += 64) {
        int my_slot = -1;
        float my_w = 1.0f;
        if (kb + lane < a.nd) {
            my_slot = a.dst[(int64_t)t * a.nd + kb + lane];
            if (a.w && a.m == 0) my_w = a.w[(int64_t)t * a.K + kb + lane];
        }
        if ((int64_t)my_slot >= a.recv_rows) {
            atomicOr(a.status, kDevRecvOverflow);
            my_slot = -1;
        }
        if (ci == 0) record_dest<PART>(a, t, kb + lane, my_slot, my_w);
        const int kn = min(64, a.nd - kb);
        for (int k = 0; k < kn; ++k) {
            const int slot = lane_read(my_slot, k);
            if (slot < 0) continue;
            if (on) row_store((ep_u32x4 *)(a.recv + (int64_t)slot * a.out_row_bytes) + (vi >> 1), q);
            if (scale_lane) store_scale(a, slot, vi >> a.group_shift, s);
        }
    }
}

// Rows go through a layout (not the cast's identity map).
inline bool routed(const DispatchK &k) { return k.dst != nullptr || k.packed != nullptr; }

template <int MODE>
hipError_t launch_queue(const DispatchK &k, int vpl, int grid, hipStream_t stream) {
#define EP_CASE(V)                                                                              \
    case V:                                                                                     \
        hipLaunchKernelGGL((dispatch_queue_kernel<V, MODE>), dim3(grid), dim3(kBlock), k.lds_bytes, \
                           stream, k);                                                          \
        break;
    switch (vpl) {
        EP_CASE(1) EP_CASE(2) EP_CASE(4) EP_CASE(7) EP_CASE(8) EP_CASE(14) EP_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef EP_CASE
    return hipGetLastError();
}

template <int MODE, bool PART>
hipError_t launch_mode(const DispatchK &k, int vpl, int grid, bool multi, hipStream_t stream) {
    if (MODE == kModeCast && routed(k) && k.group_lanes > 0) {
        hipLaunchKernelGGL((dispatch_cast_pairs_kernel<PART>), dim3(grid), dim3(kBlock), k.lds_bytes,
                           stream, k);
        return hipGetLastError();
    }
#define EP_CASE(V)                                                                              \
    case V:                                                                                     \
        if (MODE != kModeCast && multi)                                                         \
            hipLaunchKernelGGL((dispatch_stream_kernel<V, MODE, kTokensPerGroup, PART>),        \
                               dim3(grid), dim3(kBlock), k.lds_bytes, stream, k);               \
        else                                                                                    \
            hipLaunchKernelGGL((dispatch_kernel<V, MODE, PART>), dim3(grid), dim3(kBlock),      \
                               k.lds_bytes, stream, k);                                         \
        break;
    switch (vpl) {
        EP_CASE(1) EP_CASE(2) EP_CASE(4) EP_CASE(7) EP_CASE(8) EP_CASE(14) EP_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef EP_CASE
    return hipGetLastError();
}

// The stores-only instances: the expanded stream kernel only.
hipError_t launch_stores(const DispatchK &k, int vpl, int grid, hipStream_t stream) {
#define EP_CASE(V)                                                                              \
    case V:                                                                                     \
        hipLaunchKernelGGL((dispatch_stream_kernel<V, kModeStores, kTokensPerGroup, false>),    \
                           dim3(grid), dim3(kBlock), k.lds_bytes, stream, k);                   \
        break;
    switch (vpl) {
        EP_CASE(1) EP_CASE(2) EP_CASE(4) EP_CASE(7) EP_CASE(8) EP_CASE(14) EP_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef EP_CASE
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const DispatchK &k, int vpl, int grid, bool multi, hipStream_t stream) {
    return k.m > 0 ? launch_mode<MODE, true>(k, vpl, grid, multi, stream)
                   : launch_mode<MODE, false>(k, vpl, grid, multi, stream);
}

// Compute units of the current device, queried once per device.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

constexpr int64_t kMinStreamWaves = 1024;   // below this, rows are split over more waves

// Vectors per lane: the largest allowed count <= limit that divides the
// row's 64-vector chunks, else the largest <= limit and <= the chunk count.
int choose_vpl(int nvec, int limit) {
    static const int cand[] = {16, 14, 8, 7, 4, 2, 1};
    const int q = (nvec + 63) / 64;
    for (int c : cand)
        if (c <= limit && c <= q && q % c == 0 && nvec % 64 == 0) return c;
    for (int c : cand)
        if (c <= limit && c <= q) return c;
    return 1;
}

hipError_t run(DispatchK k, int mode, hipStream_t stream) {
    int vpl = choose_vpl(k.nvec, kRowVplLimit);
    // cast with a layout and groups narrower than the row: two adjacent vectors
    // per lane (dispatch_cast_pairs_kernel), i.e. 128 vectors per wave
    if (mode == kModeCast && routed(k) && k.group_lanes > 0) vpl = 2;
    if (mode == kModeCast && k.group_lanes == 0) {
        // one scale per row: the whole row must sit in one wave
        const int q = (k.nvec + 63) / 64;
        vpl = q <= 1 ? 1 : q <= 2 ? 2 : q <= 4 ? 4 : q <= 7 ? 7 : q <= 8 ? 8 : q <= 14 ? 14 : 16;
        if (q > 16) return hipErrorInvalidValue;
    }
    // copy modes with a layout: the streaming kernel, TPW tokens per group
    const int tpw = mode != kModeCast && routed(k) ? kTokensPerGroup : 1;
    const bool multi = mode != kModeCast && routed(k);
    if (multi) {
        // few tokens: split each row over more waves so the chip has work
        const int64_t groups = ((int64_t)k.T + tpw - 1) / tpw;
        while (vpl > 1 && groups * ((k.nvec + vpl * 64 - 1) / (vpl * 64)) < kMinStreamWaves)
            vpl = choose_vpl(k.nvec, vpl - 1);
    }
    k.wpr = (k.nvec + vpl * 64 - 1) / (vpl * 64);
    if (k.wpr < 1) k.wpr = 1;
    k.wpr_magic = (uint32_t)(0xFFFFFFFFu / (uint32_t)k.wpr);
    // large batches of the copy modes, whole rows per wave: the token queue
    if (multi && k.queue && k.m == 0 && k.wpr == 1 && k.T >= kQueueMinTokens) {
        int64_t qw = (int64_t)cu_count() * kQueueWavesPerCu;
        if (qw > k.T) qw = k.T;
        k.n_tok_blocks = (int)((qw + kWavesPerBlock - 1) / kWavesPerBlock);
        const int64_t qgrid = (int64_t)k.n_tok_blocks + (int64_t)k.E * k.pad_slices;
        if (qgrid > 0x7FFFFFFF) return hipErrorInvalidValue;
        return mode == kModeCopy16 ? launch_queue<kModeCopy16>(k, vpl, (int)qgrid, stream)
                                   : launch_queue<kModeCopyFp8>(k, vpl, (int)qgrid, stream);
    }
    int64_t waves = (((int64_t)k.T + tpw - 1) / tpw) * k.wpr;
    k.n_groups = (int)(((int64_t)k.T + tpw - 1) / tpw);
    if (multi) {
        const int per_cu = k.m > 0 ? kResidentWavesPerCuPart : kResidentWavesPerCu;
        int64_t cap = (int64_t)cu_count() * per_cu / k.wpr;                // group slots
        if (cap < 1) cap = 1;
        if (k.n_groups > cap) k.n_groups = (int)cap;
        waves = (int64_t)k.n_groups * k.wpr;
    }
    k.n_tok_blocks = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    int64_t grid = (int64_t)k.n_tok_blocks + (int64_t)k.E * k.pad_slices;
    if (k.meta_rows) {   // the partitioned layout has no padding: these follow the token blocks
        int64_t rows = (int64_t)k.T * k.P;
        if (rows > k.recv_rows) rows = k.recv_rows;
        grid = (int64_t)k.n_tok_blocks + (rows + kBlock - 1) / kBlock;
    }
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (mode == kModeStores) return multi ? launch_stores(k, vpl, (int)grid, stream) : hipErrorInvalidValue;
    switch (mode) {
        case kModeCopy16: return launch_mode<kModeCopy16>(k, vpl, (int)grid, multi, stream);
        case kModeCopyFp8: return launch_mode<kModeCopyFp8>(k, vpl, (int)grid, multi, stream);
        default: return launch_mode<kModeCast>(k, vpl, (int)grid, multi, stream);
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream) {
    DispatchK k = {};
    k.x = (const uint8_t *)a.x;
    k.x_scales = (const uint8_t *)a.x_scales;
    k.w = a.topk_weights;
    k.dst = a.dst;
    k.counts = a.counts;
    k.offsets = a.offsets;
    k.status = a.status;
    k.recv = (uint8_t *)a.recv;
    k.recv_scales = (uint8_t *)a.recv_scales;
    k.scale_fmt = a.scale_fmt;
    k.recv_w = a.recv_w;
    k.recv_rows = a.recv_rows;
    k.T = a.T;
    k.K = a.K;
    k.E = a.E;
    k.C = a.C;
    k.nd = a.partitioned ? a.P : a.K;
    k.m = a.partitioned ? a.E / a.P : 0;
    k.idx = a.topk_idx;
    k.recv_idx = a.recv_idx;
    k.recv_wk = a.recv_wk;
    k.meta_vec = a.K % 4 == 0 && ((uintptr_t)a.recv_idx & 15) == 0 && ((uintptr_t)a.recv_wk & 15) == 0;
    k.P = a.P;
    k.part_src = a.part_src;
    k.part_offset = a.part_offset;
    k.meta_rows = a.partitioned && a.part_src && a.part_offset && (a.recv_idx || a.recv_wk);
    if (a.partitioned) k.dst = a.token_slot;
    k.queue = a.partitioned ? nullptr : a.queue;
    // a layout derived in the row kernels: the copy modes' resident grids only
    const bool fresh = a.fresh != nullptr && !a.partitioned && a.mode != kModeCast;
    if (fresh) {
        const FreshLayout &f = *a.fresh;
        k.dst = nullptr;
        k.packed = f.packed;
        k.rows = f.rows;
        k.W = f.W;
        k.tile_tokens = f.tile_tokens;
        k.num_tiles = f.num_tiles;
        k.A = f.A;
        k.P = f.P;
        k.NG = f.NG;
        k.dst_out = f.dst_out;
        k.src_out = f.src_out;
        k.max_rows = f.max_rows;
        k.count_out = f.count_out;
        k.offset_out = f.offset_out;
        k.part_out = f.part_out;
        k.group_out = f.group_out;
        k.cum_stats = f.cum_stats;
        k.lds_bytes = (int)f.lds_bytes;
    }
    k.pattern = a.pattern;
    if (a.mode == kModeCopy16 || a.mode == kModeStores) {
        k.in_row_bytes = k.out_row_bytes = a.hidden * 2;
        k.nvec = a.hidden / 8;
    } else if (a.mode == kModeCopyFp8) {
        k.in_row_bytes = k.out_row_bytes = a.hidden;
        k.nvec = a.hidden / 16;
        k.ng = a.hidden / a.group;
    } else {
        k.in_row_bytes = a.hidden * 2;
        k.out_row_bytes = a.hidden;
        k.nvec = a.hidden / 8;
        k.ng = a.hidden / a.group;
        k.group_lanes = a.group == a.hidden ? 0 : a.group / 8;
        k.group_shift = k.group_lanes > 0 ? __builtin_ctz((unsigned)k.group_lanes) : 0;
    }
    k.zero_padding = a.zero_padding;
    int maxpad = a.C > 0 ? a.C : a.A - 1;
    // padding rows are visited for zeros, weights, or (fresh layout) src_of_slot
    if ((!a.zero_padding && !a.recv_w && !fresh) || a.partitioned) maxpad = 0;
    // Fixed capacity where at most one row in eight can hold a token (decode
    // batches): zero the whole region first, then write the token rows over
    // it, instead of finding each expert's padding rows.
    if (a.zero_padding && a.C > 0 && !a.partitioned &&
        (int64_t)a.T * a.K * 8 <= (int64_t)a.E * a.C) {
        int64_t rows = (int64_t)a.E * a.C;
        if (rows > a.recv_rows) rows = a.recv_rows;
        const hipError_t err = launch_zero_fill(k, rows, stream);
        if (err != hipSuccess) return err;
        k.zero_padding = 0;
        if (!fresh) maxpad = 0;
    }
    if (maxpad > 0)
        k.pad_slices = k.zero_padding ? (maxpad + kPadRowsPerSlice - 1) / kPadRowsPerSlice : 1;
    return run(k, a.mode, stream);
}

hipError_t launch_cast_fp8(const void *x, int T, int hidden, int group, int scale_fmt, uint8_t *q,
                           void *scales, hipStream_t stream) {
    DispatchK k = {};
    k.x = (const uint8_t *)x;
    k.dst = nullptr;
    k.status = nullptr;
    k.recv = q;
    k.recv_scales = (uint8_t *)scales;
    k.scale_fmt = scale_fmt;
    k.recv_rows = T;
    k.T = T;
    k.K = 1;
    k.nd = 1;
    k.in_row_bytes = hidden * 2;
    k.out_row_bytes = hidden;
    k.nvec = hidden / 8;
    k.ng = hidden / group;
    k.group_lanes = group == hidden ? 0 : group / 8;
    k.group_shift = k.group_lanes > 0 ? __builtin_ctz((unsigned)k.group_lanes) : 0;
    if (k.group_lanes > 0) {
        k.wpr = (k.nvec + 127) / 128;
        k.wpr_magic = (uint32_t)(0xFFFFFFFFu / (uint32_t)k.wpr);
        const int64_t blocks = ((int64_t)T * k.wpr + kWavesPerBlock - 1) / kWavesPerBlock;
        if (blocks == 0) return hipSuccess;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(cast_pairs_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, k);
        return hipGetLastError();
    }
    return run(k, kModeCast, stream);
}

}  // namespace ep
