// Combine: gather expert outputs back to their source tokens and reduce.
//
// What is computed ("DeepEP test target API reference", sec. 2.2: weighted
// reduction back to the source with 0/1/2 bias tensors, combined_x bf16
// [T, hidden]; sec. 3.2: without weights it is a plain sum; sec. 4.1: an
// ordered accumulation, no scatter_add, so results are bitwise
// reproducible):
//   acc = 0; acc += bias0; acc += bias1;
//   for k = 0..K-1 with dst[t,k] >= 0:  acc = fmaf(w[t,k], y[dst[t,k]], acc)
//   out[t] = bf16 round-to-nearest-even(acc)
//
// Kernel shape (gfx950, wave64).  A wave owns one chunk of VPL x 64 vectors
// (8 channels each) of one output row and keeps 8*VPL fp32 accumulators per
// lane.  The K destination slots and weights of the token are fetched once,
// one per lane, and broadcast with readlane, so every row address is
// wave-uniform.  Rows are fetched U at a time (U*VPL 16-byte loads in flight
// per lane) and folded in ascending k.  No atomics: each output element is
// produced by exactly one lane in a fixed order, so the result is
// deterministic and independent of the other tokens in the batch.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

struct CombineK {
    const uint8_t *y;
    int64_t y_rows;
    const float *w;
    const uint8_t *b0;
    const uint8_t *b1;
    const int32_t *dst;
    int32_t *status;
    const float *recv_w;
    float *combined_w;
    uint8_t *out;
    int T, K;
    int nvec;       // 16-byte vectors per row
    int row_bytes;
    int wpr;
    const int64_t *idx;   // reduced combine: routing [T, K]
    int E, m;             // reduced combine: experts, experts per partition
    int bf16_partials;    // reduced combine: round each partition's partial to bf16
};

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
// One 16-byte vector per lane (1 KB of a row per wave) and four rows in
// flight: 1.5 us faster at the prefill shape than two vectors and eight
// rows, 0.7 us at the decode shape; eight rows in flight or two vectors
// per lane at four rows measured no better.
constexpr int kVpl = 1;
constexpr int kRowsInFlight = 4;

__device__ __forceinline__ void add_bf16x8(float *acc, ep_u32x4 v) {
    acc[0] = acc[0] + bf16_lo(v.x);
    acc[1] = acc[1] + bf16_hi(v.x);
    acc[2] = acc[2] + bf16_lo(v.y);
    acc[3] = acc[3] + bf16_hi(v.y);
    acc[4] = acc[4] + bf16_lo(v.z);
    acc[5] = acc[5] + bf16_hi(v.z);
    acc[6] = acc[6] + bf16_lo(v.w);
    acc[7] = acc[7] + bf16_hi(v.w);
}

__device__ __forceinline__ void fma_bf16x8(float *acc, float w, ep_u32x4 v) {
    acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]);
    acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]);
    acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]);
    acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]);
    acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
}

template <int VPL>
__global__ void __launch_bounds__(kBlock) combine_kernel(CombineK a) {
    constexpr int U = kRowsInFlight;
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = gw / a.wpr;
    const int ci = gw - t * a.wpr;
    if (t >= a.T) return;
    const int v0 = ci * VPL * 64;

    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const uint8_t *biases[2] = {a.b0, a.b1};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (!biases[b]) continue;
        const ep_u32x4 *src = (const ep_u32x4 *)(biases[b] + (int64_t)t * a.row_bytes);
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int vi = v0 + i * 64 + lane;
            if (vi < a.nvec) add_bf16x8(acc[i], load_nt(src + vi));
        }
    }

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
            ep_u32x4 v[U][VPL];
            int slot[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                slot[u] = k0 + u < kn ? lane_read(my_slot, k0 + u) : -1;
                if (slot[u] >= 0) {
                    const ep_u32x4 *src = (const ep_u32x4 *)(a.y + (int64_t)slot[u] * a.row_bytes);
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        const int vi = v0 + i * 64 + lane;
                        v[u][i] = vi < a.nvec ? load_nt(src + vi) : ep_u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (slot[u] < 0) continue;
                const float wk = lane_read_f(my_w, k0 + u);
#pragma unroll
                for (int i = 0; i < VPL; ++i) fma_bf16x8(acc[i], wk, v[u][i]);
            }
        }
    }

    ep_u32x4 *dst = (ep_u32x4 *)(a.out + (int64_t)t * a.row_bytes);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int vi = v0 + i * 64 + lane;
        if (vi >= a.nvec) continue;
        ep_u32x4 o;
        o.x = bf16_rne(acc[i][0]) | (bf16_rne(acc[i][1]) << 16);
        o.y = bf16_rne(acc[i][2]) | (bf16_rne(acc[i][3]) << 16);
        o.z = bf16_rne(acc[i][4]) | (bf16_rne(acc[i][5]) << 16);
        o.w = bf16_rne(acc[i][6]) | (bf16_rne(acc[i][7]) << 16);
        store_nt(dst + vi, o);
    }
}

// A partition's partial as it enters the level-two sum.
__device__ __forceinline__ float partial(float p, int to_bf16) {
    return to_bf16 ? __uint_as_float(bf16_rne(p) << 16) : p;
}

// Two-level ("reduced") combine.  The token's kept pairs are put in
// (partition, k) order: each lane ranks its own key against the others and
// ds_permute moves the lane index to the lane named by that rank.  Rows are
// then read in that order, U at a time; a partition's fmaf chain starts at 0
// and is added (rounded to bf16 first with bf16_partials) to the running
// fp32 total, which starts from the biases.  Requires K <= 64.
template <int VPL>
__global__ void __launch_bounds__(kBlock) combine_reduced_kernel(CombineK a) {
    constexpr int U = kRowsInFlight;
    const int lane = __lane_id();
    const int gw = (int)blockIdx.x * kWavesPerBlock + wave_uniform(threadIdx.x >> 6);
    const int t = gw / a.wpr;
    const int ci = gw - t * a.wpr;
    if (t >= a.T) return;
    const int v0 = ci * VPL * 64;

    float acc[VPL][8], part[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[i][j] = 0.0f;
            part[i][j] = 0.0f;
        }
    const uint8_t *biases[2] = {a.b0, a.b1};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (!biases[b]) continue;
        const ep_u32x4 *src = (const ep_u32x4 *)(biases[b] + (int64_t)t * a.row_bytes);
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int vi = v0 + i * 64 + lane;
            if (vi < a.nvec) add_bf16x8(acc[i], load_nt(src + vi));
        }
    }

    int my_slot = -1, my_q = 0;
    float my_w = 1.0f;
    if (lane < a.K) {
        my_slot = a.dst[(int64_t)t * a.K + lane];
        const int64_t e = a.idx[(int64_t)t * a.K + lane];
        if ((int64_t)my_slot >= a.y_rows) {
            atomicOr(a.status, kDevRecvOverflow);
            my_slot = -1;
        }
        if (e < 0 || e >= a.E) my_slot = -1;
        if (my_slot >= 0) {
            my_q = (int)(e / a.m);
            if (a.w) my_w = a.w[(int64_t)t * a.K + lane];
        }
    }
    const int key = my_slot >= 0 ? (my_q << 6) | lane : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < a.K; ++j) rank += lane_read(key, j) < key ? 1 : 0;
    const int nvalid = __popcll(__ballot(my_slot >= 0));
    // lane r receives the index of the lane whose key ranks r
    const int order = __builtin_amdgcn_ds_permute(rank << 2, lane);

    int curq = -1;
    for (int r0 = 0; r0 < nvalid; r0 += U) {
        ep_u32x4 v[U][VPL];
        int slot[U], q[U];
        float wk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            slot[u] = -1;
            q[u] = -1;
            wk[u] = 0.0f;
            if (r0 + u < nvalid) {
                const int src_lane = lane_read(order, r0 + u);
                slot[u] = lane_read(my_slot, src_lane);
                q[u] = lane_read(my_q, src_lane);
                wk[u] = lane_read_f(my_w, src_lane);
                const ep_u32x4 *src = (const ep_u32x4 *)(a.y + (int64_t)slot[u] * a.row_bytes);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int vi = v0 + i * 64 + lane;
                    v[u][i] = vi < a.nvec ? load_nt(src + vi) : ep_u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (slot[u] < 0) continue;
            if (q[u] != curq) {
                if (curq >= 0) {
#pragma unroll
                    for (int i = 0; i < VPL; ++i)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            acc[i][j] = acc[i][j] + partial(part[i][j], a.bf16_partials);
                            part[i][j] = 0.0f;
                        }
                }
                curq = q[u];
            }
#pragma unroll
            for (int i = 0; i < VPL; ++i) fma_bf16x8(part[i], wk[u], v[u][i]);
        }
    }
    if (curq >= 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = acc[i][j] + partial(part[i][j], a.bf16_partials);
    }

    ep_u32x4 *dst = (ep_u32x4 *)(a.out + (int64_t)t * a.row_bytes);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int vi = v0 + i * 64 + lane;
        if (vi >= a.nvec) continue;
        ep_u32x4 o;
        o.x = bf16_rne(acc[i][0]) | (bf16_rne(acc[i][1]) << 16);
        o.y = bf16_rne(acc[i][2]) | (bf16_rne(acc[i][3]) << 16);
        o.z = bf16_rne(acc[i][4]) | (bf16_rne(acc[i][5]) << 16);
        o.w = bf16_rne(acc[i][6]) | (bf16_rne(acc[i][7]) << 16);
        store_nt(dst + vi, o);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &c, hipStream_t stream) {
    CombineK k = {};
    k.y = (const uint8_t *)c.y;
    k.y_rows = c.y_rows;
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
    k.nvec = c.hidden / 8;
    k.row_bytes = c.hidden * 2;
    k.idx = c.topk_idx;
    k.E = c.E;
    k.m = c.m;
    k.bf16_partials = c.bf16_partials;
    k.wpr = (k.nvec + kVpl * 64 - 1) / (kVpl * 64);
    if (k.wpr < 1) k.wpr = 1;
    const int64_t waves = (int64_t)k.T * k.wpr;
    const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (k.idx)
        hipLaunchKernelGGL(combine_reduced_kernel<kVpl>, dim3((unsigned)grid), dim3(kBlock), 0, stream, k);
    else
        hipLaunchKernelGGL(combine_kernel<kVpl>, dim3((unsigned)grid), dim3(kBlock), 0, stream, k);
    return hipGetLastError();
}

}  // namespace ep
