// Layout pass: routing histogram, padded per-expert offsets and the
// source -> destination slot map.
//
// Defines what the DeepEP v2 test page ("DeepEP test target API reference",
// sec. 2.1 dispatch parameters, sec. 3.1 V1 layout tensors, sec. 4.2 align)
// calls the layout derived from topk_idx, with the pairs of one expert kept in
// token-major, then k, order (the scan order of "spark_model/layers/
// ep_dispatch.rs").  Two kernels:
//
//   count  one workgroup per tile of tokens.  Each wave walks its share of
//          the tile's flat (t, k) pairs in 64-pair chunks, in order.  Pairs of
//          one chunk that name the same expert are found with one ballot per
//          bit of the expert id (no atomics, so ranks are deterministic); the
//          lowest lane of each group bumps the wave's LDS counter for that
//          expert.  A per-expert scan over the waves turns wave-local ranks
//          into tile ranks.  Outputs: per-tile counts [tiles, E], per-pair
//          (expert, tile rank) packed into dst_slot, partition membership and
//          per-tile partition counts.
//   slots  one workgroup per tile again.  Each workgroup reduces the
//          [tiles, E] counts column-wise (totals and the prefix of the tiles
//          before its own), scans align(count, A) over experts into offsets,
//          and rewrites its own pairs' packed ranks into receive slots,
//          filling src_of_slot.  Workgroup 0 also publishes the per-expert
//          counts, offsets, partition totals, cumulative stats and status.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

__global__ void __launch_bounds__(1024)
layout_count_kernel(const int64_t *__restrict__ idx, int T, int K, int E, int P, int m,
                    int tile_tokens, int32_t *__restrict__ packed, uint8_t *__restrict__ in_part,
                    int32_t *__restrict__ tile_counts, int32_t *__restrict__ tile_part,
                    int32_t *__restrict__ tile_flags) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_flag;
    const int NW = blockDim.x >> 6;
    int32_t *wcnt = lds;           // [NW][E]
    int32_t *pcnt = lds + NW * E;  // [P]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int tile = blockIdx.x;
    const int t0 = tile * tile_tokens;
    const int t1 = min(T, t0 + tile_tokens);
    const int64_t p0 = (int64_t)t0 * K;
    const int npairs = (t1 - t0) * K;
    const int nchunks = (npairs + 63) >> 6;
    const int cpw = (nchunks + NW - 1) / NW;

    for (int i = tid; i < NW * E; i += blockDim.x) wcnt[i] = 0;
    for (int i = tid; i < P; i += blockDim.x) pcnt[i] = 0;
    if (tid == 0) s_flag = 0;
    __syncthreads();

    const int bits = E > 1 ? 32 - __clz(E - 1) : 0;
    int32_t *mycnt = wcnt + w * E;
    int flag = 0;
    int rank[kMaxChunksPerWave];
    int ex[kMaxChunksPerWave];
#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c) {
        rank[c] = 0;
        ex[c] = -1;
        if (c < cpw) {
            const int p = (w * cpw + c) * 64 + lane;
            int e = -1;
            if (p < npairs) {
                const int64_t v = idx[p0 + p];
                if (v >= 0 && v < E) e = (int)v;
                else if (v != -1) flag = 1;
            }
            const uint64_t active = __ballot(e >= 0);
            uint64_t match = active;
            for (int b = 0; b < bits; ++b) {
                const int bit = (e >> b) & 1;
                const uint64_t ones = __ballot(bit);
                match &= bit ? ones : ~ones;
            }
            const int r = __popcll(match & lanes_below());
            const int n = __popcll(match);
            int leader = __builtin_ffsll((long long)match) - 1;
            leader = leader < 0 ? 0 : leader;
            int old = 0;
            if (e >= 0 && r == 0) {
                old = mycnt[e];
                mycnt[e] = old + n;
            }
            const int base = __shfl(old, leader);
            rank[c] = base + r;
            ex[c] = e;
        }
    }
    __syncthreads();

    // Per-expert exclusive scan over the waves: wave bases inside the tile.
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < NW; ++ww) {
            const int c = wcnt[ww * E + e];
            wcnt[ww * E + e] = run;
            run += c;
        }
        tile_counts[(int64_t)tile * E + e] = run;
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c) {
        if (c < cpw) {
            const int p = (w * cpw + c) * 64 + lane;
            if (p < npairs) {
                const int e = ex[c];
                packed[p0 + p] = e >= 0 ? ((e << kRankBits) | (rank[c] + mycnt[e])) : -1;
            }
        }
    }

    // Partition membership, one thread per token of the tile.
    for (int tt = tid; tt < t1 - t0; tt += blockDim.x) {
        const int64_t t = t0 + tt;
        uint8_t *row = in_part + t * P;
        if (P <= 64) {
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t v = idx[t * K + k];
                if (v >= 0 && v < E) mask |= 1ull << (int)(v / m);
            }
            for (int q = 0; q < P; ++q) row[q] = (uint8_t)((mask >> q) & 1ull);
            while (mask) {
                const int q = __builtin_ffsll((long long)mask) - 1;
                atomicAdd(&pcnt[q], 1);
                mask &= mask - 1;
            }
        } else {
            for (int q = 0; q < P; ++q) {
                int hit = 0;
                for (int k = 0; k < K; ++k) {
                    const int64_t v = idx[t * K + k];
                    hit |= (v >= q * (int64_t)m && v < (q + 1) * (int64_t)m);
                }
                row[q] = (uint8_t)hit;
                if (hit) atomicAdd(&pcnt[q], 1);
            }
        }
    }
    if (flag) atomicOr(&s_flag, kDevBadExpert);
    __syncthreads();
    for (int q = tid; q < P; q += blockDim.x) tile_part[(int64_t)tile * P + q] = pcnt[q];
    if (tid == 0) tile_flags[tile] = s_flag;
}

// Exclusive scan in place over a[0..n) in LDS; every thread of the block
// calls it.  Returns the total.  s_wave needs blockDim/64 + 1 entries.
__device__ int block_exclusive_scan(int32_t *a, int n, int32_t *s_wave) {
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int per = (n + nthreads - 1) / nthreads;
    const int beg = min(n, tid * per);
    const int end = min(n, beg + per);
    int local = 0;
    for (int i = beg; i < end; ++i) local += a[i];
    const int lane = tid & 63;
    const int w = tid >> 6;
    int x = local;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    const int nw = nthreads >> 6;
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < nw; ++i) {
            const int c = s_wave[i];
            s_wave[i] = run;
            run += c;
        }
        s_wave[nw] = run;
    }
    __syncthreads();
    int excl = s_wave[w] + x - local;
    for (int i = beg; i < end; ++i) {
        const int c = a[i];
        a[i] = excl;
        excl += c;
    }
    const int total = s_wave[nw];
    __syncthreads();
    return total;
}

__global__ void __launch_bounds__(1024)
layout_slots_kernel(int T, int K, int E, int A, int P, int C, int tile_tokens, int num_tiles,
                    int64_t max_rows, const int32_t *__restrict__ tile_counts,
                    const int32_t *__restrict__ tile_part, const int32_t *__restrict__ tile_flags,
                    int32_t *__restrict__ count_out, int32_t *__restrict__ offset_out,
                    int32_t *__restrict__ part_out, int32_t *__restrict__ dst,
                    int32_t *__restrict__ src_of_slot, int32_t *__restrict__ status,
                    int32_t *__restrict__ cum_stats) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_wave[17];
    __shared__ int32_t s_flags;
    int32_t *s_tot = lds;               // [E]
    int32_t *s_base = lds + E;          // [E]
    int32_t *s_off = lds + 2 * E;       // [E+1]
    int32_t *s_red = lds + 3 * E + 1;   // [2][G][E] when G > 1
    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int G = E <= (int)blockDim.x ? (int)blockDim.x / E : 1;

    // Column totals over all tiles, and the prefix over tiles before ours.
    if (G > 1) {
        const int g = tid / E;
        const int e = tid - g * E;
        if (g < G) {
            int tot = 0, pre = 0;
            for (int tl = g; tl < num_tiles; tl += G) {
                const int c = tile_counts[(int64_t)tl * E + e];
                tot += c;
                pre += tl < tile ? c : 0;
            }
            s_red[g * E + e] = tot;
            s_red[(G + g) * E + e] = pre;
        }
        __syncthreads();
        for (int e2 = tid; e2 < E; e2 += blockDim.x) {
            int tot = 0, pre = 0;
            for (int g2 = 0; g2 < G; ++g2) {
                tot += s_red[g2 * E + e2];
                pre += s_red[(G + g2) * E + e2];
            }
            s_tot[e2] = tot;
            s_base[e2] = pre;
        }
    } else {
        for (int e = tid; e < E; e += blockDim.x) {
            int tot = 0, pre = 0;
            for (int tl = 0; tl < num_tiles; ++tl) {
                const int c = tile_counts[(int64_t)tl * E + e];
                tot += c;
                pre += tl < tile ? c : 0;
            }
            s_tot[e] = tot;
            s_base[e] = pre;
        }
    }
    __syncthreads();

    // Offsets: exclusive scan of align(count, A), or e*C in fixed mode.
    int R;
    if (C == 0) {
        for (int e = tid; e < E; e += blockDim.x) s_off[e] = (s_tot[e] + A - 1) / A * A;
        __syncthreads();
        R = block_exclusive_scan(s_off, E, s_wave);
        if (tid == 0) s_off[E] = R;
    } else {
        for (int e = tid; e <= E; e += blockDim.x) s_off[e] = e * C;
        R = E * C;
    }
    __syncthreads();

    if (tile == 0) {
        if (tid == 0) s_flags = 0;
        __syncthreads();
        int fl = 0;
        for (int tl = tid; tl < num_tiles; tl += blockDim.x) fl |= tile_flags[tl];
        for (int e = tid; e < E; e += blockDim.x) {
            const int c = s_tot[e];
            count_out[e] = c;
            offset_out[e] = s_off[e];
            if (cum_stats) cum_stats[e] += c;
            if (C > 0 && c > C) fl |= kDevCapacity;
        }
        if (tid == 0) {
            offset_out[E] = R;
            if ((int64_t)R > max_rows) fl |= kDevRecvOverflow;
        }
        for (int q = tid; q < P; q += blockDim.x) {
            int s = 0;
            for (int tl = 0; tl < num_tiles; ++tl) s += tile_part[(int64_t)tl * P + q];
            part_out[q] = s;
        }
        if (fl) atomicOr(&s_flags, fl);
        __syncthreads();
        if (tid == 0) *status = s_flags;
    }

    // Slots of this tile's pairs.
    const int t0 = tile * tile_tokens;
    const int t1 = min(T, t0 + tile_tokens);
    const int64_t p0 = (int64_t)t0 * K;
    const int64_t p1 = (int64_t)t1 * K;
    for (int64_t p = p0 + tid; p < p1; p += blockDim.x) {
        const int v = dst[p];
        if (v < 0) continue;
        const int e = v >> kRankBits;
        const int j = s_base[e] + (v & ((1 << kRankBits) - 1));
        if (C > 0 && j >= C) {
            dst[p] = -1;
            continue;
        }
        const int slot = s_off[e] + j;
        dst[p] = slot;
        if ((int64_t)slot < max_rows) src_of_slot[slot] = (int32_t)p;
    }

    // Padding slots of the experts this workgroup owns (e = tile mod tiles).
    const int owner_step = num_tiles > 0 ? num_tiles : 1;
    for (int e = tile; e < E; e += owner_step) {
        const int c = s_tot[e];
        const int used = C > 0 ? min(c, C) : c;
        const int64_t beg = (int64_t)s_off[e] + used;
        int64_t end = C > 0 ? (int64_t)s_off[e] + C : (int64_t)s_off[e + 1];
        if (end > max_rows) end = max_rows;
        for (int64_t s = beg + tid; s < end; s += blockDim.x) src_of_slot[s] = -1;
    }
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_layout_plan(const ep_layout_params *p, LayoutPlan *plan) {
    LayoutPlan L;
    L.T = p->num_tokens;
    L.K = p->num_topk;
    L.E = p->num_experts;
    L.A = p->expert_alignment;
    L.P = p->num_partitions;
    L.C = p->capacity;
    L.max_rows = p->max_recv_rows;
    int nw = 12288 / L.E;
    nw = nw > 16 ? 16 : (nw < 1 ? 1 : nw);
    L.block = nw * 64;
    const int64_t pairs = (int64_t)L.T * L.K;
    const int64_t target_tile_pairs = (pairs + 31) / 32;
    int64_t cpw = (target_tile_pairs + (int64_t)nw * 64 - 1) / ((int64_t)nw * 64);
    cpw = cpw < 1 ? 1 : (cpw > kMaxChunksPerWave ? kMaxChunksPerWave : cpw);
    L.chunks_per_wave = (int)cpw;
    int tt = (int)((int64_t)nw * 64 * cpw / L.K);
    if (tt < 1) return false;
    L.tile_tokens = tt;
    L.num_tiles = L.T > 0 ? (L.T + tt - 1) / tt : 0;
    const size_t nt = (size_t)(L.num_tiles > 0 ? L.num_tiles : 1);
    L.ws_tile_counts = 0;
    L.ws_tile_part = align256(nt * L.E * 4);
    L.ws_tile_flags = L.ws_tile_part + align256(nt * L.P * 4);
    L.ws_bytes = L.ws_tile_flags + align256(nt * 4);
    *plan = L;
    return true;
}

hipError_t launch_layout(const LayoutPlan &L, const int64_t *topk_idx, const ep_layout *lay,
                         int32_t *cum_stats, void *workspace, hipStream_t stream) {
    char *ws = (char *)workspace;
    int32_t *tile_counts = (int32_t *)(ws + L.ws_tile_counts);
    int32_t *tile_part = (int32_t *)(ws + L.ws_tile_part);
    int32_t *tile_flags = (int32_t *)(ws + L.ws_tile_flags);
    const int m = L.E / L.P;
    if (L.num_tiles > 0) {
        const size_t lds = ((size_t)(L.block / 64) * L.E + L.P) * sizeof(int32_t);
        hipLaunchKernelGGL(layout_count_kernel, dim3(L.num_tiles), dim3(L.block), lds, stream,
                           topk_idx, L.T, L.K, L.E, L.P, m, L.tile_tokens, lay->dst_slot,
                           lay->is_token_in_partition, tile_counts, tile_part, tile_flags);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const int slots_block = 1024;
    const int G = L.E <= slots_block ? slots_block / L.E : 1;
    const size_t lds2 = (size_t)(3 * L.E + 1 + (G > 1 ? 2 * G * L.E : 0)) * sizeof(int32_t);
    const int grid2 = L.num_tiles > 0 ? L.num_tiles : 1;
    hipLaunchKernelGGL(layout_slots_kernel, dim3(grid2), dim3(slots_block), lds2, stream, L.T, L.K,
                       L.E, L.A, L.P, L.C, L.tile_tokens, L.num_tiles, L.max_rows, tile_counts,
                       tile_part, tile_flags, lay->num_tokens_per_expert, lay->expert_offset,
                       lay->num_tokens_per_partition, lay->dst_slot, lay->src_of_slot, lay->status,
                       cum_stats);
    return hipGetLastError();
}

}  // namespace ep
