// Layout pass: routing histogram, padded per-expert offsets and the
// source -> destination slot map.  "Expert" below stands for the receive
// segment: the expert itself, or with partition_major its partition (the
// pair's expert id divided by E/P).  Partitions stand for the ranks of
// "DeepEP test target API reference" sec. 3.1 (per-rank layout tensors), and
// the multi-level combine of sec. 2.2 reduces rank by rank; a receive buffer
// grouped by partition is that rank-major order.
//
// Computes what the DeepEP v2 test page ("DeepEP test target API reference",
// sec. 2.1 dispatch parameters, sec. 3.1 V1 layout tensors, sec. 4.2 align)
// describes as the layout derived from topk_idx, with the pairs of one expert
// kept in token-major, then k, order (the scan order of "spark_model/layers/
// ep_dispatch.rs").  Two phases over tiles of consecutive tokens:
//
//   count  each wave walks its share of the tile's flat (t, k) pairs in
//          64-pair chunks, in order.  Pairs of one chunk that name the same
//          expert are found with one ballot per bit of the expert id (no
//          atomics, so ranks are deterministic); the lowest lane of each group
//          bumps the wave's LDS counter for that expert.  A per-expert scan
//          over the waves turns wave-local ranks into tile ranks.  Outputs:
//          partition membership and one row per tile of [E expert counts |
//          P partition token counts | bad-id flag]; each pair's (expert, tile
//          rank) stays with the thread that found it.
//   slots  each tile reduces the per-tile rows column-wise (totals and the
//          prefix over the tiles before it) in one pass, scans align(count, A) over
//          experts into offsets, and turns its pairs' ranks into receive
//          slots, filling src_of_slot.  Designated tiles also publish the
//          per-expert counts and offsets, the partition totals, the
//          cumulative stats and the status word.
//
// The phases run as two kernels, the pair ranks travelling through the
// workspace packed as (e << kRankBits) | rank; above kPrescanTiles tiles a
// third kernel between them scans the tile rows once.  A very small batch
// (a few hundred pairs) runs both phases in one 1024-thread workgroup, one
// launch, with only a workgroup barrier between them and the ranks kept in
// registers.  A dispatch that derives its own layout runs the count kernel
// alone: the dispatch kernels then do the slots phase themselves from the
// tile rows and the packed ranks.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

// Count workgroups of the two-kernel tiling: 16 waves, one 64-pair chunk
// each at the prefill shape (1.1 µs faster than 4 waves of four chunks),
// while their per-wave expert counters fit LDS easily; 4 waves above that.
constexpr int kCountBlock = 1024;
constexpr int kCountBlockLargeE = 256;
constexpr int kCountBlockMaxE = 1024;
constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS one workgroup may allocate on gfx950
constexpr int kSlotsBlock = 1024;  // slots workgroup, and the one-workgroup batch: 16 waves
constexpr int kReduceBatch = 8;    // loads in flight per thread in column_sums
constexpr int kMaxSingleExperts = 512;
constexpr int64_t kSinglePairs = 256;   // batches up to this many pairs: one workgroup
constexpr int kPrescanTiles = 96;  // above this many tiles: scan the tile rows once first
constexpr int kScanBlock = 256;       // scan kernel: one workgroup per 4 columns
constexpr int kScanMaxRowsPerThread = 8;
// Tiles the count aims for (at most 4 chunks per wave).  32 measured best for
// a dispatch that derives its layout (its workgroups hold the tile rows in
// LDS: 64 tiles took 4.7 µs longer at the prefill shape, 128 did not fit
// twice per CU) and no worse for the layout alone (two kernels, no scan).
constexpr int kTargetTiles = 32;
constexpr int kRedInts = 2 * 4 * kSlotsBlock;

struct CountArgs {
    const int64_t *idx;
    int T, K, E, P, m;      // E: receive segments; m: experts per partition
    int E_ids;              // ids are valid in [0, E_ids)
    int seg_div;            // segment of an id: id / seg_div
    int tile_tokens;
    int tile_pairs_max;
    int G, NG;              // partitions per group, groups
    uint8_t *in_part;
    int32_t *tile_counts;   // [tiles, W]: E expert counts | P partition counts |
                            //             NG group counts | bad-id flag
    int W;                  // row stride of tile_counts, a multiple of 4
    uint64_t *tok_mask;     // [T] partition bit mask per token (P <= 64), or NULL
    int32_t *packed;        // [T*K] (e << kRankBits) | tile rank, or -1
    uint32_t *zero_words;   // words workgroup 0 sets to zero (the dispatch's token-queue
    int n_zero;             //   counters, the status word of a counts-only launch)
    int32_t *status_zero;
};

struct SlotsArgs {
    int T, K, E, A, P, C;
    int tile_tokens;
    int num_tiles;
    int64_t max_rows;
    const int32_t *tile_counts;
    int W;
    int NG;
    const uint64_t *tok_mask;
    int32_t *part_offset_out;   // [P+1] or NULL
    int32_t *token_slot_out;    // [T*P] or NULL
    int32_t *part_src_out;      // [T*P] token of each partition row, or NULL (needs token_slot)
    int32_t *group_out;         // [NG] or NULL
    int32_t *count_out;
    int32_t *offset_out;
    int32_t *part_out;
    int32_t *dst;
    int32_t *src_of_slot;
    int32_t *status;
    int32_t *cum_stats;
    const int32_t *packed;
    int prescanned;             // tile_counts holds exclusive prefixes and, at row
                                // num_tiles, the totals
};

// Count phase for tile blockIdx.x.  LDS: [waves][E] counters (one per
// receive segment), [tile pairs] expert ids, [P] partition counters.  On
// return rank[c] / ex[c] hold the tile rank and segment of pair
// (wave * cpw + c) * 64 + lane (ex = -1: none).
__device__ void count_phase(const CountArgs &a, int32_t *lds, int32_t *s_flag,
                            int rank[kMaxChunksPerWave], int ex[kMaxChunksPerWave], int &cpw) {
    const int nw = blockDim.x >> 6;
    const int E = a.E;
    int32_t *wcnt = lds;                   // [nw][E]
    int32_t *pe = lds + nw * E;            // [tile pairs]
    int32_t *pcnt = pe + a.tile_pairs_max; // [P] then [NG]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int tile = blockIdx.x;
    const int t0 = tile * a.tile_tokens;
    const int t1 = min(a.T, t0 + a.tile_tokens);
    const int64_t p0 = (int64_t)t0 * a.K;
    const int npairs = (t1 - t0) * a.K;
    const int nchunks = (npairs + 63) >> 6;
    cpw = (nchunks + nw - 1) / nw;

    // Issue every routing load of this wave before touching LDS.
    int64_t raw[kMaxChunksPerWave];
#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c) {
        const int p = (w * cpw + c) * 64 + lane;
        raw[c] = (c < cpw && p < npairs) ? a.idx[p0 + p] : -1;
    }
    for (int i = tid; i < nw * E; i += blockDim.x) wcnt[i] = 0;
    for (int i = tid; i < a.P + a.NG; i += blockDim.x) pcnt[i] = 0;
    if (tid == 0) *s_flag = 0;
    __syncthreads();

    const int bits = E > 1 ? 32 - __clz(E - 1) : 0;
    int32_t *mycnt = wcnt + w * E;
    int flag = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c) {
        rank[c] = 0;
        ex[c] = -1;
        if (c < cpw) {
            const int p = (w * cpw + c) * 64 + lane;
            const int64_t v = raw[c];
            int id = -1;
            if (v >= 0 && v < a.E_ids) id = (int)v;
            else if (v != -1) flag = 1;
            if (p < npairs) pe[p] = id;   // the expert id, for partition membership
            // the pair's receive segment: its expert, or its partition
            const int e = id < 0 ? -1 : (a.seg_div == 1 ? id : id / a.seg_div);
            // Lanes naming the same expert: intersect one ballot per id bit.
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
            rank[c] = __shfl(old, leader) + r;
            ex[c] = e;
        }
    }
    __syncthreads();

    // Per-expert exclusive scan over the waves: wave bases inside the tile.
    int32_t *row_out = a.tile_counts + (int64_t)tile * a.W;
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < nw; ++ww) {
            const int c = wcnt[ww * E + e];
            wcnt[ww * E + e] = run;
            run += c;
        }
        row_out[e] = run;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c)
        if (c < cpw && ex[c] >= 0) rank[c] += mycnt[ex[c]];

    // Partition and group membership, one thread per token, from the ids
    // staged in LDS.  Group n is partitions [n*G, (n+1)*G).
    const int K = a.K, P = a.P, m = a.m, G = a.G, NG = a.NG;
    int32_t *gcnt = pcnt + P;
    for (int tt = tid; tt < t1 - t0; tt += blockDim.x) {
        uint8_t *row = a.in_part + (int64_t)(t0 + tt) * P;
        const int32_t *ids = pe + tt * K;
        if (P <= 64) {
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int e = ids[k];
                if (e >= 0) mask |= 1ull << (e / m);
            }
            for (int q = 0; q < P; ++q) row[q] = (uint8_t)((mask >> q) & 1ull);
            if (a.tok_mask) a.tok_mask[t0 + tt] = mask;
            const uint64_t gm = G == 64 ? ~0ull : ((1ull << G) - 1);
            for (int n = 0; n < NG; ++n)
                if ((mask >> (n * G)) & gm) atomicAdd(&gcnt[n], 1);
            while (mask) {
                const int q = __builtin_ffsll((long long)mask) - 1;
                atomicAdd(&pcnt[q], 1);
                mask &= mask - 1;
            }
        } else {
            int ghit = -1;   // last group counted for this token
            for (int q = 0; q < P; ++q) {
                int hit = 0;
                for (int k = 0; k < K; ++k) hit |= (ids[k] >= 0 && ids[k] / m == q);
                row[q] = (uint8_t)hit;
                if (hit) {
                    atomicAdd(&pcnt[q], 1);
                    if (q / G != ghit) {
                        ghit = q / G;
                        atomicAdd(&gcnt[ghit], 1);
                    }
                }
            }
        }
    }
    if (flag) atomicOr(s_flag, 1);
    __syncthreads();
    for (int q = tid; q < P + NG; q += blockDim.x) row_out[E + q] = pcnt[q];
    for (int c = E + P + NG + tid; c < a.W; c += blockDim.x)
        row_out[c] = c == E + P + NG ? *s_flag : 0;
}

// Column sums of a row-major [rows, cols] int32 matrix in global memory:
// tot[c] = sum over all rows, pre[c] = sum over rows < my_row (both LDS).
// Threads split the columns (4 at a time when cols % 4 == 0) and stride over
// the rows in batches of kReduceBatch independent loads, so the whole matrix
// is requested in a few round trips; at most 16 partials per column are
// combined through red (LDS, kRedInts ints).  Ends with a barrier.
__device__ void column_sums(const int32_t *__restrict__ mat, int rows, int cols, int my_row,
                            int32_t *tot, int32_t *pre, int32_t *red) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int vec = (cols & 3) == 0 ? 4 : 1;
    const int Q = cols / vec;                           // column groups
    const int G = Q <= nt ? min(nt / Q, 16) : 1;        // row strides (partials per column)
    for (int q0 = 0; q0 < Q; q0 += nt) {
        const int span = Q <= nt ? Q : nt;
        const int g = tid / span;
        const int q = q0 + tid - g * span;
        int at[4] = {0, 0, 0, 0}, ap[4] = {0, 0, 0, 0};
        if (g < G && q < Q) {
            for (int r0 = g; r0 < rows; r0 += G * kReduceBatch) {
                int v[kReduceBatch][4];
#pragma unroll
                for (int u = 0; u < kReduceBatch; ++u) {
                    const int r = r0 + u * G;
                    if (r < rows) {
                        const int32_t *src = mat + (int64_t)r * cols + q * vec;
                        if (vec == 4) {
                            const ep_u32x4 x = *(const ep_u32x4 *)src;
                            v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
                        } else {
                            v[u][0] = src[0]; v[u][1] = v[u][2] = v[u][3] = 0;
                        }
                    } else {
                        v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0;
                    }
                }
#pragma unroll
                for (int u = 0; u < kReduceBatch; ++u) {
                    const int r = r0 + u * G;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        at[j] += v[u][j];
                        ap[j] += r < my_row ? v[u][j] : 0;
                    }
                }
            }
        }
        if (G > 1) {
            if (g < G && q < Q)
                for (int j = 0; j < vec; ++j) {
                    red[g * cols + q * vec + j] = at[j];
                    red[(G + g) * cols + q * vec + j] = ap[j];
                }
            __syncthreads();
            for (int c = tid; c < cols; c += nt) {
                int s = 0, sp = 0;
                for (int g2 = 0; g2 < G; ++g2) {
                    s += red[g2 * cols + c];
                    sp += red[(G + g2) * cols + c];
                }
                tot[c] = s;
                pre[c] = sp;
            }
        } else if (g < G && q < Q) {
            // one partial per column: only the threads that summed it write
            // (with Q in (nt/2, nt] the threads past the first span hold none)
            for (int j = 0; j < vec; ++j) {
                tot[q * vec + j] = at[j];
                pre[q * vec + j] = ap[j];
            }
        }
    }
    __syncthreads();
}

// Slots phase for tile blockIdx.x (blockDim == kSlotsBlock).  pv[i] holds a
// packed (e << kRankBits) | tile rank (or -1) for flat pair pidx[i] (or -1).
// The tiles that publish results are distinct where possible, so their extra
// global reads overlap instead of queueing in one workgroup.
__device__ void slots_phase(const SlotsArgs &a, int32_t *lds, int32_t *s_flags,
                            const int pv[4], const int64_t pidx[4]) {
    const int E = a.E, P = a.P, C = a.C, A = a.A, W = a.W;
    const int NG = a.NG;
    int32_t *s_tot = lds;                    // [W]  column totals
    int32_t *s_base = s_tot + W;             // [W]  totals over the tiles before this one
    int32_t *s_off = s_base + W;             // [E+1]
    int32_t *s_poff = s_off + E + 1;         // [P+1] partition offsets
    int32_t *s_wq = s_poff + P + 1;          // [waves][P] per-wave partition token counts,
                                             // only with token_slot (P <= 64)
    int32_t *s_red = s_wq + (blockDim.x >> 6) * (a.token_slot_out ? P : 0);   // [kRedInts]
    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int nt = a.num_tiles > 0 ? a.num_tiles : 1;
    const bool pub_counts = tile == 0;
    const bool pub_status = tile == 1 % nt;
    const bool pub_stats = tile == 2 % nt;

    // This tile's token masks for the partition layout: requested first.
    const bool want_tok = a.token_slot_out != nullptr;
    const int t0 = tile * a.tile_tokens;
    const int ntok = a.num_tiles > 0 ? min(a.T, t0 + a.tile_tokens) - t0 : 0;
    uint64_t tmask = 0;
    if (want_tok && tid < ntok) tmask = a.tok_mask[t0 + tid];

    if (a.prescanned) {
        const int32_t *base = a.tile_counts + (int64_t)tile * W;
        const int32_t *tot = a.tile_counts + (int64_t)a.num_tiles * W;
        for (int c = tid; c < W; c += blockDim.x) {
            s_base[c] = base[c];
            s_tot[c] = tot[c];
        }
        __syncthreads();
    } else {
        column_sums(a.tile_counts, a.num_tiles, W, tile, s_tot, s_base, s_red);
    }

    int R;
    if (C == 0) {
        for (int e = tid; e < E; e += blockDim.x) s_off[e] = (s_tot[e] + A - 1) / A * A;
        __syncthreads();
        if (tid < 64) {
            const int total = wave_exclusive_scan(s_off, E);
            if (tid == 0) s_off[E] = total;
        }
    } else {
        for (int e = tid; e <= E; e += blockDim.x) s_off[e] = e * C;
    }
    if ((want_tok || a.part_offset_out) && tid >= 64 && tid < 128) {
        // a second wave scans the partition token counts meanwhile
        for (int q = tid - 64; q < P; q += 64) s_poff[q] = s_tot[E + q];
    }
    __syncthreads();
    R = s_off[E];
    if ((want_tok || a.part_offset_out) && tid < 64) {
        const int total = wave_exclusive_scan(s_poff, P);
        if (tid == 0) s_poff[P] = total;
    }

    if (pub_counts) {
        for (int e = tid; e < E; e += blockDim.x) {
            a.count_out[e] = s_tot[e];
            a.offset_out[e] = s_off[e];
        }
        for (int q = tid; q < P; q += blockDim.x) a.part_out[q] = s_tot[E + q];
        if (a.group_out)
            for (int n = tid; n < NG; n += blockDim.x) a.group_out[n] = s_tot[E + P + n];
        if (tid == 0) a.offset_out[E] = R;
    }
    if (pub_stats && a.cum_stats)
        for (int e = tid; e < E; e += blockDim.x) a.cum_stats[e] += s_tot[e];
    if (pub_status) {
        if (tid == 0) *s_flags = s_tot[E + P + NG] > 0 ? kDevBadExpert : 0;
        __syncthreads();
        int fl = 0;
        for (int e = tid; e < E; e += blockDim.x)
            if (C > 0 && s_tot[e] > C) fl |= kDevCapacity;
        if (tid == 0 && (int64_t)R > a.max_rows) fl |= kDevRecvOverflow;
        if (fl) atomicOr(s_flags, fl);
        __syncthreads();
        if (tid == 0) *a.status = *s_flags;
    }

    // Partition layout: a token's row in partition q is the partition's
    // offset + tokens of q in earlier tiles + earlier waves + earlier lanes.
    if (want_tok || a.part_offset_out) {
        __syncthreads();   // s_poff complete
        if (pub_counts && a.part_offset_out)
            for (int q = tid; q <= P; q += blockDim.x) a.part_offset_out[q] = s_poff[q];
    }
    if (want_tok) {
        const int lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
        // per-wave token counts of each partition (lanes past the tile have
        // an empty mask, so they vote 0)
        for (int q = 0; q < P; ++q) {
            const uint64_t b = __ballot((tmask >> q) & 1ull);
            if (lane == 0) s_wq[w * P + q] = __popcll(b);
        }
        __syncthreads();
        for (int q = tid; q < P; q += blockDim.x) {
            int run = 0;
            for (int ww = 0; ww < nw; ++ww) {
                const int c = s_wq[ww * P + q];
                s_wq[ww * P + q] = run;
                run += c;
            }
        }
        __syncthreads();
        int32_t *row = a.token_slot_out + (int64_t)(t0 + tid) * P;
        for (int q = 0; q < P; ++q) {
            const int bit = (int)((tmask >> q) & 1ull);
            const uint64_t b = __ballot(bit);
            const int rank = __popcll(b & lanes_below());
            const int slot = s_poff[q] + s_base[E + q] + s_wq[w * P + q] + rank;
            if (tid < ntok) row[q] = bit ? slot : -1;
            // the inverse map: a wave's tokens of one partition take consecutive rows
            if (tid < ntok && bit && a.part_src_out) a.part_src_out[slot] = t0 + tid;
        }
    }

    // Slots of this tile's pairs.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = pv[i];
        const int64_t p = pidx[i];
        if (p < 0) continue;
        if (v < 0) {
            a.dst[p] = -1;
            continue;
        }
        const int e = v >> kRankBits;
        const int j = s_base[e] + (v & ((1 << kRankBits) - 1));
        if (C > 0 && j >= C) {
            a.dst[p] = -1;
            continue;
        }
        const int slot = s_off[e] + j;
        a.dst[p] = slot;
        if ((int64_t)slot < a.max_rows) a.src_of_slot[slot] = (int32_t)p;
    }

    // Padding slots of the experts this workgroup owns (e = tile mod tiles),
    // one expert per wave at a time: an expert's padding is at most
    // max(A - 1, C) rows, so whole-block passes would leave most lanes idle.
    {
        const int lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
        for (int e = tile + w * nt; e < E; e += nt * nw) {
            const int c = s_tot[e];
            const int used = C > 0 ? min(c, C) : c;
            const int64_t beg = (int64_t)s_off[e] + used;
            int64_t end = C > 0 ? (int64_t)s_off[e] + C : (int64_t)s_off[e + 1];
            if (end > a.max_rows) end = a.max_rows;
            for (int64_t s = beg + lane; s < end; s += 64) a.src_of_slot[s] = -1;
        }
    }
}

// Many tiles: each column of the [tiles, W] count rows scanned once.  A
// workgroup owns four adjacent columns; thread i takes a run of consecutive
// tiles, sums it, the runs' sums are scanned across the workgroup (wave
// scans by shuffles, then the four wave totals), and every row is rewritten
// with the exclusive prefix of the tiles before it; the totals go to row
// `tiles`.  The slots kernel then reads two rows per tile instead of
// reducing the whole matrix in every tile.
__global__ void __launch_bounds__(kScanBlock) layout_scan_kernel(int32_t *mat, int tiles, int W) {
    __shared__ ep_u32x4 s_wave[kScanBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = blockIdx.x;                       // column group
    const int per = (tiles + kScanBlock - 1) / kScanBlock;
    const int r0 = tid * per;
    ep_u32x4 *col = (ep_u32x4 *)(mat + 4 * q);
    const int64_t stride = W / 4;                   // row stride in 16-byte vectors
    ep_u32x4 v[kScanMaxRowsPerThread];
    ep_u32x4 sum = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kScanMaxRowsPerThread; ++i) {
        v[i] = ep_u32x4{0u, 0u, 0u, 0u};
        if (i < per && r0 + i < tiles) v[i] = col[(int64_t)(r0 + i) * stride];
        sum += v[i];
    }
    // inclusive scan of the run sums within the wave, then across waves
    ep_u32x4 inc = sum;
    for (int o = 1; o < 64; o <<= 1) {
        ep_u32x4 up;
        up.x = __shfl_up(inc.x, o);
        up.y = __shfl_up(inc.y, o);
        up.z = __shfl_up(inc.z, o);
        up.w = __shfl_up(inc.w, o);
        if (lane >= o) inc += up;
    }
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    ep_u32x4 run = inc - sum;                       // exclusive within the wave
    for (int ww = 0; ww < w; ++ww) run += s_wave[ww];
#pragma unroll
    for (int i = 0; i < kScanMaxRowsPerThread; ++i) {
        if (i < per && r0 + i < tiles) {
            col[(int64_t)(r0 + i) * stride] = run;
            run += v[i];
        }
    }
    if (tid == kScanBlock - 1) {
        ep_u32x4 tot = {0u, 0u, 0u, 0u};
        for (int ww = 0; ww < kScanBlock / 64; ++ww) tot += s_wave[ww];
        col[(int64_t)tiles * stride] = tot;
    }
}

__global__ void __launch_bounds__(kSlotsBlock) layout_count_kernel(CountArgs a) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_flag;
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < a.n_zero; i += blockDim.x) a.zero_words[i] = 0u;
        if (a.status_zero && threadIdx.x == 0) *a.status_zero = 0;
    }
    int rank[kMaxChunksPerWave], ex[kMaxChunksPerWave], cpw;
    count_phase(a, lds, &s_flag, rank, ex, cpw);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int t0 = blockIdx.x * a.tile_tokens;
    const int npairs = (min(a.T, t0 + a.tile_tokens) - t0) * a.K;
    const int64_t p0 = (int64_t)t0 * a.K;
#pragma unroll
    for (int c = 0; c < kMaxChunksPerWave; ++c) {
        const int p = (w * cpw + c) * 64 + lane;
        if (c < cpw && p < npairs)
            a.packed[p0 + p] = ex[c] >= 0 ? ((ex[c] << kRankBits) | rank[c]) : -1;
    }
}

__global__ void __launch_bounds__(kSlotsBlock) layout_slots_kernel(SlotsArgs a) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_flags;
    const int t0 = blockIdx.x * a.tile_tokens;
    const int64_t p0 = (int64_t)t0 * a.K;
    const int npairs = a.num_tiles > 0 ? (min(a.T, t0 + a.tile_tokens) - t0) * a.K : 0;
    int pv[4];
    int64_t pidx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = threadIdx.x + i * kSlotsBlock;
        pidx[i] = p < npairs ? p0 + p : -1;
        pv[i] = p < npairs ? a.packed[p0 + p] : -1;
    }
    slots_phase(a, lds, &s_flags, pv, pidx);
}

// The whole layout of a batch that is one tile: both phases in one
// workgroup, the ranks kept in registers between them.
__global__ void __launch_bounds__(kSlotsBlock) layout_single_kernel(CountArgs ca, SlotsArgs sa) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_flag;
    for (int i = threadIdx.x; i < ca.n_zero; i += blockDim.x) ca.zero_words[i] = 0u;
    int rank[kMaxChunksPerWave], ex[kMaxChunksPerWave], cpw;
    count_phase(ca, lds, &s_flag, rank, ex, cpw);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int npairs = ca.T * ca.K;
    int pv[4];
    int64_t pidx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int p = (w * cpw + c) * 64 + lane;
        const bool ok = c < cpw && p < npairs;
        pidx[c] = ok ? p : -1;
        pv[c] = ok && ex[c] >= 0 ? ((ex[c] << kRankBits) | rank[c]) : -1;
    }
    __syncthreads();   // the workgroup reads back its own tile row
    slots_phase(sa, lds, &s_flag, pv, pidx);
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_layout_plan(const ep_layout_params *p, LayoutPlan *plan) {
    LayoutPlan L;
    L.T = p->num_tokens;
    L.K = p->num_topk;
    L.E_ids = p->num_experts;
    L.seg_div = p->partition_major ? p->num_experts / p->num_partitions : 1;
    L.E = p->num_experts / L.seg_div;   // receive segments
    L.A = p->expert_alignment;
    L.P = p->num_partitions;
    L.C = p->capacity;
    L.max_rows = p->max_recv_rows;
    const int64_t pairs = (int64_t)L.T * L.K;
    // A batch of at most kSinglePairs pairs is one tile: both phases run in
    // one workgroup, in one launch.  (Measured: 12.3 -> 11.1 µs at 128 pairs;
    // already slower than the two kernels at 1,024 pairs, 13.1 -> 15.6 µs.)
    L.single = pairs > 0 && L.E <= kMaxSingleExperts && pairs <= kSinglePairs && L.T <= kSlotsBlock;
    L.block = L.single ? kSlotsBlock : (L.E <= kCountBlockMaxE ? kCountBlock : kCountBlockLargeE);
    const int64_t per_round = L.block;   // pairs when every wave takes one 64-pair chunk
    // Chunks per wave: enough tiles to spread the count over the chip, few
    // enough that each slots workgroup reduces the [tiles, W] count rows in
    // one or two round trips (and that a dispatch can hold them in LDS).
    const int64_t target_tiles = L.single ? 1 : kTargetTiles;
    int64_t cpw = (pairs + target_tiles * per_round - 1) / (target_tiles * per_round);
    cpw = cpw < 1 ? 1 : (cpw > kMaxChunksPerWave ? kMaxChunksPerWave : cpw);
    L.chunks_per_wave = (int)cpw;
    int tt = (int)(per_round * cpw / L.K);
    if (tt > kSlotsBlock) tt = kSlotsBlock;   // one slots thread per token of a tile
    if (tt < 1) return false;
    L.tile_tokens = tt;
    L.num_tiles = L.T > 0 ? (L.T + tt - 1) / tt : 0;
    L.single = L.single && L.num_tiles == 1;
    L.prescan = !L.single && L.num_tiles > kPrescanTiles &&
                L.num_tiles <= kScanBlock * kScanMaxRowsPerThread;
    const size_t nt = (size_t)(L.num_tiles > 0 ? L.num_tiles : 1);
    L.G = p->partitions_per_group > 0 ? p->partitions_per_group : L.P;
    L.NG = L.P / L.G;
    L.row_stride = (L.E + L.P + L.NG + 1 + 3) & ~3;
    L.ws_queue = 0;
    L.ws_rows = kQueueBytes;
    L.ws_packed = L.ws_rows + align256((nt + 1) * L.row_stride * 4);   // + a totals row for the scan
    L.ws_tok_mask = L.ws_packed + align256((size_t)(pairs > 0 ? pairs : 1) * 4);
    L.ws_bytes = L.ws_tok_mask + align256((size_t)(L.T > 0 ? L.T : 1) * 8);
    *plan = L;
    return true;
}

hipError_t launch_layout(const LayoutPlan &L, const int64_t *topk_idx, const ep_layout *lay,
                         int32_t *cum_stats, void *workspace, hipStream_t stream,
                         bool counts_only) {
    char *ws = (char *)workspace;
    CountArgs ca;
    ca.idx = topk_idx;
    ca.T = L.T;
    ca.K = L.K;
    ca.E = L.E;
    ca.E_ids = L.E_ids;
    ca.seg_div = L.seg_div;
    ca.P = L.P;
    ca.m = L.E_ids / L.P;
    ca.tile_tokens = L.tile_tokens;
    ca.tile_pairs_max = L.tile_tokens * L.K;
    ca.in_part = lay->is_token_in_partition;
    ca.tile_counts = (int32_t *)(ws + L.ws_rows);
    ca.W = L.row_stride;
    ca.G = L.G;
    ca.NG = L.NG;
    const bool want_part = lay->token_slot != nullptr || lay->partition_offset != nullptr;
    ca.tok_mask = (want_part && L.P <= 64) ? (uint64_t *)(ws + L.ws_tok_mask) : nullptr;
    ca.packed = (int32_t *)(ws + L.ws_packed);
    // the count kernel clears the dispatch's token queue, and in a
    // counts-only launch the status word (the dispatch then ORs its bits in)
    ca.zero_words = (uint32_t *)(ws + L.ws_queue);
    ca.n_zero = (int)(kQueueBytes / 4);
    ca.status_zero = counts_only ? lay->status : nullptr;
    SlotsArgs sa;
    sa.T = L.T;
    sa.K = L.K;
    sa.E = L.E;
    sa.A = L.A;
    sa.P = L.P;
    sa.C = L.C;
    sa.tile_tokens = L.tile_tokens;
    sa.num_tiles = L.num_tiles;
    sa.max_rows = L.max_rows;
    sa.tile_counts = ca.tile_counts;
    sa.W = L.row_stride;
    sa.NG = L.NG;
    sa.tok_mask = ca.tok_mask;
    sa.part_offset_out = lay->partition_offset;
    sa.token_slot_out = lay->token_slot;
    sa.part_src_out = lay->token_slot ? lay->partition_src : nullptr;
    sa.group_out = lay->num_tokens_per_group;
    sa.count_out = lay->num_tokens_per_expert;
    sa.offset_out = lay->expert_offset;
    sa.part_out = lay->num_tokens_per_partition;
    sa.dst = lay->dst_slot;
    sa.src_of_slot = lay->src_of_slot;
    sa.status = lay->status;
    sa.cum_stats = cum_stats;
    sa.packed = ca.packed;
    sa.prescanned = L.prescan ? 1 : 0;

    const size_t lds_count =
        ((size_t)(L.block / 64) * L.E + ca.tile_pairs_max + L.P + L.NG) * 4;
    const size_t lds_slots = ((size_t)2 * L.row_stride + L.E + 1 + L.P + 1 +
                              (size_t)(kSlotsBlock / 64) * (lay->token_slot ? L.P : 0) + kRedInts) * 4;
    if (lds_count > kMaxLdsBytes || lds_slots > kMaxLdsBytes) return hipErrorInvalidConfiguration;

    if (L.single) {
        const size_t lds = lds_count > lds_slots ? lds_count : lds_slots;
        hipLaunchKernelGGL(layout_single_kernel, dim3(1), dim3(kSlotsBlock), lds, stream, ca, sa);
        return hipGetLastError();
    }
    if (L.num_tiles > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3(L.num_tiles), dim3(L.block), lds_count, stream,
                           ca);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || counts_only) return err;
        if (L.prescan) {
            hipLaunchKernelGGL(layout_scan_kernel, dim3(L.row_stride / 4), dim3(kScanBlock), 0, stream,
                               ca.tile_counts, L.num_tiles, L.row_stride);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    hipLaunchKernelGGL(layout_slots_kernel, dim3(L.num_tiles > 0 ? L.num_tiles : 1),
                       dim3(kSlotsBlock), lds_slots, stream, sa);
    return hipGetLastError();
}

bool fresh_layout_of(const LayoutPlan &L, const ep_layout *lay, int32_t *cum_stats, void *workspace,
                     FreshLayout *f) {
    // one tile: the single kernel writes the slots itself; no tiles: nothing
    // to derive; the partition layout needs the slots kernel; and the tile
    // rows must fit a dispatch workgroup's LDS
    if (L.single || L.num_tiles == 0 || lay->token_slot || lay->partition_offset) return false;
    const size_t lds = fresh_lds_bytes(L.num_tiles, L.row_stride, L.E);
    if (lds > kFreshLdsMax) return false;
    char *ws = (char *)workspace;
    f->packed = (const int32_t *)(ws + L.ws_packed);
    f->rows = (const int32_t *)(ws + L.ws_rows);
    f->W = L.row_stride;
    f->tile_tokens = L.tile_tokens;
    f->num_tiles = L.num_tiles;
    f->A = L.A;
    f->P = L.P;
    f->NG = L.NG;
    f->lds_bytes = lds;
    f->dst_out = lay->dst_slot;
    f->src_out = lay->src_of_slot;
    f->max_rows = L.max_rows;
    f->count_out = lay->num_tokens_per_expert;
    f->offset_out = lay->expert_offset;
    f->part_out = lay->num_tokens_per_partition;
    f->group_out = lay->num_tokens_per_group;
    f->cum_stats = cum_stats;
    return true;
}

uint32_t *queue_of(const LayoutPlan &L, void *workspace) {
    return (uint32_t *)((char *)workspace + L.ws_queue);
}

}  // namespace ep
