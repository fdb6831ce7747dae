// Host-side launchers shared between the kernel files and the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

// Token-queue counters in the layout workspace: 8 of them, 256 bytes apart.
constexpr size_t kQueueBytes = 8 * 256;

// Tiling of the layout pass, chosen on the host from the shapes alone.
struct LayoutPlan {
    int T, K, E, A, P, C;   // E: receive segments (experts, or partitions when partition-major)
    int E_ids;              // expert ids are valid in [0, E_ids)
    int seg_div;            // an expert's segment is id / seg_div (1, or E_ids / P)
    int64_t max_rows;
    int tile_tokens;   // tokens per count tile (one workgroup)
    int num_tiles;     // ceil(T / tile_tokens)
    int block;         // threads per count workgroup (multiple of 64)
    bool single;       // the whole batch is one tile: count and slots in one workgroup
    bool prescan;      // many tiles: a scan kernel turns the tile rows into prefixes first
    int chunks_per_wave;
    int G, NG;              // partitions per group, number of groups
    int row_stride;         // ints per tile row: E + P + NG + 1 rounded up to 4 (E segments)
    size_t ws_queue;        // byte offsets inside the workspace: the dispatch's token queue,
    size_t ws_rows;         //   [tiles + 1, row_stride] count rows,
    size_t ws_packed;       //   [T*K] (expert << 12) | rank in tile,
    size_t ws_tok_mask;     //   [T] partition masks
    size_t ws_bytes;
};

bool make_layout_plan(const ep_layout_params *p, LayoutPlan *plan);

// The whole layout (count, scan and slots kernels); the count kernel also
// clears the dispatch's token-queue counters.  With counts_only only the
// count kernel runs (and clears layout->status too):
// the dispatch kernels then derive the slots themselves (DispatchArgs::fresh).
hipError_t launch_layout(const LayoutPlan &plan, const int64_t *topk_idx, const ep_layout *layout,
                         int32_t *cum_stats, void *workspace, hipStream_t stream,
                         bool counts_only = false);

// What a dispatch needs to derive a layout's slots after its count kernel:
// the per-tile count rows and packed ranks in the workspace, and the layout
// buffers it writes (dst_slot, src_of_slot, counts, offsets, partition and
// group totals, cumulative stats; status gets its bits OR-ed in).
struct FreshLayout {
    const int32_t *packed;     // [T*K]
    const int32_t *rows;       // [tiles, W]
    int W;
    int tile_tokens;
    int num_tiles;
    int A, P, NG;
    size_t lds_bytes;          // dynamic LDS of a dispatch workgroup
    int32_t *dst_out;
    int32_t *src_out;
    int64_t max_rows;
    int32_t *count_out;
    int32_t *offset_out;
    int32_t *part_out;
    int32_t *group_out;        // or NULL
    int32_t *cum_stats;        // or NULL
};

// LDS of a dispatch workgroup that rebuilds the layout's prefixes: the tile
// rows as prefixes, the totals row, the expert offsets.
inline size_t fresh_lds_bytes(int tiles, int W, int E) {
    return ((size_t)tiles * W + W + ((E + 1 + 3) & ~3)) * 4;
}
constexpr size_t kFreshLdsMax = 64 * 1024;   // two dispatch workgroups per CU

// Fills `f` for a layout of this plan launched with counts_only; false when
// the plan does not allow it (one tile, no tiles, the partition layout, or
// tile rows too large for LDS): then the whole layout runs first.
bool fresh_layout_of(const LayoutPlan &plan, const ep_layout *layout, int32_t *cum_stats,
                     void *workspace, FreshLayout *f);

// The token-queue counters in a layout workspace.
uint32_t *queue_of(const LayoutPlan &plan, void *workspace);

// Row modes of a dispatch: bf16 rows copied, fp8 rows copied with their
// scales, bf16 rows cast to fp8 on the way.
// kModeStores is a measurement aid, not a step of the method: the bf16 copy's
// stores with every token row replaced by a fixed pattern (no row is read).
enum { kModeCopy16 = 0, kModeCopyFp8 = 1, kModeCast = 2, kModeStores = 3 };

struct DispatchArgs {
    const void *x;
    const void *x_scales;          // fp32 or UE8M0 bytes [T, hidden/group]
    const float *topk_weights;
    const int32_t *dst;            // [T*K]
    const int32_t *counts;         // [E]
    const int32_t *offsets;        // [E+1]
    int32_t *status;
    void *recv;
    void *recv_scales;
    float *recv_w;
    int64_t recv_rows;
    int T, K, E, A, C;             // E: receive segments (expanded), experts (partitioned)
    int hidden;
    int group;                     // fp8 scale group (0 when bf16 -> bf16)
    int mode;                      // kModeCopy16, kModeCopyFp8 or kModeCast
    int scale_fmt;                 // 0 fp32 amax/448, 1 fp32 power of two, 2 UE8M0 byte
    int zero_padding;
    // partitioned (non-expanded) dispatch
    int partitioned;
    int P;
    const int32_t *token_slot;     // [T*P]
    const int64_t *topk_idx;       // [T*K]
    int64_t *recv_idx;             // [rows*K] or NULL
    float *recv_wk;                // [rows*K] or NULL
    const int32_t *part_src;       // [T*P] token of each receive row, or NULL
    const int32_t *part_offset;    // [P+1]
    uint32_t pattern;              // kModeStores: the 32-bit word every row is filled with
    const FreshLayout *fresh;      // non-NULL: slots derived here from the count kernel's output
    uint32_t *queue;               // token-queue counters, zero when the dispatch starts, or NULL
};

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream);

struct CombineArgs {
    const void *y;
    int64_t y_rows;
    const float *w;
    const void *bias0;
    const void *bias1;
    const int32_t *dst;
    int32_t *status;
    const float *recv_w;
    float *combined_w;
    void *out;
    int T, K, hidden;
    // reduced (two-level) combine: routing and experts per partition
    const int64_t *topk_idx;
    int E, m;
    int bf16_partials;
};

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

// 10-bit logarithmic payload: bytes of one packed row, the encode (bf16 rows
// -> payload) or decode (payload -> bf16 rows) pass, and the combine that
// reads payload rows (CombineArgs.y) instead of bf16 rows.  Encode skips rows
// with row_src < 0 (when given); max_used_rows bounds the rows it marks and
// picks the launch for sparse batches.
int64_t logfmt_row_bytes(int hidden);
hipError_t launch_logfmt(const void *src, void *dst, int64_t rows, int hidden, bool encode,
                         const int32_t *row_src, int64_t max_used_rows, hipStream_t stream);
hipError_t launch_combine_logfmt(const CombineArgs &a, hipStream_t stream);

hipError_t launch_cast_fp8(const void *x, int T, int hidden, int group, int scale_fmt, uint8_t *q,
                           void *scales,
                           hipStream_t stream);

}  // namespace ep
