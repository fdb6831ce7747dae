// Host-side launchers shared between the kernel files and the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

// Tiling of the layout pass, chosen on the host from the shapes alone.
struct LayoutPlan {
    int T, K, E, A, P, C;
    int64_t max_rows;
    int tile_tokens;   // tokens per count tile (one workgroup)
    int num_tiles;     // ceil(T / tile_tokens)
    int block;         // threads per count workgroup (multiple of 64)
    bool fused;        // count and slots in one cooperative launch when it fits
    bool single;       // the whole batch is one tile: count and slots in one workgroup
    bool prescan;      // many tiles: a scan kernel turns the tile rows into prefixes first
    int chunks_per_wave;
    int G, NG;              // partitions per group, number of groups
    int row_stride;         // ints per tile row: E + P + NG + 1 rounded up to 4
    size_t ws_tile_counts;  // byte offsets inside the workspace
    size_t ws_tok_mask;
    size_t ws_bytes;
};

bool make_layout_plan(const ep_layout_params *p, LayoutPlan *plan);

hipError_t launch_layout(const LayoutPlan &plan, const int64_t *topk_idx, const ep_layout *layout,
                         int32_t *cum_stats, void *workspace, hipStream_t stream);

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
    int T, K, E, A, C;
    int hidden;
    int group;                     // fp8 scale group (0 when bf16 -> bf16)
    int mode;                      // 0 copy bf16, 1 copy fp8 (+scales), 2 cast bf16 -> fp8
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
};

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

hipError_t launch_cast_fp8(const void *x, int T, int hidden, int group, int scale_fmt, uint8_t *q,
                           void *scales,
                           hipStream_t stream);

}  // namespace ep
