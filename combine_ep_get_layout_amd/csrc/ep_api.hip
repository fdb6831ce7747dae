// C ABI of libep.so: argument validation and launches.  Every entry point
// checks what the host can see (sizes, null pointers, alignment, limits) and
// returns a negative ep_status before enqueuing anything, like the length
// checks of the Rust EP=2 routing table ("spark_model/layers/ep_dispatch.rs",
// build_ep_routing_table).  Nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/ep.h"
#include "ep_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int to_status(hipError_t e) {
    if (e == hipSuccess) return EP_OK;
    // a shape whose kernels would need more LDS than a workgroup can have
    return e == hipErrorInvalidConfiguration ? EP_ERR_UNSUPPORTED : EP_ERR_LAUNCH;
}

// Receive segments of a layout: one per expert, or one per partition.
int64_t segments(const ep_layout_params *p) {
    return p->partition_major ? p->num_partitions : p->num_experts;
}

// Shape checks shared by every call that takes layout params.
int check_params(const ep_layout_params *p) {
    if (!p) return EP_ERR_INVALID_ARG;
    if (p->num_tokens < 0 || p->num_topk < 1 || p->num_experts < 1 || p->expert_alignment < 1 ||
        p->num_partitions < 1 || p->capacity < 0 || p->max_recv_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (p->num_experts % p->num_partitions != 0) return EP_ERR_INVALID_ARG;
    if (p->partitions_per_group < 0 ||
        (p->partitions_per_group > 0 && p->num_partitions % p->partitions_per_group != 0))
        return EP_ERR_INVALID_ARG;
    if (p->partition_major != 0 && p->partition_major != 1) return EP_ERR_INVALID_ARG;
    if (p->capacity > 0 && p->capacity % p->expert_alignment != 0) return EP_ERR_INVALID_ARG;
    if (p->num_experts > EP_MAX_EXPERTS || p->num_partitions > EP_MAX_PARTITIONS)
        return EP_ERR_UNSUPPORTED;
    if (p->num_topk > EP_MAX_TOPK) return EP_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)p->num_tokens * p->num_topk;
    if (pairs >= ((int64_t)1 << 31)) return EP_ERR_INVALID_ARG;
    const int64_t worst = ep_worst_case_recv_rows(p);
    if (worst >= ((int64_t)1 << 31)) return EP_ERR_INVALID_ARG;
    if ((int64_t)p->num_tokens * p->num_partitions >= ((int64_t)1 << 40)) return EP_ERR_INVALID_ARG;
    if (p->capacity > 0 && segments(p) * p->capacity > p->max_recv_rows)
        return EP_ERR_INVALID_ARG;
    return EP_OK;
}

// Scratch of ep_get_layout_noalloc: the layout workspace in device memory
// the library itself holds for the life of the process, one copy per GPU.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// This device's copy of the scratch, looked up once per device with that
// device current (the array's host-side name is not a device address);
// NULL if the runtime cannot give it.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" {

int64_t ep_worst_case_recv_rows(const ep_layout_params *p) {
    if (!p) return 0;
    const int64_t S = p->partition_major == 1 ? p->num_partitions : p->num_experts;
    if (p->capacity > 0) return S * p->capacity;
    const int64_t pairs = (int64_t)p->num_tokens * p->num_topk;
    const int64_t ne = pairs < S ? pairs : S;
    return pairs + ne * (int64_t)(p->expert_alignment - 1);
}

size_t ep_get_layout_workspace_bytes(const ep_layout_params *p) {
    if (check_params(p) != EP_OK) return 0;
    ep::LayoutPlan plan;
    if (!ep::make_layout_plan(p, &plan)) return 0;
    return plan.ws_bytes;
}

// Host checks of a layout call; fills the plan.
static int layout_checks(const int64_t *topk_idx, const ep_layout_params *p, const ep_layout *layout,
                         void *workspace, size_t workspace_bytes, ep::LayoutPlan *plan) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (!layout || !layout->num_tokens_per_expert || !layout->expert_offset ||
        !layout->num_tokens_per_partition || !layout->status)
        return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0 && (!topk_idx || !layout->is_token_in_partition || !layout->dst_slot))
        return EP_ERR_INVALID_ARG;
    if (p->max_recv_rows > 0 && !layout->src_of_slot) return EP_ERR_INVALID_ARG;
    if (layout->token_slot && p->num_partitions > EP_MAX_SLOT_PARTITIONS) return EP_ERR_UNSUPPORTED;
    if (layout->partition_src && !layout->token_slot && p->num_tokens > 0) return EP_ERR_INVALID_ARG;
    if (!ep::make_layout_plan(p, plan)) return EP_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < plan->ws_bytes || !aligned16(workspace))
        return EP_ERR_WORKSPACE;
    return EP_OK;
}

int ep_get_layout(const int64_t *topk_idx, const ep_layout_params *p, const ep_layout *layout,
                  int32_t *cumulative_expert_stats, void *workspace, size_t workspace_bytes,
                  void *stream) {
    ep::LayoutPlan plan;
    const int rc = layout_checks(topk_idx, p, layout, workspace, workspace_bytes, &plan);
    if (rc != EP_OK) return rc;
    return to_status(ep::launch_layout(plan, topk_idx, layout, cumulative_expert_stats, workspace,
                                       (hipStream_t)stream));
}

int ep_get_layout_noalloc(const int64_t *topk_idx, const ep_layout_params *p,
                          const ep_layout *layout, int32_t *cumulative_expert_stats,
                          void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    ep::LayoutPlan plan;
    if (!ep::make_layout_plan(p, &plan)) return EP_ERR_UNSUPPORTED;
    if (plan.ws_bytes > kScratchBytes) return EP_ERR_WORKSPACE;   // before any GPU call
    void *ws = device_scratch();
    if (!ws) return EP_ERR_LAUNCH;
    rc = layout_checks(topk_idx, p, layout, ws, kScratchBytes, &plan);
    if (rc != EP_OK) return rc;
    return to_status(ep::launch_layout(plan, topk_idx, layout, cumulative_expert_stats, ws,
                                       (hipStream_t)stream));
}

static bool valid_group(int hidden, int group) {
    if (group == hidden) return true;
    if (group < 16 || group > 512 || (group & (group - 1)) != 0) return false;
    return hidden % group == 0;
}

static bool is_fp8(int d) {
    return d == EP_DTYPE_FP8_E4M3 || d == EP_DTYPE_FP8_E4M3_POW2 || d == EP_DTYPE_FP8_E4M3_UE8M0;
}

static int scale_fmt_of(int d) {
    return d == EP_DTYPE_FP8_E4M3_POW2 ? 1 : (d == EP_DTYPE_FP8_E4M3_UE8M0 ? 2 : 0);
}

// Row mode (0 copy bf16, 1 copy fp8 with its scales, 2 cast bf16 -> fp8) and
// scale format from the two dtypes, with the checks both dispatches share.
static int dispatch_io(int x_dtype, const void *x, const void *x_scales, int recv_dtype,
                       int32_t hidden, int32_t scale_group, int32_t T, const void *recv_x,
                       const void *recv_scales, int64_t num_recv_rows, int *mode, int *fmt) {
    if (num_recv_rows < 0 || hidden < 1) return EP_ERR_INVALID_ARG;
    if (hidden > EP_MAX_HIDDEN) return EP_ERR_UNSUPPORTED;
    if (x_dtype == EP_DTYPE_BF16 && recv_dtype == EP_DTYPE_BF16) *mode = 0;
    else if (is_fp8(x_dtype) && x_dtype == recv_dtype) *mode = 1;
    else if (x_dtype == EP_DTYPE_BF16 && is_fp8(recv_dtype)) *mode = 2;
    else return EP_ERR_INVALID_ARG;
    *fmt = scale_fmt_of(recv_dtype);
    if (*mode == 0 && hidden % 8 != 0) return EP_ERR_INVALID_ARG;
    if (*mode != 0) {
        if (hidden % 16 != 0) return EP_ERR_INVALID_ARG;
        if (!valid_group(hidden, scale_group)) return EP_ERR_UNSUPPORTED;
        if (*mode == 2 && scale_group == hidden && hidden > 16 * 64 * 8) return EP_ERR_UNSUPPORTED;
        if (!recv_scales && num_recv_rows > 0) return EP_ERR_INVALID_ARG;
        if (*mode == 1 && !x_scales && T > 0) return EP_ERR_INVALID_ARG;
        // fp32 scales are written (and, for a copy, read) as whole floats
        if (*fmt != 2 && !aligned4(recv_scales)) return EP_ERR_INVALID_ARG;
        if (*mode == 1 && *fmt != 2 && !aligned4(x_scales)) return EP_ERR_INVALID_ARG;
    }
    if (T > 0 && (!x || !aligned16(x))) return EP_ERR_INVALID_ARG;
    if (num_recv_rows > 0 && (!recv_x || !aligned16(recv_x))) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

// Host checks of an (expanded) dispatch call; fills everything of the
// launch arguments but the layout's source (dst_slot, or a fresh layout).
static int dispatch_checks(const void *x, int x_dtype, const void *x_scales, int recv_dtype,
                           int32_t hidden, int32_t scale_group, const float *topk_weights,
                           const ep_layout_params *p, const ep_layout *layout, void *recv_x,
                           void *recv_scales, float *recv_topk_weights, int64_t num_recv_rows,
                           int zero_padding, ep::DispatchArgs *out) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (!layout || !layout->num_tokens_per_expert || !layout->expert_offset || !layout->status)
        return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0 && !layout->dst_slot) return EP_ERR_INVALID_ARG;
    int mode = 0, fmt = 0;
    rc = dispatch_io(x_dtype, x, x_scales, recv_dtype, hidden, scale_group, p->num_tokens, recv_x,
                     recv_scales, num_recv_rows, &mode, &fmt);
    if (rc != EP_OK) return rc;
    ep::DispatchArgs &a = *out;
    a = ep::DispatchArgs{};
    a.x = x;
    a.x_scales = x_scales;
    a.scale_fmt = fmt;
    a.topk_weights = topk_weights;
    a.dst = layout->dst_slot;
    a.counts = layout->num_tokens_per_expert;
    a.offsets = layout->expert_offset;
    a.status = layout->status;
    a.recv = recv_x;
    a.recv_scales = recv_scales;
    a.recv_w = recv_topk_weights;
    a.recv_rows = num_recv_rows;
    a.T = p->num_tokens;
    a.K = p->num_topk;
    a.E = (int)segments(p);   // the receive segments the padding workgroups visit
    a.A = p->expert_alignment;
    a.C = p->capacity;
    a.hidden = hidden;
    a.group = mode == 0 ? 0 : scale_group;
    a.mode = mode;
    a.zero_padding = zero_padding ? 1 : 0;
    return EP_OK;
}

int ep_dispatch(const void *x, int x_dtype, const void *x_scales, int recv_dtype, int32_t hidden,
                int32_t scale_group, const float *topk_weights, const ep_layout_params *p,
                const ep_layout *layout, void *recv_x, void *recv_scales,
                float *recv_topk_weights, int64_t num_recv_rows, int zero_padding, void *stream) {
    ep::DispatchArgs a;
    const int rc = dispatch_checks(x, x_dtype, x_scales, recv_dtype, hidden, scale_group,
                                   topk_weights, p, layout, recv_x, recv_scales, recv_topk_weights,
                                   num_recv_rows, zero_padding, &a);
    if (rc != EP_OK) return rc;
    return to_status(ep::launch_dispatch(a, (hipStream_t)stream));
}

int ep_dispatch_with_layout(const int64_t *topk_idx, const ep_layout_params *p,
                            const ep_layout *layout, int32_t *cumulative_expert_stats,
                            void *workspace, size_t workspace_bytes, const void *x, int x_dtype,
                            const void *x_scales, int recv_dtype, int32_t hidden,
                            int32_t scale_group, const float *topk_weights, void *recv_x,
                            void *recv_scales, float *recv_topk_weights, int64_t num_recv_rows,
                            int zero_padding, void *stream) {
    ep::LayoutPlan plan;
    int rc = layout_checks(topk_idx, p, layout, workspace, workspace_bytes, &plan);
    if (rc != EP_OK) return rc;
    ep::DispatchArgs a;
    rc = dispatch_checks(x, x_dtype, x_scales, recv_dtype, hidden, scale_group, topk_weights, p,
                         layout, recv_x, recv_scales, recv_topk_weights, num_recv_rows,
                         zero_padding, &a);
    if (rc != EP_OK) return rc;
    const hipStream_t st = (hipStream_t)stream;
    // The count kernel alone, then dispatch kernels that derive the slots.
    // Only the copy modes do: their rows run on a resident grid of a few
    // hundred workgroups, while the cast launches one workgroup per row piece
    // (thousands), each of which would repeat the derivation.  Shapes that do
    // not allow it (one tile, the partition layout, tile rows too large for
    // LDS) and the cast run the whole layout first.
    ep::FreshLayout f;
    const bool fold = a.mode != ep::kModeCast &&
                      ep::fresh_layout_of(plan, layout, cumulative_expert_stats, workspace, &f);
    hipError_t err = ep::launch_layout(plan, topk_idx, layout, cumulative_expert_stats, workspace,
                                       st, fold);
    if (err != hipSuccess) return to_status(err);
    if (fold) a.fresh = &f;
    a.queue = ep::queue_of(plan, workspace);
    return to_status(ep::launch_dispatch(a, st));
}

int ep_probe_dispatch_stores(int32_t hidden, uint32_t pattern, const ep_layout_params *p,
                             const ep_layout *layout, void *recv_x, int64_t num_recv_rows,
                             void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (!layout || !layout->status || (p->num_tokens > 0 && !layout->dst_slot))
        return EP_ERR_INVALID_ARG;
    if (hidden < 8 || hidden % 8 != 0 || num_recv_rows < 0) return EP_ERR_INVALID_ARG;
    if (hidden > EP_MAX_HIDDEN) return EP_ERR_UNSUPPORTED;
    if (p->num_tokens > 0 && num_recv_rows > 0 && (!recv_x || !aligned16(recv_x)))
        return EP_ERR_INVALID_ARG;
    ep::DispatchArgs a = {};
    a.dst = layout->dst_slot;
    a.counts = layout->num_tokens_per_expert;
    a.offsets = layout->expert_offset;
    a.status = layout->status;
    a.recv = recv_x;
    a.recv_rows = num_recv_rows;
    a.T = p->num_tokens;
    a.K = p->num_topk;
    a.E = (int)segments(p);
    a.A = p->expert_alignment;
    a.C = p->capacity;
    a.hidden = hidden;
    a.mode = ep::kModeStores;
    a.pattern = pattern;
    return to_status(ep::launch_dispatch(a, (hipStream_t)stream));
}

int ep_combine(const void *y, int32_t hidden, int64_t num_y_rows, const float *topk_weights,
               const void *bias0, const void *bias1, const ep_layout_params *p,
               const ep_layout *layout, const float *recv_topk_weights,
               float *combined_topk_weights, void *out, void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (!layout || !layout->status || (p->num_tokens > 0 && !layout->dst_slot))
        return EP_ERR_INVALID_ARG;
    if (hidden < 8 || hidden % 8 != 0 || num_y_rows < 0) return EP_ERR_INVALID_ARG;
    if (combined_topk_weights && !recv_topk_weights) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0) {
        if (!out || !aligned16(out)) return EP_ERR_INVALID_ARG;
        if (num_y_rows > 0 && (!y || !aligned16(y))) return EP_ERR_INVALID_ARG;
        if ((bias0 && !aligned16(bias0)) || (bias1 && !aligned16(bias1))) return EP_ERR_INVALID_ARG;
    }
    ep::CombineArgs c = {};
    c.y = y;
    c.y_rows = num_y_rows;
    c.w = topk_weights;
    c.bias0 = bias0;
    c.bias1 = bias1;
    c.dst = layout->dst_slot;
    c.status = layout->status;
    c.recv_w = recv_topk_weights;
    c.combined_w = combined_topk_weights;
    c.out = out;
    c.T = p->num_tokens;
    c.K = p->num_topk;
    c.hidden = hidden;
    return to_status(ep::launch_combine(c, (hipStream_t)stream));
}

int ep_dispatch_partitioned(const void *x, int x_dtype, const void *x_scales, int recv_dtype,
                            int32_t hidden, int32_t scale_group, const int64_t *topk_idx,
                            const float *topk_weights, const ep_layout_params *p,
                            const ep_layout *layout, void *recv_x, void *recv_scales,
                            int64_t *recv_topk_idx, float *recv_topk_weights,
                            int64_t num_recv_rows, void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (p->num_partitions > EP_MAX_SLOT_PARTITIONS) return EP_ERR_UNSUPPORTED;
    if (!layout || !layout->status) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0 && !layout->token_slot) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0 && (recv_topk_idx || recv_topk_weights) && !topk_idx)
        return EP_ERR_INVALID_ARG;
    int mode = 0, fmt = 0;
    rc = dispatch_io(x_dtype, x, x_scales, recv_dtype, hidden, scale_group, p->num_tokens, recv_x,
                     recv_scales, num_recv_rows, &mode, &fmt);
    if (rc != EP_OK) return rc;
    ep::DispatchArgs a = {};
    a.x = x;
    a.x_scales = x_scales;
    a.scale_fmt = fmt;
    a.topk_weights = topk_weights;
    a.status = layout->status;
    a.recv = recv_x;
    a.recv_scales = recv_scales;
    a.recv_rows = num_recv_rows;
    a.T = p->num_tokens;
    a.K = p->num_topk;
    a.E = p->num_experts;
    a.A = 1;
    a.C = 0;
    a.hidden = hidden;
    a.group = mode == 0 ? 0 : scale_group;
    a.mode = mode;
    a.partitioned = 1;
    a.P = p->num_partitions;
    a.token_slot = layout->token_slot;
    a.topk_idx = topk_idx;
    a.recv_idx = recv_topk_idx;
    a.recv_wk = recv_topk_weights;
    a.part_src = layout->partition_src;
    a.part_offset = layout->partition_offset;
    return to_status(ep::launch_dispatch(a, (hipStream_t)stream));
}

int ep_combine_partitioned(const void *y, int32_t hidden, int64_t num_y_rows, const void *bias0,
                           const void *bias1, const ep_layout_params *p, const ep_layout *layout,
                           void *out, void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (p->num_partitions > EP_MAX_SLOT_PARTITIONS) return EP_ERR_UNSUPPORTED;
    if (!layout || !layout->status || (p->num_tokens > 0 && !layout->token_slot))
        return EP_ERR_INVALID_ARG;
    if (hidden < 8 || hidden % 8 != 0 || num_y_rows < 0) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0) {
        if (!out || !aligned16(out)) return EP_ERR_INVALID_ARG;
        if (num_y_rows > 0 && (!y || !aligned16(y))) return EP_ERR_INVALID_ARG;
        if ((bias0 && !aligned16(bias0)) || (bias1 && !aligned16(bias1))) return EP_ERR_INVALID_ARG;
    }
    ep::CombineArgs c = {};
    c.y = y;
    c.y_rows = num_y_rows;
    c.bias0 = bias0;
    c.bias1 = bias1;
    c.dst = layout->token_slot;
    c.status = layout->status;
    c.out = out;
    c.T = p->num_tokens;
    c.K = p->num_partitions;
    c.hidden = hidden;
    return to_status(ep::launch_combine(c, (hipStream_t)stream));
}

int ep_combine_reduced(const void *y, int32_t hidden, int64_t num_y_rows, const int64_t *topk_idx,
                       const float *topk_weights, const void *bias0, const void *bias1,
                       const ep_layout_params *p, const ep_layout *layout, void *out,
                       int bf16_partials, void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (p->num_topk > 64) return EP_ERR_UNSUPPORTED;
    if (!layout || !layout->status || (p->num_tokens > 0 && (!layout->dst_slot || !topk_idx)))
        return EP_ERR_INVALID_ARG;
    if (hidden < 8 || hidden % 8 != 0 || num_y_rows < 0) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0) {
        if (!out || !aligned16(out)) return EP_ERR_INVALID_ARG;
        if (num_y_rows > 0 && (!y || !aligned16(y))) return EP_ERR_INVALID_ARG;
        if ((bias0 && !aligned16(bias0)) || (bias1 && !aligned16(bias1))) return EP_ERR_INVALID_ARG;
    }
    ep::CombineArgs c = {};
    c.y = y;
    c.y_rows = num_y_rows;
    c.w = topk_weights;
    c.bias0 = bias0;
    c.bias1 = bias1;
    c.dst = layout->dst_slot;
    c.status = layout->status;
    c.out = out;
    c.T = p->num_tokens;
    c.K = p->num_topk;
    c.hidden = hidden;
    c.topk_idx = topk_idx;
    c.E = p->num_experts;
    c.m = p->num_experts / p->num_partitions;
    c.bf16_partials = bf16_partials ? 1 : 0;
    return to_status(ep::launch_combine(c, (hipStream_t)stream));
}

int ep_cast_fp8(const void *x, int32_t num_tokens, int32_t hidden, int32_t group, int out_dtype,
                uint8_t *x_fp8, void *scales, void *stream) {
    if (num_tokens < 0 || hidden < 16 || hidden % 16 != 0) return EP_ERR_INVALID_ARG;
    if (!is_fp8(out_dtype)) return EP_ERR_INVALID_ARG;
    if (!valid_group(hidden, group)) return EP_ERR_UNSUPPORTED;
    if (group == hidden && hidden > 16 * 64 * 8) return EP_ERR_UNSUPPORTED;
    if (num_tokens == 0) return EP_OK;
    if (!x || !x_fp8 || !scales || !aligned16(x) || !aligned16(x_fp8)) return EP_ERR_INVALID_ARG;
    if (out_dtype != EP_DTYPE_FP8_E4M3_UE8M0 && !aligned4(scales)) return EP_ERR_INVALID_ARG;
    return to_status(ep::launch_cast_fp8(x, num_tokens, hidden, group, scale_fmt_of(out_dtype),
                                         x_fp8, scales, (hipStream_t)stream));
}

static bool logfmt_hidden_ok(int32_t hidden) {
    return hidden >= 128 && hidden % 128 == 0;
}

int64_t ep_logfmt_row_bytes(int32_t hidden) {
    if (!logfmt_hidden_ok(hidden)) return EP_ERR_INVALID_ARG;
    return ep::logfmt_row_bytes(hidden);
}

int ep_logfmt_encode(const void *x, int64_t num_rows, int32_t hidden,
                     const ep_layout_params *p, const ep_layout *layout, void *payload,
                     void *stream) {
    if (!logfmt_hidden_ok(hidden) || num_rows < 0) return EP_ERR_INVALID_ARG;
    if ((p == nullptr) != (layout == nullptr)) return EP_ERR_INVALID_ARG;
    const int32_t *row_src = nullptr;
    int64_t pairs = 0;
    if (p) {
        int rc = check_params(p);
        if (rc != EP_OK) return rc;
        if (!layout->src_of_slot || num_rows > p->max_recv_rows) return EP_ERR_INVALID_ARG;
        row_src = layout->src_of_slot;
        pairs = (int64_t)p->num_tokens * p->num_topk;
    }
    if (num_rows == 0) return EP_OK;
    if (!x || !payload || !aligned16(x) || !aligned16(payload)) return EP_ERR_INVALID_ARG;
    return to_status(ep::launch_logfmt(x, payload, num_rows, hidden, true, row_src, pairs,
                                       (hipStream_t)stream));
}

int ep_logfmt_decode(const void *payload, int64_t num_rows, int32_t hidden, void *out,
                     void *stream) {
    if (!logfmt_hidden_ok(hidden) || num_rows < 0) return EP_ERR_INVALID_ARG;
    if (num_rows == 0) return EP_OK;
    if (!payload || !out || !aligned16(payload) || !aligned16(out)) return EP_ERR_INVALID_ARG;
    return to_status(ep::launch_logfmt(payload, out, num_rows, hidden, false, nullptr, 0,
                                       (hipStream_t)stream));
}

int ep_combine_logfmt(const void *payload, int32_t hidden, int64_t num_y_rows,
                      const float *topk_weights, const void *bias0, const void *bias1,
                      const ep_layout_params *p, const ep_layout *layout,
                      const float *recv_topk_weights, float *combined_topk_weights, void *out,
                      void *stream) {
    int rc = check_params(p);
    if (rc != EP_OK) return rc;
    if (!layout || !layout->status || (p->num_tokens > 0 && !layout->dst_slot))
        return EP_ERR_INVALID_ARG;
    if (!logfmt_hidden_ok(hidden) || num_y_rows < 0) return EP_ERR_INVALID_ARG;
    if (combined_topk_weights && !recv_topk_weights) return EP_ERR_INVALID_ARG;
    if (p->num_tokens > 0) {
        if (!out || !aligned16(out)) return EP_ERR_INVALID_ARG;
        if (num_y_rows > 0 && (!payload || !aligned16(payload))) return EP_ERR_INVALID_ARG;
        if ((bias0 && !aligned16(bias0)) || (bias1 && !aligned16(bias1))) return EP_ERR_INVALID_ARG;
    }
    ep::CombineArgs c = {};
    c.y = payload;
    c.y_rows = num_y_rows;
    c.w = topk_weights;
    c.bias0 = bias0;
    c.bias1 = bias1;
    c.dst = layout->dst_slot;
    c.status = layout->status;
    c.recv_w = recv_topk_weights;
    c.combined_w = combined_topk_weights;
    c.out = out;
    c.T = p->num_tokens;
    c.K = p->num_topk;
    c.hidden = hidden;
    return to_status(ep::launch_combine_logfmt(c, (hipStream_t)stream));
}

const char *ep_status_string(int code) {
    switch (code) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARG: return "invalid argument";
        case EP_ERR_UNSUPPORTED: return "outside the library's limits";
        case EP_ERR_WORKSPACE: return "workspace missing or too small";
        case EP_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
