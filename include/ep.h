/*
 * ep.h - C ABI of the MI355X (gfx950) MoE expert-parallel layout / dispatch /
 * combine library (libep.so).
 *
 * One GPU's share of DeepEP-style token dispatch and combine: derive a
 * receive layout from top-k routing, permute token rows into an
 * expert-ordered, alignment-padded receive buffer, and reduce expert outputs
 * back to their source tokens.  Sources, cited by page title:
 *
 *   [API]  "DeepEP test target API reference" (DeepEP v2 test page):
 *          2.1 dispatch() and its parameter table, 2.2 combine(),
 *          3.1 V1 Buffer.dispatch() layout tensors, 3.2 V1 combine (no
 *          weights), 3.3 low-latency dispatch scale options, 4.1 refs
 *          (ordered accumulation), 4.2 math (align, per-token cast to
 *          float8_e4m3fn).
 *   [RUST] "spark_model/layers/ep_dispatch.rs": partition of (token, expert,
 *          weight) pairs by expert ownership; length checks.
 *
 * Conventions for every entry point:
 *   - Pointers named in the comments as "device" point to GPU memory the
 *     caller allocated (hipMalloc, or a framework allocator); "host" pointers
 *     point to CPU memory read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without synchronising.  No call
 *     allocates or frees memory.  Apart from the scratch array behind
 *     ep_get_layout_noalloc and a cached compute-unit count per device, the
 *     library keeps no state between calls.
 *   - Argument errors the host can see return a negative ep_status before
 *     anything is enqueued.  Errors only the device can see set bits in
 *     layout->status (EP_DEV_*), read by the caller after synchronising.
 *   - Counts, offsets and slots are int32; callers keep T*K, R < 2^31.
 *   - A call may enqueue more than one kernel, all on `stream` in order (the
 *     layout runs one to three; a zero-padded fixed-capacity dispatch that is
 *     mostly padding zero-fills the region first).  Calls that share a
 *     layout, workspace or output buffer must be ordered by the caller (one
 *     stream, or events): there is no locking, and overlapping calls on such
 *     buffers race.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = -1,  /* bad size, null required pointer, misalignment */
    EP_ERR_UNSUPPORTED = -2,  /* valid but outside the library's limits      */
    EP_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required   */
    EP_ERR_LAUNCH = -4        /* the HIP runtime refused a launch             */
} ep_status;

/* Bits OR-ed into layout->status by the device. */
enum {
    EP_DEV_BAD_EXPERT = 1,     /* an id outside [-1, E): the pair is ignored    */
    EP_DEV_CAPACITY = 2,       /* fixed capacity: a segment got more than C     */
    EP_DEV_RECV_OVERFLOW = 4   /* a slot >= the rows the caller allocated       */
};

/* Row types.  The fp8 types carry one scale per (row, group of G channels):
 *   EP_DTYPE_FP8_E4M3        fp32 scale s = max(amax, 1e-4f) / 448 ([API] 4.2)
 *   EP_DTYPE_FP8_E4M3_POW2   fp32 scale rounded up to a power of two
 *                            ([API] 3.3 round_scale)
 *   EP_DTYPE_FP8_E4M3_UE8M0  the same power of two stored as one UE8M0 byte,
 *                            its biased exponent b, value 2^(b-127)
 *                            ([API] 3.3 use_ue8m0)
 * Codes are e4m3_rne(x / s) in every case (exact division for powers of two). */
enum { EP_DTYPE_BF16 = 0, EP_DTYPE_FP8_E4M3 = 1, EP_DTYPE_FP8_E4M3_POW2 = 2,
       EP_DTYPE_FP8_E4M3_UE8M0 = 3 };

/* Limits of the library. */
enum { EP_MAX_EXPERTS = 4096, EP_MAX_PARTITIONS = 1024, EP_MAX_TOPK = 256,
       EP_MAX_SLOT_PARTITIONS = 64, EP_MAX_HIDDEN = 1 << 20 };

/* Shape of one layout ([API] 2.1 parameter table: num_experts,
 * expert_alignment, num_max_tokens_per_rank; 3.1 num_tokens_per_rank). */
typedef struct ep_layout_params {
    int32_t num_tokens;        /* T >= 0                                          */
    int32_t num_topk;          /* K >= 1                                          */
    int32_t num_experts;       /* E in [1, EP_MAX_EXPERTS]                        */
    int32_t expert_alignment;  /* A >= 1: each expert's rows padded to a multiple */
    int32_t num_partitions;    /* P in [1, EP_MAX_PARTITIONS], E % P == 0;        */
                               /* partition q owns experts [q*E/P, (q+1)*E/P)     */
    int32_t capacity;          /* 0: compact padded layout; C > 0: fixed-capacity */
                               /* ("expand") layout, expert e owns rows           */
                               /* [e*C, (e+1)*C); requires C % A == 0             */
    int32_t partitions_per_group; /* G: partitions per group (0 = P, one group);  */
                               /* P % G == 0; [API] 3.1 num_tokens_per_rdma_rank  */
    int32_t partition_major;   /* 0: one receive segment per expert (expert-      */
                               /* major order); 1: one segment per partition,     */
                               /* the pairs of its experts in (t, k) order        */
                               /* (partition- or rank-major receive order)        */
    int64_t max_recv_rows;     /* rows of src_of_slot the caller allocated        */
} ep_layout_params;

/* Receive segments.  The receive rows are split into S segments laid out
 * back to back: S = E (segment e holds the pairs routed to expert e), or,
 * with partition_major, S = P (segment q holds the pairs whose expert is in
 * partition q, [q*E/P, (q+1)*E/P)).  Inside a segment the pairs are in
 * ascending t*K+k order, and each segment is padded to a multiple of
 * expert_alignment (or has C rows with a fixed capacity).  The per-segment
 * tables (num_tokens_per_expert, expert_offset, cumulative_expert_stats)
 * have S (S + 1) entries; their names keep the expert-major reading. */

/* The layout ("handle", [API] 2.1 return values and 3.1 layout tensors):
 * caller-owned device buffers, written by ep_get_layout and read by
 * ep_dispatch / ep_combine. */
typedef struct ep_layout {
    int32_t *num_tokens_per_expert;     /* [S]   pairs routed to each segment         */
    int32_t *expert_offset;             /* [S+1] first receive row of each segment;  */
                                        /*       [S] = R, the receive rows in use     */
    int32_t *num_tokens_per_partition;  /* [P]   tokens with >= 1 pair in partition   */
    uint8_t *is_token_in_partition;     /* [T*P] 0/1                                  */
    int32_t *dst_slot;                  /* [T*K] receive row of pair (t,k), or -1     */
    int32_t *src_of_slot;               /* [max_recv_rows] t*K+k, or -1 for padding   */
    int32_t *status;                    /* [1]   EP_DEV_* bits                        */
    /* Optional (NULL = not computed): the non-expanded partition ("rank")       */
    /* layout of [API] 2.1 (do_expand = False) and 3.1.  A token is received    */
    /* once by every partition owning one of its experts, tokens in order.      */
    int32_t *partition_offset;          /* [P+1] first row of each partition         */
    int32_t *token_slot;                /* [T*P] row of (t, q) or -1; needs P <= 64  */
    int32_t *num_tokens_per_group;      /* [P/G] tokens reaching any partition of    */
                                        /*       the group (num_tokens_per_rdma_rank) */
    int32_t *partition_src;             /* [T*P] token of partition row r (r < Rp):  */
                                        /*       the inverse of token_slot; needs it */
} ep_layout;

/* Bytes of device workspace ep_get_layout needs for these params (host call,
 * no GPU work).  Returns 0 when the params are invalid. */
size_t ep_get_layout_workspace_bytes(const ep_layout_params *params);

/* Worst-case receive rows for these params (host call): S*C in fixed mode,
 * else T*K + min(S, T*K)*(A-1), S the number of receive segments.  Buffers
 * of this many rows never overflow. */
int64_t ep_worst_case_recv_rows(const ep_layout_params *params);

/* ep_get_layout - derive the receive layout from top-k routing.
 * ([API] 2.1: V2 derives the layout from topk_idx; 3.1: the V1 layout
 *  tensors num_tokens_per_expert / is_token_in_rank / num_tokens_per_rank;
 *  4.2 align; [RUST] partition by expert range, token-major then k order.)
 *
 *   topk_idx   device int64 [T, K], row-major; -1 = no expert.
 *   params     host; shape of the layout.
 *   layout     host struct of device buffers (all seven required, except that
 *              arrays with zero elements may be NULL).
 *   cumulative_expert_stats  device int32 [S] or NULL: += per-segment counts
 *              ([API] 2.1 cumulative_local_expert_recv_stats).
 *   workspace  device, >= ep_get_layout_workspace_bytes(params) bytes, 16-byte
 *              aligned; contents need no initialisation and are scratch.
 *
 * Computes, with s(t,k) the segment of pair (t,k) (its expert, or with
 * partition_major its partition): count[s] = #{(t,k): segment s};
 * padded[s] = align(count[s], A); expert_offset = exclusive scan of padded
 * (compact) or s*C (fixed); dst_slot[t,k] = expert_offset[s] + j where j is
 * the rank of (t,k) among the pairs of segment s in ascending t*K+k order
 * (-1 for idx = -1, for an invalid id, and for pairs with j >= C in fixed
 * mode); src_of_slot[r] = t*K+k for
 * used slots and -1 for padding slots (slots >= max_recv_rows are not
 * written); partition membership and per-partition token counts; and, for
 * the optional pointers that are set, the partition layout (offsets,
 * token_slot, tokens per group of G partitions).  token_slot needs
 * P <= EP_MAX_SLOT_PARTITIONS (else EP_ERR_UNSUPPORTED); the offsets and the
 * group counts work for any P.
 * layout->status is overwritten with EP_DEV_BAD_EXPERT / EP_DEV_CAPACITY /
 * EP_DEV_RECV_OVERFLOW (R > max_recv_rows).  T = 0 is valid.
 * Errors: EP_ERR_INVALID_ARG (null pointer, T < 0, K < 1, E < 1, A < 1,
 * P < 1, E % P != 0, partitions_per_group < 0 or not dividing P,
 * partition_major not 0 or 1, C < 0, C % A != 0, fixed mode with
 * S*C > max_recv_rows, int32 overflow of T*K or of the worst-case rows),
 * EP_ERR_UNSUPPORTED
 * (E > EP_MAX_EXPERTS, P > EP_MAX_PARTITIONS, K > EP_MAX_TOPK),
 * EP_ERR_WORKSPACE. */
int ep_get_layout(const int64_t *topk_idx, const ep_layout_params *params,
                  const ep_layout *layout, int32_t *cumulative_expert_stats,
                  void *workspace, size_t workspace_bytes, void *stream);

/* ep_get_layout_noalloc - ep_get_layout with no workspace argument, for
 * callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it).  The workspace is a static device array
 * the library holds for the life of the process, one per GPU, of 8 MiB;
 * layouts whose workspace (ep_get_layout_workspace_bytes) exceeds it return
 * EP_ERR_WORKSPACE before anything is enqueued.  Nothing is allocated.  All
 * calls on one GPU share that array (it keeps the last call's contents;
 * nothing in it needs to start at zero): calls that overlap on one GPU, on
 * different streams, race.  Arguments and outputs are ep_get_layout's. */
int ep_get_layout_noalloc(const int64_t *topk_idx, const ep_layout_params *params,
                          const ep_layout *layout, int32_t *cumulative_expert_stats,
                          void *stream);

/* ep_dispatch - permute token rows into the receive buffer.
 * ([API] 2.1: x is bf16 [T, hidden] or the pair (fp8 codes, scales); recv_x
 *  has the input's type; do_zero_padding; 4.2 per-token cast to e4m3;
 *  3.3 round_scale / use_ue8m0 scale formats.)
 *
 *   x            device [T, hidden]: bf16 (x_dtype EP_DTYPE_BF16) or e4m3 codes
 *                (one of the EP_DTYPE_FP8_* types); 16-byte aligned.
 *   x_scales     device [T, hidden/scale_group] when x is fp8, else NULL:
 *                float (4-byte aligned), or uint8 for EP_DTYPE_FP8_E4M3_UE8M0.
 *   recv_dtype   == x_dtype, or an fp8 type with bf16 x: the rows are cast
 *                on the fly, exactly as ep_cast_fp8 to that type followed by
 *                an fp8 dispatch would do.
 *   hidden       channels per row; multiple of 8 (bf16) or 16 (fp8 rows).
 *   scale_group  G, channels per fp32 scale when fp8 is involved: a power of
 *                two in [16, 512] dividing hidden, or hidden itself (one scale
 *                per token).  Ignored for bf16 -> bf16.
 *   topk_weights device float [T, K] or NULL.
 *   params, layout  as produced by ep_get_layout for the same routing.
 *   recv_x       device [num_recv_rows, hidden] of recv_dtype; 16-byte aligned.
 *   recv_scales  device [num_recv_rows, hidden/G] when recv is fp8: float
 *                (4-byte aligned), or uint8 for EP_DTYPE_FP8_E4M3_UE8M0.
 *   recv_topk_weights device float [num_recv_rows] or NULL: weight of the pair
 *                in each row (1 when topk_weights is NULL), 0 for padding rows.
 *   num_recv_rows rows allocated for recv_x / recv_scales / recv_topk_weights;
 *                rows past it are skipped and EP_DEV_RECV_OVERFLOW is set.
 *   zero_padding 1: padding rows (and their scales) are written with zeros;
 *                0: their bytes are left as they were.
 * recv_x[dst_slot[t,k]] = x[t] byte for byte (fp8: codes and scale row).
 * Errors: EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED (a scale_group outside the
 * set above, one scale per row, G = hidden, above 8192 channels in a cast:
 * the row must fit one wave, or hidden > EP_MAX_HIDDEN). */
int ep_dispatch(const void *x, int x_dtype, const void *x_scales, int recv_dtype,
                int32_t hidden, int32_t scale_group, const float *topk_weights,
                const ep_layout_params *params, const ep_layout *layout,
                void *recv_x, void *recv_scales, float *recv_topk_weights,
                int64_t num_recv_rows, int zero_padding, void *stream);

/* ep_dispatch_with_layout - ep_get_layout followed by ep_dispatch, in one
 * call ([API] 2.1: V2's dispatch derives the layout from topk_idx itself and
 * returns the handle for combine).  Arguments are those of the two calls;
 * every output (the layout buffers, cumulative stats and the receive
 * buffers) is bit for bit what the two calls in sequence write.  Only the
 * layout's count kernel runs before the rows: each dispatch workgroup
 * derives the offsets and its pairs' slots from the count kernel's tile rows
 * in LDS and writes dst_slot / src_of_slot as it goes.  That applies to
 * the copy modes (bf16 and fp8 rows as they are); the bf16 -> fp8 cast, a
 * batch of one count tile, the partition layout requested through
 * layout->token_slot or partition_offset, and tile rows beyond 64 KB run the
 * two calls' kernels as they are.  The workspace is ep_get_layout's.
 * Errors: those of ep_get_layout and ep_dispatch, checked before anything is
 * enqueued. */
int ep_dispatch_with_layout(const int64_t *topk_idx, const ep_layout_params *params,
                            const ep_layout *layout, int32_t *cumulative_expert_stats,
                            void *workspace, size_t workspace_bytes, const void *x, int x_dtype,
                            const void *x_scales, int recv_dtype, int32_t hidden,
                            int32_t scale_group, const float *topk_weights, void *recv_x,
                            void *recv_scales, float *recv_topk_weights, int64_t num_recv_rows,
                            int zero_padding, void *stream);

/* ep_combine - gather expert outputs back to their tokens and reduce.
 * ([API] 2.2: weighted reduction back to the source, bias 0/1/2 tensors,
 *  returns combined_x bf16 [T, hidden] and combined_topk_weights; 3.2: V1
 *  combine is an unweighted sum; 4.1: ordered accumulation.)
 *
 *   y            device bf16 [num_y_rows, hidden] (the receive layout's rows);
 *                16-byte aligned; hidden % 8 == 0.
 *   topk_weights device float [T, K], or NULL for the unweighted sum.
 *   bias0, bias1 device bf16 [T, hidden] or NULL.
 *   recv_topk_weights      device float [num_y_rows] or NULL (input).
 *   combined_topk_weights  device float [T, K] or NULL (output):
 *                recv_topk_weights[dst_slot[t,k]] for kept pairs, else 0;
 *                requires recv_topk_weights.
 *   out          device bf16 [T, hidden].
 * out[t,c] = bf16_rne(acc) where acc = 0; acc += bias0; acc += bias1; then for
 * k = 0..K-1 with dst_slot[t,k] >= 0: acc = fmaf(w[t,k], y[dst_slot[t,k], c], acc)
 * in fp32.  No atomics: the result is deterministic and does not depend on
 * which other tokens are in the batch.  Slots >= num_y_rows are skipped and
 * set EP_DEV_RECV_OVERFLOW. */
int ep_combine(const void *y, int32_t hidden, int64_t num_y_rows,
               const float *topk_weights, const void *bias0, const void *bias1,
               const ep_layout_params *params, const ep_layout *layout,
               const float *recv_topk_weights, float *combined_topk_weights,
               void *out, void *stream);

/* ep_dispatch_partitioned - the non-expanded dispatch ([API] 2.1 with
 * do_expand = False: every token once to each partition (rank) that owns one
 * of its experts; recv_topk_idx / recv_topk_weights come with the row).
 * Needs layout->token_slot (from ep_get_layout).  Arguments as ep_dispatch,
 * plus:
 *   topk_idx            device int64 [T, K] (the routing the layout came from).
 *   recv_topk_idx       device int64 [num_recv_rows, K] or NULL: for the row of
 *                       (t, q), e - q*E/P when pair (t, k) goes to partition q
 *                       (the expert id local to the partition), else -1.
 *   recv_topk_weights   device float [num_recv_rows, K] or NULL: w[t,k] (1 when
 *                       topk_weights is NULL) for local pairs, else 0.
 * With layout->partition_src set, these two are written row by row in
 * receive order (coalesced); without it, by the token's wave at scattered
 * rows (the same values). 
 * Receive rows are [partition_offset[q], partition_offset[q+1]) for partition
 * q, tokens ascending; there is no padding.  Errors as ep_dispatch;
 * EP_ERR_UNSUPPORTED when P > EP_MAX_SLOT_PARTITIONS. */
int ep_dispatch_partitioned(const void *x, int x_dtype, const void *x_scales, int recv_dtype,
                            int32_t hidden, int32_t scale_group, const int64_t *topk_idx,
                            const float *topk_weights, const ep_layout_params *params,
                            const ep_layout *layout, void *recv_x, void *recv_scales,
                            int64_t *recv_topk_idx, float *recv_topk_weights,
                            int64_t num_recv_rows, void *stream);

/* ep_combine_partitioned - combine for the non-expanded layout ([API] 3.2:
 * a plain sum; each partition's row already holds its weighted expert sum):
 * out[t] = bf16_rne(acc), acc = 0; acc += bias0; acc += bias1; then for q
 * ascending with token_slot[t,q] >= 0: acc += y[token_slot[t,q]] (fp32).
 * y is bf16 [num_y_rows, hidden]; needs layout->token_slot. */
int ep_combine_partitioned(const void *y, int32_t hidden, int64_t num_y_rows, const void *bias0,
                           const void *bias1, const ep_layout_params *params,
                           const ep_layout *layout, void *out, void *stream);

/* ep_combine_reduced - the two-level ("reduced") combine on the expanded
 * layout ([API] 2.2: reduced combine, multi-level reduction).  Level 1, per
 * partition q: p_q = fmaf chain from 0 over the token's pairs in q (k
 * ascending), fp32; with bf16_partials = 1 each p_q is rounded to bf16 (the
 * dtype a partial would travel in between ranks).  Level 2: acc = 0;
 * acc += bias0; acc += bias1; acc += p_q for q ascending (fp32);
 * out = bf16_rne(acc).  topk_idx is the routing (device int64 [T, K]); a
 * pair's partition is its expert id / (E/P), whether the layout is expert-
 * or partition-major.  The other arguments are as ep_combine.
 * EP_ERR_UNSUPPORTED when K > 64. */
int ep_combine_reduced(const void *y, int32_t hidden, int64_t num_y_rows, const int64_t *topk_idx,
                       const float *topk_weights, const void *bias0, const void *bias1,
                       const ep_layout_params *params, const ep_layout *layout, void *out,
                       int bf16_partials, void *stream);

/* ep_cast_fp8 - per (token, group) cast of bf16 rows to OCP e4m3
 * ([API] 4.2 per_token_cast_to_fp8, with one scale per group of G channels;
 *  G = hidden is the page's one-scale-per-token form; 3.3 round_scale and
 *  use_ue8m0 through out_dtype).
 *
 *   x         device bf16 [T, hidden], 16-byte aligned, hidden % 16 == 0.
 *   group     G: a power of two in [16, 512] dividing hidden, or hidden.
 *   out_dtype EP_DTYPE_FP8_E4M3, EP_DTYPE_FP8_E4M3_POW2 or
 *             EP_DTYPE_FP8_E4M3_UE8M0 (else EP_ERR_INVALID_ARG).
 *   x_fp8     device uint8 [T, hidden], 16-byte aligned (e4m3fn codes).
 *   scales    device [T, hidden/G]: float (4-byte aligned), or uint8 for UE8M0.
 * amax = max |x| over the group; s = max(amax, 1e-4f) / 448 (fp32, nearest),
 * rounded up to a power of two for POW2 / UE8M0; code = e4m3_rne(x / s)
 * (fp32 nearest division, ties to even, sign kept on underflow).
 * Decode: x ~= float(code) * s. */
int ep_cast_fp8(const void *x, int32_t num_tokens, int32_t hidden, int32_t group,
                int out_dtype, uint8_t *x_fp8, void *scales, void *stream);

/* 10-bit logarithmic combine payload ([API] 3.4: low_latency_combine's
 * use_logfmt, a "10-bit log format" for the expert outputs on their way back;
 * the page fixes only the width, so the format below is this library's
 * reading of it).
 *
 * Values travel in groups of 128 channels of one row.  The log of a bf16
 * magnitude is its 15 magnitude bits read as a fixed-point base-2 logarithm
 * (exponent field, then the stored mantissa as the fraction), rounded half to
 * even to five fraction bits and held at 0x1FDF (bf16 0x7F7C, the largest
 * value kept).  Each group stores its largest log as the reference; a value's
 * 10-bit code is its sign (bit 9) over the index log - reference + 511
 * (bits 0..8): the largest magnitude has index 511; index 0 is zero, used for
 * zeros and for values 511 or more log units (about 16 octaves) under the
 * reference, and keeps the input's sign (-0 and flushed negative values
 * decode to -0).  A group that holds an infinity or NaN has the reference 0xFFFF
 * and all codes 0, and decodes to NaN in its 128 channels.  Decoding is exact:
 * the value is the bf16 number with magnitude bits (reference - 511 + index)
 * << 2, i.e. x rounded to five fraction bits (relative error <= 2^-6 for
 * normal values).
 *
 * Packed row, ep_logfmt_row_bytes(hidden) bytes (a multiple of 128, so rows
 * start on cache lines): bytes [0, H) hold code bits 0..7 of each channel;
 * then H/16 little-endian uint32 words, word v carrying the high bits of
 * channels 16v..16v+15: channel 16v+2p+e (p = 0..7, e = 0 or 1) has its
 * code's bit 8 in bit 7-p+16e and its sign in bit 15-p+16e; then H/128
 * little-endian uint16 references; the tail up to the row size is neither
 * written nor read.  The encoder writes only valid
 * codes; a payload written by anything else decodes to unspecified values
 * (never a memory fault).  hidden must be a positive multiple of 128. */

/* Bytes of one packed payload row, or EP_ERR_INVALID_ARG for a bad hidden. */
int64_t ep_logfmt_row_bytes(int32_t hidden);

/* ep_logfmt_encode - bf16 rows to payload rows.
 *   x        device bf16 [num_rows, hidden], 16-byte aligned.
 *   params, layout  the receive layout the rows belong to, or both NULL.
 *            With a layout only rows that hold a pair (src_of_slot >= 0) are
 *            encoded, the rows a combine reads (the low-latency combine sends
 *            no others); the others keep their payload bytes, so the padding
 *            rows of an aligned layout, or the unused rows of a
 *            fixed-capacity region, cost nothing.  num_rows must not exceed
 *            params->max_recv_rows; the layout writes no src_of_slot entry at
 *            or past its R rows, so rows there are encoded or skipped by
 *            whatever those entries hold (no combine reads them).  When the
 *            pairs (num_tokens * num_topk) fill at most a quarter of num_rows
 *            the encoder launches for a sparse batch (the result is the same).
 *   payload  device uint8 [num_rows, ep_logfmt_row_bytes(hidden)], 16-byte
 *            aligned (caller-owned; may be reused across calls).
 * EP_ERR_INVALID_ARG for a bad hidden, negative num_rows, only one of params
 * and layout, num_rows above max_recv_rows, or a NULL or misaligned x /
 * payload (with num_rows > 0); the layout parameter errors of
 * ep_get_layout. */
int ep_logfmt_encode(const void *x, int64_t num_rows, int32_t hidden,
                     const ep_layout_params *params, const ep_layout *layout, void *payload,
                     void *stream);

/* ep_logfmt_decode - payload rows to bf16 rows (exact; NaN = 0x7FC0 for a
 * marked group).  out: device bf16 [num_rows, hidden], 16-byte aligned.
 * Errors as ep_logfmt_encode. */
int ep_logfmt_decode(const void *payload, int64_t num_rows, int32_t hidden, void *out,
                     void *stream);

/* ep_combine_logfmt - ep_combine over payload rows ([API] 3.4: the weighted
 * low-latency combine with use_logfmt): payload is device uint8 [num_y_rows,
 * ep_logfmt_row_bytes(hidden)], 16-byte aligned, from ep_logfmt_encode of the
 * receive rows.  The result is bit for bit ep_combine over the decoded rows
 * (same fp32 order: biases, then fmaf over kept pairs in ascending k); every
 * other argument, the status bits and the errors are as ep_combine, except
 * that hidden must be a positive multiple of 128. */
int ep_combine_logfmt(const void *payload, int32_t hidden, int64_t num_y_rows,
                      const float *topk_weights, const void *bias0, const void *bias1,
                      const ep_layout_params *params, const ep_layout *layout,
                      const float *recv_topk_weights, float *combined_topk_weights, void *out,
                      void *stream);

/* ep_probe_dispatch_stores - a measurement aid, not a step of the method:
 * the stores of ep_dispatch for bf16 rows (the same row kernel, grid and
 * store order) with each token's row replaced by a fixed pattern held in
 * registers, so that no token row is read.  It shows what the scatter's
 * writes alone cost at a given routing.
 *
 *   hidden       channels per row (bf16), a multiple of 8, at most EP_MAX_HIDDEN.
 *   pattern      the 32-bit word every written row is filled with.
 *   params, layout  as produced by ep_get_layout; only dst_slot and status
 *                are read.
 *   recv_x       device [num_recv_rows, hidden] bf16, 16-byte aligned.
 * Writes recv_x[dst_slot[t,k]] = pattern (every 4-byte word) for every kept
 * pair; padding rows and everything else keep their bytes.  Slots at or past
 * num_recv_rows are skipped and EP_DEV_RECV_OVERFLOW is set.
 * Errors: EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED (hidden > EP_MAX_HIDDEN). */
int ep_probe_dispatch_stores(int32_t hidden, uint32_t pattern, const ep_layout_params *params,
                             const ep_layout *layout, void *recv_x, int64_t num_recv_rows,
                             void *stream);

/* Static description of a status code (never NULL). */
const char *ep_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
