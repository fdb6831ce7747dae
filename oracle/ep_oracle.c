/*
 * CPU oracle for MoE expert-parallel layout / dispatch / combine / fp8 cast.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or helper with the GPU library: every step is written
 * again here from its definition, in plain loops, in the order the pages
 * describe, with no blocking, fusion or reordering.
 *
 * Sources (page titles as cited throughout):
 *   [API]  "DeepEP test target API reference" (DeepEP v2 test page):
 *          sec. 2.1 dispatch() parameter table (topk_idx int64 [T,K] with -1 for
 *          "not selected", topk_weights, num_experts, expert_alignment,
 *          do_expand, do_zero_padding), sec. 2.2 combine() (weighted
 *          reduction back to the source token, optional bias, 0/1/2 of them),
 *          sec. 3.1 V1 layout tensors (num_tokens_per_rank, is_token_in_rank,
 *          num_tokens_per_expert), sec. 3.2 (V1 combine is an unweighted sum),
 *          sec. 4.1 refs (ordered accumulation instead of scatter_add),
 *          sec. 4.2 math (align, ceil_div, per-token cast to e4m3: scale =
 *          amax / fp8_max, codes = x / scale cast to float8_e4m3fn).
 *   [RUST] "spark_model/layers/ep_dispatch.rs" (EP=2 routing table): a
 *          token-major, then k, scan that splits (token, expert, weight)
 *          triples by the owning expert range [start, end).
 *
 * Readings of points the pages leave open (each one is also listed in the
 * design notes of the repository):
 *   - pairs inside one expert's receive segment are in ascending (t, k)
 *     order, i.e. flat index t*K + k ([RUST] scan order);
 *   - padding rows sit at the tail of each expert's segment; an expert with no
 *     pair gets align(0, A) = 0 rows;
 *   - partition-major receive order (partitions standing for ranks): one
 *     segment per partition holding the pairs of its experts in (t, k) order,
 *     padded like an expert's segment;
 *   - an expert id outside [-1, E) is treated as -1 and reported with status
 *     bit 1; in fixed-capacity mode a pair whose rank j >= C is dropped
 *     (dst = -1) and reported with status bit 2;
 *   - fp8: one fp32 scale per (token, group of G channels) (G = H gives the
 *     page's per-token formula), amax floored at 1e-4f, scale = amax / 448 and
 *     code = E4M3(x / scale) with fp32 round-to-nearest division, then OCP
 *     e4m3fn round-to-nearest-even (bias 7, max 448, no infinities, NaN =
 *     S.1111.111, sign kept on underflow); magnitudes from 464 up are NaN;
 *   - combine: acc = 0; acc += bias0; acc += bias1; then for k ascending over
 *     valid pairs acc = fmaf(w, y, acc); out = bf16 round-to-nearest-even;
 *     NULL weights mean w = 1 (the V1 unweighted sum).  A float64 version
 *     gives the tolerance reference;
 *   - the 10-bit log format of the low-latency combine ([API] sec. 3.4): a
 *     sign bit over a 9-bit log index under a per-128-channel reference, the
 *     log being the bf16 magnitude bits rounded to five fraction bits (the
 *     full statement is at the logfmt functions below).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -o liboracle.so ep_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_BAD_EXPERT 1
#define OR_CAPACITY 2
#define OR_RECV_OVERFLOW 4

/* ------------------------------------------------------------------ */
/* [API] sec. 4.2 math: align(x, y) rounds x up to a multiple of y.      */
static int64_t or_align(int64_t x, int64_t y) { return ((x + y - 1) / y) * y; }

/* ------------------------------------------------------------------ */
/* Layout: [API] sec. 2.1 (expert_alignment, do_expand), sec. 3.1
 * (num_tokens_per_expert, is_token_in_rank, num_tokens_per_rank), sec. 3.1
 * "V2 derives the routing from topk_idx"; [RUST] partition by expert range.
 *
 * Inputs: idx int64 [T*K]; T, K, E, A, P (E % P == 0), C (0 = compact),
 * partition_major (0: one receive segment per expert; 1: one per partition,
 * the rank-major receive order of partitions standing for ranks, sec. 3.1).
 * S, the number of segments, is E or P; the segment of expert e is e, or
 * its partition e / (E/P).
 * Outputs (all caller-allocated, host memory):
 *   count [S], offset [S+1], dst [T*K], src_of_slot [rows_cap] (written for
 *   slots < rows_cap), in_part [T*P] (0/1), tok_per_part [P],
 *   pairs_per_part [P], *R_out, *status_out.
 * Returns OR_OK or OR_EINVAL for bad sizes.                                 */
int oracle_get_layout(const int64_t *idx, int64_t T, int64_t K, int64_t E,
                      int64_t A, int64_t P, int64_t C, int64_t partition_major,
                      int32_t *count, int32_t *offset, int32_t *dst,
                      int32_t *src_of_slot, int64_t rows_cap,
                      uint8_t *in_part, int32_t *tok_per_part,
                      int32_t *pairs_per_part, int64_t *R_out, int32_t *status_out)
{
    if (T < 0 || K < 1 || E < 1 || A < 1 || P < 1 || E % P != 0 || C < 0)
        return OR_EINVAL;
    if (C > 0 && C % A != 0)
        return OR_EINVAL;
    if (partition_major != 0 && partition_major != 1)
        return OR_EINVAL;
    int32_t status = 0;
    int64_t m = E / P;
    int64_t S = partition_major ? P : E;         /* receive segments */
    int64_t seg_div = partition_major ? m : 1;   /* segment of expert e: e / seg_div */

    /* O-1: count[s] = number of (t, k) whose expert idx[t, k] lies in
     * segment s. */
    for (int64_t s = 0; s < S; ++s) count[s] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = idx[t * K + k];
            if (e == -1) continue;
            if (e < -1 || e >= E) { status |= OR_BAD_EXPERT; continue; }
            count[e / seg_div] += 1;
        }
    }

    /* O-2: padded[s] = align(count[s], A); offsets are the exclusive scan
     * of the padded counts (compact) or s*C (fixed capacity). */
    int64_t R;
    if (C == 0) {
        offset[0] = 0;
        for (int64_t s = 0; s < S; ++s)
            offset[s + 1] = (int32_t)(offset[s] + or_align(count[s], A));
        R = offset[S];
    } else {
        for (int64_t s = 0; s <= S; ++s) offset[s] = (int32_t)(s * C);
        R = S * C;
        for (int64_t s = 0; s < S; ++s)
            if (count[s] > C) status |= OR_CAPACITY;
    }
    if (R > rows_cap) status |= OR_RECV_OVERFLOW;

    /* O-3: the j-th pair of segment s, in ascending (t, k) order, takes slot
     * offset[s] + j.  Walk the pairs in that order with one cursor per
     * segment. */
    int32_t *cursor = (int32_t *)calloc((size_t)S, sizeof(int32_t));
    if (!cursor) return OR_EINVAL;
    for (int64_t r = 0; r < R && r < rows_cap; ++r) src_of_slot[r] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t p = t * K + k;
            int64_t e = idx[p];
            dst[p] = -1;
            if (e < 0 || e >= E) continue;
            int64_t s = e / seg_div;
            int64_t j = cursor[s]++;
            if (C > 0 && j >= C) continue;       /* dropped by capacity */
            int64_t slot = offset[s] + j;
            dst[p] = (int32_t)slot;
            if (slot < rows_cap) src_of_slot[slot] = (int32_t)p;
        }
    }
    free(cursor);

    /* O-4: partition q owns experts [q*m, (q+1)*m). */
    for (int64_t q = 0; q < P; ++q) { tok_per_part[q] = 0; pairs_per_part[q] = 0; }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t q = 0; q < P; ++q) in_part[t * P + q] = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = idx[t * K + k];
            if (e < 0 || e >= E) continue;
            in_part[t * P + e / m] = 1;
        }
        for (int64_t q = 0; q < P; ++q) tok_per_part[q] += in_part[t * P + q];
    }
    for (int64_t e = 0; e < E; ++e) pairs_per_part[e / m] += count[e];

    *R_out = R;
    *status_out = status;
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Dispatch rows: [API] sec. 2.1 - recv_x has the type of x; in fp8 mode x
 * is (codes, scales) and both travel.  recv[dst[t,k]] = x[t] byte for byte.
 * Padding slots (src_of_slot == -1) are zero-filled only when asked
 * (do_zero_padding); recv_w padding is 0.
 *   x [T, row_bytes], xs [T, srow_bytes] (nullable), w [T*K] (nullable).
 *   recv [R, row_bytes], recv_s [R, srow_bytes], recv_w [R].             */
void oracle_dispatch(const uint8_t *x, int64_t row_bytes, const uint8_t *xs,
                     int64_t srow_bytes, const float *w, int64_t T, int64_t K,
                     const int32_t *dst, const int32_t *src_of_slot, int64_t R,
                     int zero_padding, uint8_t *recv, uint8_t *recv_s, float *recv_w)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t slot = dst[t * K + k];
            if (slot < 0 || slot >= R) continue;
            memcpy(recv + slot * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            if (xs && recv_s)
                memcpy(recv_s + slot * srow_bytes, xs + t * srow_bytes, (size_t)srow_bytes);
            if (recv_w) recv_w[slot] = w ? w[t * K + k] : 1.0f;
        }
    }
    for (int64_t s = 0; s < R; ++s) {
        if (src_of_slot[s] >= 0) continue;
        if (recv_w) recv_w[s] = 0.0f;
        if (zero_padding) {
            memset(recv + s * row_bytes, 0, (size_t)row_bytes);
            if (recv_s) memset(recv_s + s * srow_bytes, 0, (size_t)srow_bytes);
        }
    }
}

/* ------------------------------------------------------------------ */
/* bf16: 1 sign, 8 exponent, 7 stored mantissa bits (the upper half of an
 * IEEE-754 binary32).  Widening is exact. */
float oracle_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary32 value to bf16, nearest, ties to even, from the
 * definition: find the quantum of v's binade (8 significant bits), divide,
 * round half to even on the integer multiple, scale back.  Done in double,
 * where every step below is exact. */
uint16_t oracle_bf16_from_float(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
    double a = fabs((double)v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                  /* a = f * 2^e, f in [0.5, 1) */
    int qexp = e - 8;              /* 8 significant bits */
    if (qexp < -133) qexp = -133;  /* bf16 subnormal quantum 2^-133 */
    double n = ldexp(a, -qexp);
    double lo = floor(n);
    double fr = n - lo;
    double r = lo;
    if (fr > 0.5 || (fr == 0.5 && fmod(lo, 2.0) != 0.0)) r = lo + 1.0;
    double res = ldexp(r, qexp);
    if (res >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)res;         /* exact: res has <= 8 significant bits */
    uint32_t ru;
    memcpy(&ru, &rf, 4);
    return (uint16_t)(sign | (ru >> 16));
}

/* ------------------------------------------------------------------ */
/* OCP 8-bit floating point, E4M3 ("float8_e4m3fn"): exponent bias 7, three
 * mantissa bits, normal range 2^-6 .. 448, subnormal step 2^-9, no
 * infinities, S.1111.111 is NaN. */
float oracle_e4m3_to_float(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 15, mt = c & 7;
    double v;
    if (ex == 15 && mt == 7) return NAN;
    if (ex == 0) v = ldexp((double)mt, -9);
    else v = ldexp(1.0 + mt / 8.0, ex - 7);
    return (float)(s ? -v : v);
}

/* Nearest e4m3 value, ties to the even mantissa, from the definition:
 * quantum of the binade (2^(e-3) for normals, 2^-9 below 2^-6), integer
 * rounding, then re-encode.  Magnitudes >= 464 (the midpoint above 448 that
 * ties to 448, and everything past it) have no finite neighbour: NaN. */
uint8_t oracle_e4m3_from_float(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a > 464.0) return (uint8_t)(sign | 0x7F);
    int qexp;
    if (a < ldexp(1.0, -6)) {
        qexp = -9;
    } else {
        int e;
        frexp(a, &e);              /* a in [2^(e-1), 2^e) */
        qexp = (e - 1) - 3;
    }
    double n = ldexp(a, -qexp);
    double lo = floor(n);
    double fr = n - lo;
    double r = lo;
    if (fr > 0.5 || (fr == 0.5 && fmod(lo, 2.0) != 0.0)) r = lo + 1.0;
    double res = ldexp(r, qexp);   /* the chosen e4m3 magnitude */
    if (res == 0.0) return sign;
    if (res < ldexp(1.0, -6)) {
        int mt = (int)ldexp(res, 9);                 /* 1..7 */
        return (uint8_t)(sign | mt);
    }
    int e;
    double f = frexp(res, &e);     /* res = f * 2^e, f in [0.5, 1) */
    int ex = (e - 1) + 7;
    int mt = (int)((f * 2.0 - 1.0) * 8.0);
    if (ex > 15 || (ex == 15 && mt == 7)) return (uint8_t)(sign | 0x7F);
    return (uint8_t)(sign | (ex << 3) | mt);
}

/* [API] sec. 4.2 per-token cast to fp8, with one scale per (token, group of
 * G channels): a = max |x| over the group (exact), a' = max(a, 1e-4f),
 * s = a' / 448 (fp32, nearest), q = E4M3(x / s) (fp32 nearest division).
 *   x bf16 bits [T, H]; q [T, H]; scales [T, H/G].                       */
int oracle_cast_fp8(const uint16_t *x, int64_t T, int64_t H, int64_t G,
                    uint8_t *q, float *scales)
{
    if (T < 0 || H < 1 || G < 1 || H % G != 0) return OR_EINVAL;
    int64_t ng = H / G;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g = 0; g < ng; ++g) {
            float amax = 0.0f;
            for (int64_t c = g * G; c < (g + 1) * G; ++c) {
                float a = fabsf(oracle_bf16_to_float(x[t * H + c]));
                if (a > amax) amax = a;
            }
            volatile float ap = amax > 1e-4f ? amax : 1e-4f;
            volatile float s = ap / 448.0f;
            scales[t * ng + g] = s;
            for (int64_t c = g * G; c < (g + 1) * G; ++c) {
                volatile float xv = oracle_bf16_to_float(x[t * H + c]);
                volatile float d = xv / s;
                q[t * H + c] = oracle_e4m3_from_float(d);
            }
        }
    }
    return OR_OK;
}

/* Low-latency scale formats ([API] 3.3 low_latency_dispatch: round_scale
 * rounds the scale to a power of two; use_ue8m0 stores it as UE8M0).
 * Readings: the power of two is the smallest one >= amax'/448 (rounding up
 * keeps |x| / scale <= 448, so no code overflows), taken on the fp32 quotient;
 * UE8M0 is an unsigned 8-bit biased exponent b with value 2^(b - 127), one
 * byte per (token, group).  Codes are E4M3(x / scale) as before; with a
 * power-of-two scale the division is exact.
 * fmt 1: fp32 power-of-two scales into scales_f32; fmt 2: UE8M0 bytes into
 * scales_e8 (and, when non-NULL, the same scales as fp32 into scales_f32). */
float oracle_pow2_ceil(float s)
{
    int e;
    float m = frexpf(s, &e);          /* s = m * 2^e, m in [0.5, 1) */
    return m == 0.5f ? s : ldexpf(1.0f, e);
}

uint8_t oracle_ue8m0_of(float pow2)
{
    int e;
    frexpf(pow2, &e);                 /* pow2 = 0.5 * 2^e = 2^(e-1) */
    return (uint8_t)(e - 1 + 127);
}

float oracle_ue8m0_to_float(uint8_t b)
{
    return ldexpf(1.0f, (int)b - 127);
}

int oracle_cast_fp8_pow2(const uint16_t *x, int64_t T, int64_t H, int64_t G, int fmt,
                         uint8_t *q, float *scales_f32, uint8_t *scales_e8)
{
    if (T < 0 || H < 1 || G < 1 || H % G != 0 || (fmt != 1 && fmt != 2)) return OR_EINVAL;
    int64_t ng = H / G;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g = 0; g < ng; ++g) {
            float amax = 0.0f;
            for (int64_t c = g * G; c < (g + 1) * G; ++c) {
                float a = fabsf(oracle_bf16_to_float(x[t * H + c]));
                if (a > amax) amax = a;
            }
            volatile float ap = amax > 1e-4f ? amax : 1e-4f;
            volatile float s0 = ap / 448.0f;
            float s = oracle_pow2_ceil(s0);
            if (scales_f32) scales_f32[t * ng + g] = s;
            if (fmt == 2 && scales_e8) scales_e8[t * ng + g] = oracle_ue8m0_of(s);
            for (int64_t c = g * G; c < (g + 1) * G; ++c) {
                volatile float xv = oracle_bf16_to_float(x[t * H + c]);
                volatile float d = xv / s;
                q[t * H + c] = oracle_e4m3_from_float(d);
            }
        }
    }
    return OR_OK;
}

/* Decode (the page's per_token_cast_back): x^ = float(q) * s, in fp32. */
void oracle_cast_back(const uint8_t *q, const float *scales, int64_t T,
                      int64_t H, int64_t G, float *out)
{
    int64_t ng = H / G;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c)
            out[t * H + c] = oracle_e4m3_to_float(q[t * H + c]) * scales[t * ng + c / G];
}

/* ------------------------------------------------------------------ */
/* Combine: [API] sec. 2.2 weighted reduction back to the source token with
 * 0/1/2 biases; sec. 3.2 NULL weights = unweighted sum; sec. 4.1 ordered
 * accumulation.  Rows of y are read at dst[t,k] for every valid pair.
 * `tokens` (nullable) restricts the output to the listed tokens: out row i
 * holds token tokens[i] (all T tokens in order when NULL).
 *   y bf16 [*, H]; w [T*K] nullable; bias0/bias1 bf16 [T, H] nullable.   */
void oracle_combine_f64(const uint16_t *y, int64_t H, const float *w,
                        const uint16_t *bias0, const uint16_t *bias1,
                        int64_t T, int64_t K, const int32_t *dst,
                        const int64_t *tokens, int64_t n_out, double *out)
{
    int64_t n = tokens ? n_out : T;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            if (bias0) acc += (double)oracle_bf16_to_float(bias0[t * H + c]);
            if (bias1) acc += (double)oracle_bf16_to_float(bias1[t * H + c]);
            for (int64_t k = 0; k < K; ++k) {
                int64_t slot = dst[t * K + k];
                if (slot < 0) continue;
                double wk = w ? (double)w[t * K + k] : 1.0;
                acc += wk * (double)oracle_bf16_to_float(y[slot * H + c]);
            }
            out[i * H + c] = acc;
        }
    }
}

void oracle_combine_f32(const uint16_t *y, int64_t H, const float *w,
                        const uint16_t *bias0, const uint16_t *bias1,
                        int64_t T, int64_t K, const int32_t *dst,
                        const int64_t *tokens, int64_t n_out, uint16_t *out)
{
    int64_t n = tokens ? n_out : T;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t c = 0; c < H; ++c) {
            volatile float acc = 0.0f;
            if (bias0) acc = acc + oracle_bf16_to_float(bias0[t * H + c]);
            if (bias1) acc = acc + oracle_bf16_to_float(bias1[t * H + c]);
            for (int64_t k = 0; k < K; ++k) {
                int64_t slot = dst[t * K + k];
                if (slot < 0) continue;
                float wk = w ? w[t * K + k] : 1.0f;
                acc = fmaf(wk, oracle_bf16_to_float(y[slot * H + c]), acc);
            }
            out[i * H + c] = oracle_bf16_from_float(acc);
        }
    }
}

/* combined_topk_weights[t,k] = recv_w[dst[t,k]] for valid pairs, else 0. */
void oracle_combined_weights(const float *recv_w, int64_t T, int64_t K,
                             const int32_t *dst, float *out)
{
    for (int64_t p = 0; p < T * K; ++p)
        out[p] = dst[p] >= 0 ? recv_w[dst[p]] : 0.0f;
}

/* Array forms of the scalar conversions (for exhaustive tests). */
void oracle_e4m3_from_float_n(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_float(v[i]);
}

void oracle_bf16_from_float_n(const float *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_float(v[i]);
}

void oracle_div_f32_n(const float *a, const float *b, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) {
        volatile float q = a[i] / b[i];
        out[i] = q;
    }
}

/* ------------------------------------------------------------------ */
/* Partition ("rank") receive layout, the non-expanded form: [API] sec. 2.1
 * (do_expand = False: a token travels once to every rank that owns one of
 * its experts; recv_topk_idx / recv_topk_weights come with it), sec. 3.1
 * (is_token_in_rank, num_tokens_per_rank, num_tokens_per_rdma_rank).
 * Readings: partition q's rows are [part_offset[q], part_offset[q+1]) with
 * part_offset the exclusive scan of the per-partition token counts, tokens
 * in ascending t, no padding; a group is G consecutive partitions (G = P:
 * one group) and counts the tokens that reach any partition in it.
 *   token_slot [T*P]: receive row of (t, q), or -1.                       */
int oracle_partition_layout(const int64_t *idx, int64_t T, int64_t K, int64_t E, int64_t P,
                            int64_t G, uint8_t *in_part, int32_t *tok_per_part,
                            int32_t *part_offset, int32_t *token_slot,
                            int32_t *tok_per_group, int32_t *part_src, int64_t *Rp_out)
{
    if (T < 0 || K < 1 || E < 1 || P < 1 || E % P != 0 || G < 1 || P % G != 0) return OR_EINVAL;
    int64_t m = E / P;
    for (int64_t q = 0; q < P; ++q) tok_per_part[q] = 0;
    for (int64_t n = 0; n < P / G; ++n) tok_per_group[n] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t q = 0; q < P; ++q) in_part[t * P + q] = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = idx[t * K + k];
            if (e < 0 || e >= E) continue;
            in_part[t * P + e / m] = 1;
        }
        for (int64_t q = 0; q < P; ++q) tok_per_part[q] += in_part[t * P + q];
        for (int64_t n = 0; n < P / G; ++n) {
            int hit = 0;
            for (int64_t q = n * G; q < (n + 1) * G; ++q) hit |= in_part[t * P + q];
            tok_per_group[n] += hit;
        }
    }
    part_offset[0] = 0;
    for (int64_t q = 0; q < P; ++q) part_offset[q + 1] = part_offset[q] + tok_per_part[q];
    int32_t *cursor = (int32_t *)calloc((size_t)P, sizeof(int32_t));
    if (!cursor) return OR_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t q = 0; q < P; ++q) {
            token_slot[t * P + q] = in_part[t * P + q] ? part_offset[q] + cursor[q]++ : -1;
            /* the inverse: the token each partition row holds */
            if (part_src && token_slot[t * P + q] >= 0) part_src[token_slot[t * P + q]] = (int32_t)t;
        }
    free(cursor);
    *Rp_out = part_offset[P];
    return OR_OK;
}

/* Non-expanded dispatch: recv[token_slot[t,q]] = x[t] (and its scales);
 * recv_idx[row, k] = e - q*m when pair (t,k) belongs to partition q (its
 * expert's id local to the partition), else -1; recv_w[row, k] = w[t,k]
 * (1 without weights) for local pairs, else 0.                            */
void oracle_dispatch_partitioned(const uint8_t *x, int64_t row_bytes, const uint8_t *xs,
                                 int64_t srow_bytes, const int64_t *idx, const float *w,
                                 int64_t T, int64_t K, int64_t E, int64_t P,
                                 const int32_t *token_slot, int64_t Rp, uint8_t *recv,
                                 uint8_t *recv_s, int64_t *recv_idx, float *recv_w)
{
    int64_t m = E / P;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t q = 0; q < P; ++q) {
            int64_t row = token_slot[t * P + q];
            if (row < 0 || row >= Rp) continue;
            memcpy(recv + row * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            if (xs && recv_s)
                memcpy(recv_s + row * srow_bytes, xs + t * srow_bytes, (size_t)srow_bytes);
            for (int64_t k = 0; k < K; ++k) {
                int64_t e = idx[t * K + k];
                int local = e >= 0 && e < E && e / m == q;
                if (recv_idx) recv_idx[row * K + k] = local ? e - q * m : -1;
                if (recv_w) recv_w[row * K + k] = local ? (w ? w[t * K + k] : 1.0f) : 0.0f;
            }
        }
    }
}

/* Combine for the non-expanded layout ([API] sec. 3.2: a plain sum; the
 * rows already carry their partition's weighted expert sum):
 * acc = 0; acc += bias0; acc += bias1; for q ascending with a row:
 * acc += y[row]; out = bf16(acc).  float64 variant for the tolerance.    */
void oracle_combine_partitioned_f32(const uint16_t *y, int64_t H, const uint16_t *bias0,
                                    const uint16_t *bias1, int64_t T, int64_t P,
                                    const int32_t *token_slot, const int64_t *tokens,
                                    int64_t n_out, uint16_t *out)
{
    int64_t n = tokens ? n_out : T;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t c = 0; c < H; ++c) {
            volatile float acc = 0.0f;
            if (bias0) acc = acc + oracle_bf16_to_float(bias0[t * H + c]);
            if (bias1) acc = acc + oracle_bf16_to_float(bias1[t * H + c]);
            for (int64_t q = 0; q < P; ++q) {
                int64_t row = token_slot[t * P + q];
                if (row < 0) continue;
                acc = acc + oracle_bf16_to_float(y[row * H + c]);
            }
            out[i * H + c] = oracle_bf16_from_float(acc);
        }
    }
}

void oracle_combine_partitioned_f64(const uint16_t *y, int64_t H, const uint16_t *bias0,
                                    const uint16_t *bias1, int64_t T, int64_t P,
                                    const int32_t *token_slot, const int64_t *tokens,
                                    int64_t n_out, double *out)
{
    int64_t n = tokens ? n_out : T;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            if (bias0) acc += (double)oracle_bf16_to_float(bias0[t * H + c]);
            if (bias1) acc += (double)oracle_bf16_to_float(bias1[t * H + c]);
            for (int64_t q = 0; q < P; ++q) {
                int64_t row = token_slot[t * P + q];
                if (row >= 0) acc += (double)oracle_bf16_to_float(y[row * H + c]);
            }
            out[i * H + c] = acc;
        }
    }
}

/* "Reduced" combine on the expanded layout ([API] sec. 2.2: reduced combine,
 * multi-level reduction under allow_multiple_reduction).  Reading: level 1
 * sums a token's pairs inside each partition (k ascending, fp32 fmaf from
 * 0); level 2 adds bias0, bias1, then the partials for q ascending (fp32),
 * and rounds to bf16.  The page gives the partials no rounding, so they stay
 * fp32; with bf16_partials each partial is first rounded to bf16, the dtype
 * it would travel in between ranks.  The float64 reference is
 * oracle_combine_f64.                                                      */
void oracle_combine_reduced_f32(const uint16_t *y, int64_t H, const int64_t *idx,
                                const float *w, const uint16_t *bias0, const uint16_t *bias1,
                                int64_t T, int64_t K, int64_t E, int64_t P, const int32_t *dst,
                                int bf16_partials, const int64_t *tokens, int64_t n_out,
                                uint16_t *out)
{
    int64_t m = E / P;
    int64_t n = tokens ? n_out : T;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t c = 0; c < H; ++c) {
            volatile float acc = 0.0f;
            if (bias0) acc = acc + oracle_bf16_to_float(bias0[t * H + c]);
            if (bias1) acc = acc + oracle_bf16_to_float(bias1[t * H + c]);
            for (int64_t q = 0; q < P; ++q) {
                int any = 0;
                volatile float part = 0.0f;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t e = idx[t * K + k];
                    int64_t slot = dst[t * K + k];
                    if (e < 0 || e >= E || e / m != q || slot < 0) continue;
                    any = 1;
                    float wk = w ? w[t * K + k] : 1.0f;
                    part = fmaf(wk, oracle_bf16_to_float(y[slot * H + c]), part);
                }
                if (!any) continue;
                if (bf16_partials) acc = acc + oracle_bf16_to_float(oracle_bf16_from_float(part));
                else acc = acc + part;
            }
            out[i * H + c] = oracle_bf16_from_float(acc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* 10-bit logarithmic combine payload ([API] sec. 3.4: low_latency_combine's
 * use_logfmt option, a "10-bit log format" for the expert outputs sent back
 * to their tokens; the page fixes only the width).  Reading:
 *   - values travel in groups of 128 channels of one row (the grouping of the
 *     same API's fp8 payload, sec. 4.2), with one 16-bit reference per group;
 *   - the log of a bf16 magnitude is its 15 magnitude bits read as a
 *     fixed-point base-2 logarithm (exponent field, then the stored mantissa
 *     as the fraction: Mitchell's piecewise-linear log2, exact at powers of
 *     two), rounded to five fractional bits, nearest, ties to even, and held
 *     at the largest finite value 0x1FDF (bf16 0x7F7C);
 *   - the reference is the group's largest log; a value's code is its sign
 *     bit over a 9-bit index = log - reference + 511, so the largest
 *     magnitude maps to 511; index 0 is zero, for zeros, for logs of 0 and for
 *     values more than 510/32 log units below the reference (flushed); a zero
 *     keeps the sign of its input, so -0 and flushed negative values come
 *     back as -0 (as e4m3 keeps the sign on underflow in the fp8 cast);
 *   - a group holding an infinity or NaN has the reference 0xFFFF and all
 *     codes 0; it decodes to NaN in all 128 channels;
 *   - decoding is exact: sign, then magnitude bits (reference - 511 + index)
 *     shifted left by two (0 for index 0), a bf16 number with five fraction
 *     bits. */
#define OR_LOGFMT_GROUP 128
#define OR_LOGFMT_MAXLOG 0x1FDF
#define OR_LOGFMT_POISON 0xFFFF

/* Log code of a bf16 pattern, -1 for an infinity or NaN. */
int32_t oracle_logfmt_log(uint16_t b)
{
    uint32_t u = b & 0x7FFFu;
    if (u >= 0x7F80u) return -1;
    uint32_t q = u / 4, r = u % 4;
    if (r > 2 || (r == 2 && q % 2 == 1)) q += 1;
    if (q > OR_LOGFMT_MAXLOG) q = OR_LOGFMT_MAXLOG;
    return (int32_t)q;
}

/* codes [rows, H] (10-bit values in uint16), refs [rows, H/128]. */
int oracle_logfmt_encode(const uint16_t *x, int64_t rows, int64_t H, uint16_t *codes,
                         uint16_t *refs)
{
    if (H <= 0 || H % OR_LOGFMT_GROUP != 0 || rows < 0) return OR_EINVAL;
    int64_t G = H / OR_LOGFMT_GROUP;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *xs = x + r * H + g * OR_LOGFMT_GROUP;
            uint16_t *cs = codes + r * H + g * OR_LOGFMT_GROUP;
            int poison = 0;
            int32_t top = 0;
            for (int c = 0; c < OR_LOGFMT_GROUP; ++c) {
                int32_t l = oracle_logfmt_log(xs[c]);
                if (l < 0) poison = 1;
                else if (l > top) top = l;
            }
            refs[r * G + g] = (uint16_t)(poison ? OR_LOGFMT_POISON : top);
            for (int c = 0; c < OR_LOGFMT_GROUP; ++c) {
                uint16_t code = 0;
                if (!poison) {
                    int32_t l = oracle_logfmt_log(xs[c]);
                    int32_t idx = l - top + 511;
                    if (l < 1 || idx < 1) idx = 0;
                    code = (uint16_t)(idx | ((xs[c] & 0x8000u) ? 512 : 0));
                }
                cs[c] = code;
            }
        }
    }
    return OR_OK;
}

/* bf16 patterns [rows, H] from codes and refs; OR_EINVAL for a code or
 * reference the encoder never writes. */
int oracle_logfmt_decode(const uint16_t *codes, const uint16_t *refs, int64_t rows, int64_t H,
                         uint16_t *out)
{
    if (H <= 0 || H % OR_LOGFMT_GROUP != 0 || rows < 0) return OR_EINVAL;
    int64_t G = H / OR_LOGFMT_GROUP;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < H; ++c) {
            uint16_t ref = refs[r * G + c / OR_LOGFMT_GROUP];
            uint16_t code = codes[r * H + c];
            if (code > 1023) return OR_EINVAL;
            if (ref == OR_LOGFMT_POISON) {
                if (code != 0) return OR_EINVAL;
                out[r * H + c] = 0x7FC0u;
                continue;
            }
            if (ref > OR_LOGFMT_MAXLOG) return OR_EINVAL;
            int32_t idx = code & 511, sign = code >> 9;
            if (idx == 0) {
                out[r * H + c] = (uint16_t)(sign ? 0x8000u : 0u);
                continue;
            }
            int32_t n = (int32_t)ref - 511 + idx;
            if (n < 1 || n > OR_LOGFMT_MAXLOG) return OR_EINVAL;
            out[r * H + c] = (uint16_t)((sign ? 0x8000u : 0u) | ((uint32_t)n << 2));
        }
    }
    return OR_OK;
}
