/*
 * CPU oracle for the MoE dispatch layout, token pack, handle reuse and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only through the seeded input arrays.
 *
 * Plain, slow, scalar C written to be checked by eye against the pages:
 *   [EO]  "How DeepEP Achieves Communication-Computation Overlapping with
 *          EventOverlap"
 *   [HK]  "How DeepEP Enables Hook-Based Overlapping Without SM Occupation"
 *   [GCU] the EnflameTechnology/DeepEP README (GCU port): the normal-kernel
 *          example (dispatch_forward / combine_forward / ..._backward), the
 *          low-latency example and the feature notes
 *   [HR]  "How DeepEP Optimizes Handle Reuse for Repeated Dispatches"
 *
 * Notation: T tokens, H hidden, K top-k slots, E experts, R logical ranks
 * (expert-group buckets), P = E / R experts per bucket, C channels.
 * Expert e lives in bucket b(e) = e / P (contiguous blocks; the low-latency
 * example asserts num_experts % num_ranks == 0 and gives each rank
 * num_experts / num_ranks experts).
 *
 * Floating point: the combine is an fp32 accumulation in fixed top-k order with
 * one bf16 round-to-nearest-even at the end; the FP8 path is an fp32 per-1x128
 * amax scale and OCP E4M3FN codes.  Build with -O2 -ffp-contract=off so that
 * every multiply-add is either an explicit fmaf() or two rounded operations.
 *
 * Parity pins (tests/): hand-worked routings, library special cases
 * (bincount, cumsum, nonzero, index_select, torch's bf16 and float8_e4m3fn
 * casts), invariants and closed forms.  Parity unpinned: whether send_head,
 * recv_channel_prefix_matrix and rank_prefix_matrix carry exactly the meaning
 * of upstream code the pages only name (our definitions are pinned, fidelity
 * to unseen code is not); the 1e-4 amax floor of the FP8 scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* bf16 = the top 16 bits of an fp32.  Round to nearest, ties to even, written
 * as "pick the nearer of the two bf16 neighbours"; NaN stays NaN (quiet, sign
 * kept); above the largest finite value the upper neighbour is +/-inf, whose
 * distance is measured as if it were 2^128 (IEEE overflow rule). */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    if ((u & 0x7fffffffu) == 0x7f800000u) return (uint16_t)(u >> 16);
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7fffffffu;
    uint32_t lo = mag & 0xffff0000u;          /* neighbour toward zero */
    uint32_t hi = lo + 0x10000u;              /* neighbour away from zero */
    double a = (double)f32_from_bits(mag);
    double vlo = (double)f32_from_bits(lo);
    double vhi = (hi >= 0x7f800000u) ? ldexp(1.0, 128) : (double)f32_from_bits(hi);
    double dlo = a - vlo, dhi = vhi - a;
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;  /* tie: even last bit */
    return (uint16_t)((sign | pick) >> 16);
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;
 * 0x7F / 0xFF are NaN; the largest finite magnitude is code 0x7E = 448. */
float oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);                 /* subnormal m * 2^-9 */
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3FN code to v, ties to the even code, |v| >= 448 saturates to
 * +/-448 (0x7E / 0xFE), NaN -> 0x7F, the sign of zero is kept.
 * The non-negative finite codes 0x00..0x7E are strictly increasing in value,
 * so the nearest code is one of the two that bracket |v|. */
uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v)) return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    uint8_t code;
    if (a >= 448.0) {
        code = 0x7e;
    } else {
        int lo = 0, hi = 0x7e;                 /* largest c with value(c) <= a */
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if ((double)oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
        }
        int c = lo;
        double d0 = a - (double)oracle_e4m3_decode((uint8_t)c);
        double d1 = (double)oracle_e4m3_decode((uint8_t)(c + 1)) - a;
        if (d0 < d1) code = (uint8_t)c;
        else if (d1 < d0) code = (uint8_t)(c + 1);
        else code = (uint8_t)((c & 1) ? c + 1 : c);
    }
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* Dispatch layout  ([GCU] normal-kernel example, get_dispatch_layout)       */
/* ------------------------------------------------------------------------ */

/* Per-token routing to buckets and experts.
 *   num_tokens_per_expert[e] = number of (t,k) with topk_idx[t,k] == e
 *   is_token_in_rank[t,r]    = 1 iff some valid slot of t has b(expert) == r
 *   num_tokens_per_rank[r]   = number of tokens t with is_token_in_rank[t,r]
 * A slot holding -1 is empty and ignored.  Returns 0, or -1 on an expert id
 * outside {-1} u [0,E) or a token that names one expert twice. */
int oracle_layout(const int64_t *topk_idx, int64_t T, int K, int E, int R,
                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                  uint8_t *is_token_in_rank)
{
    int P = E / R;
    for (int r = 0; r < R; ++r) num_tokens_per_rank[r] = 0;
    for (int e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r) is_token_in_rank[t * R + r] = 0;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) { if (e != -1) return -1; continue; }
            if (e >= E) return -1;
            for (int k2 = 0; k2 < k; ++k2)
                if (topk_idx[t * K + k2] == e) return -1;
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + (int)(e / P)] = 1;
        }
        for (int r = 0; r < R; ++r) num_tokens_per_rank[r] += is_token_in_rank[t * R + r];
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Handle contents  ([HR] What the Handle Contains)                          */
/* ------------------------------------------------------------------------ */

/* Start row of bucket r in the receive buffer. */
static int64_t bucket_base(const int32_t *rank_prefix_matrix, int r)
{
    return r == 0 ? 0 : rank_prefix_matrix[r - 1];
}

/* Receive layout of one GPU's tokens across its buckets.
 *
 * Channels are contiguous token ranges: per = ceil(T / C), channel c owns
 * tokens [min(c*per, T), min((c+1)*per, T)); trailing channels may be empty.
 * Rows of the receive buffer are bucket-major; inside a bucket they follow
 * channel order and token order inside a channel, i.e. ascending token id.
 *
 *   rank_prefix_matrix[r]           = sum_{r' <= r} num_tokens_per_rank[r'] (inclusive)
 *   channel_prefix_matrix[r][c]     = sum_{c' <= c} n[r][c']               (inclusive)
 *   recv_channel_prefix_matrix[r][c]= channel_prefix_matrix[r][c] - n[r][c] (exclusive)
 *   send_head[t][r]                 = #{t' < t : in[t'][r]} if in[t][r], else -1
 *   recv_src_idx[base[r] + send_head[t][r]] = t,  base[r] = rank_prefix_matrix[r] - count[r]
 * where n[r][c] counts the tokens of channel c routed to bucket r.
 * *n_recv receives N = rank_prefix_matrix[R-1] (0 when R == 0). */
void oracle_prefix(const uint8_t *in, int64_t T, int R, int C,
                   int32_t *rank_prefix_matrix, int32_t *channel_prefix_matrix,
                   int32_t *recv_channel_prefix_matrix, int32_t *send_head,
                   int32_t *recv_src_idx, int64_t *n_recv)
{
    int64_t per = (T + C - 1) / C;
    int64_t running = 0;
    for (int r = 0; r < R; ++r) {
        int64_t count = 0;                          /* tokens so far in bucket r */
        for (int c = 0; c < C; ++c) {
            int64_t t0 = c * per < T ? c * per : T;
            int64_t t1 = (c + 1) * per < T ? (c + 1) * per : T;
            int64_t n_rc = 0;
            for (int64_t t = t0; t < t1; ++t) n_rc += in[t * R + r];
            recv_channel_prefix_matrix[r * C + c] = (int32_t)count;
            count += n_rc;
            channel_prefix_matrix[r * C + c] = (int32_t)count;
        }
        running += count;
        rank_prefix_matrix[r] = (int32_t)running;
    }
    for (int r = 0; r < R; ++r) {
        int64_t base = bucket_base(rank_prefix_matrix, r);
        int64_t seen = 0;                           /* earlier tokens in bucket r */
        for (int64_t t = 0; t < T; ++t) {
            if (in[t * R + r]) {
                send_head[t * R + r] = (int32_t)seen;
                recv_src_idx[base + seen] = (int32_t)t;
                seen += 1;
            } else {
                send_head[t * R + r] = -1;
            }
        }
    }
    *n_recv = R ? rank_prefix_matrix[R - 1] : 0;
}

/* ------------------------------------------------------------------------ */
/* Token pack  ([GCU] dispatch_forward; [HR] First Dispatch)                 */
/* ------------------------------------------------------------------------ */

/* recv_x[row(t,r)] = x[t] bit for bit, for every bucket r of token t.
 * recv_topk_idx[row,k]   = topk_idx[t,k] - r*P if that expert is in bucket r, else -1
 * recv_topk_weights[row,k] = topk_weights[t,k] under the same condition, else +0.0f
 * recv_topk_idx / recv_topk_weights / topk_weights may be NULL (handle reuse
 * produces rows only). */
void oracle_pack_bf16(const uint16_t *x, int64_t T, int64_t H,
                      const int64_t *topk_idx, const float *topk_weights, int K, int E, int R,
                      const int32_t *send_head, const int32_t *rank_prefix_matrix,
                      uint16_t *recv_x, int64_t *recv_topk_idx, float *recv_topk_weights)
{
    int P = E / R;
    for (int64_t t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r) {
            int32_t pos = send_head[t * R + r];
            if (pos < 0) continue;
            int64_t row = bucket_base(rank_prefix_matrix, r) + pos;
            for (int64_t h = 0; h < H; ++h) recv_x[row * H + h] = x[t * H + h];
            if (recv_topk_idx) {
                for (int k = 0; k < K; ++k) {
                    int64_t e = topk_idx[t * K + k];
                    int mine = e >= 0 && (int)(e / P) == r;
                    recv_topk_idx[row * K + k] = mine ? e - (int64_t)r * P : -1;
                    if (recv_topk_weights)
                        recv_topk_weights[row * K + k] = mine ? topk_weights[t * K + k] : 0.0f;
                }
            }
        }
    }
}

/* FP8 dispatch with a per-group scale ([GCU] feature notes: FP8 dispatch with
 * per-group scales).  Groups are 1x128 blocks of a row.  For block j of token t:
 *   a = max |x| over the block, a' = max(a, 1e-4), s = a' / 448 (fp32 division)
 *   code = E4M3FN(x / s) (fp32 division, then nearest-even E4M3FN)
 * Every receive row of t gets the same codes; recv_scales[row, j] = s.
 *
 * FP8 scale modes ([GCU] feature notes: FP8 dispatch supports round_scale,
 * power-of-two scales, and use_ue8m0, the UE8M0 scale format; a single
 * per-tensor scale can be given with fp8_quant_scale, exclusive with
 * use_ue8m0).  With a' = max(amax, 1e-4) of the block:
 *   ORACLE_FP8_AMAX   s = a' / 448 (fp32 division); scale stored as fp32
 *   ORACLE_FP8_POW2   s = the smallest power of two with s >= a' / 448 (the
 *                     real quotient); scale stored as fp32
 *   ORACLE_FP8_UE8M0  s as POW2; stored as one byte, log2(s) + 127
 *   ORACLE_FP8_TENSOR s = the caller's scale for every block; nothing stored
 * and in every mode code = E4M3FN(x / s) with an fp32 division (exact for a
 * power of two), saturating at +/-448.  A block whose a' is infinite has
 * s = inf (UE8M0 byte 0xFF). */
enum { ORACLE_FP8_AMAX = 0, ORACLE_FP8_POW2 = 1, ORACLE_FP8_UE8M0 = 2, ORACLE_FP8_TENSOR = 3 };

/* a' / 448 = m * 2^e with m in [0.5, 1): the quotient is itself a power of two
 * exactly when m == 0.5 (then s = 2^(e-1)), else s = 2^e.  The double quotient
 * cannot round onto a power of two from elsewhere: a' has at most 24
 * significant bits, so a' / 448 is a power of two only for a' = 7 * 2^k, and
 * every other quotient lies far more than 2^-53 (relative) from one. */
float oracle_pow2_scale(float ap)
{
    if (isinf(ap)) return INFINITY;
    int e;
    double m = frexp((double)ap / 448.0, &e);
    return (float)ldexp(1.0, m == 0.5 ? e - 1 : e);
}

void oracle_quant_row_fp8_mode(const uint16_t *xrow, int64_t H, int mode, float tensor_scale,
                               uint8_t *codes, float *scales_f32, uint8_t *scales_u8)
{
    for (int64_t j = 0; j < H / 128; ++j) {
        float a = 0.0f;
        for (int m = 0; m < 128; ++m) {
            float v = fabsf(oracle_bf16_to_f32(xrow[j * 128 + m]));
            if (v > a) a = v;
        }
        float ap = a > 1e-4f ? a : 1e-4f;
        float s;
        if (mode == ORACLE_FP8_AMAX) s = ap / 448.0f;  /* the default per-group scale */
        else if (mode == ORACLE_FP8_TENSOR) s = tensor_scale;
        else s = oracle_pow2_scale(ap);
        for (int m = 0; m < 128; ++m)
            codes[j * 128 + m] = oracle_e4m3_encode(oracle_bf16_to_f32(xrow[j * 128 + m]) / s);
        if (mode == ORACLE_FP8_AMAX || mode == ORACLE_FP8_POW2) scales_f32[j] = s;
        if (mode == ORACLE_FP8_UE8M0) scales_u8[j] = isinf(s) ? 0xFF : (uint8_t)(ilogbf(s) + 127);
    }
}

void oracle_pack_fp8_mode(const uint16_t *x, int64_t T, int64_t H, int R,
                          const int32_t *send_head, const int32_t *rank_prefix_matrix, int mode,
                          float tensor_scale, uint8_t *recv_x8, float *recv_scales_f32,
                          uint8_t *recv_scales_u8)
{
    int64_t G = H / 128;
    uint8_t *codes = (uint8_t *)malloc((size_t)H);
    float *sf = (float *)malloc((size_t)(G ? G : 1) * sizeof(float));
    uint8_t *su = (uint8_t *)malloc((size_t)(G ? G : 1));
    for (int64_t t = 0; t < T; ++t) {
        oracle_quant_row_fp8_mode(x + t * H, H, mode, tensor_scale, codes, sf, su);
        for (int r = 0; r < R; ++r) {
            int32_t pos = send_head[t * R + r];
            if (pos < 0) continue;
            int64_t row = bucket_base(rank_prefix_matrix, r) + pos;
            memcpy(recv_x8 + row * H, codes, (size_t)H);
            if (mode == ORACLE_FP8_AMAX || mode == ORACLE_FP8_POW2)
                memcpy(recv_scales_f32 + row * G, sf, (size_t)G * sizeof(float));
            if (mode == ORACLE_FP8_UE8M0) memcpy(recv_scales_u8 + row * G, su, (size_t)G);
        }
    }
    free(codes);
    free(sf);
    free(su);
}

/* Pre-quantised input passed through ([GCU]: the dispatch of an (x_fp8,
 * scales) tuple): every W-byte row of src goes unchanged to the receive rows
 * of its token, as the bf16 pack moves x. */
void oracle_pack_rows_bytes(const uint8_t *src, int64_t T, int64_t W, int R,
                            const int32_t *send_head, const int32_t *rank_prefix_matrix,
                            uint8_t *dst)
{
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            int32_t pos = send_head[t * R + r];
            if (pos < 0) continue;
            int64_t row = bucket_base(rank_prefix_matrix, r) + pos;
            memcpy(dst + row * W, src + t * W, (size_t)W);
        }
}

/* The default FP8 dispatch (per-group fp32 scale s = a' / 448) as used by the
 * plain FP8 pack. */
void oracle_quant_row_fp8(const uint16_t *xrow, int64_t H, uint8_t *codes, float *scales)
{
    oracle_quant_row_fp8_mode(xrow, H, ORACLE_FP8_AMAX, 0.0f, codes, scales, NULL);
}

void oracle_pack_fp8(const uint16_t *x, int64_t T, int64_t H, int R,
                     const int32_t *send_head, const int32_t *rank_prefix_matrix,
                     uint8_t *recv_x8, float *recv_scales)
{
    oracle_pack_fp8_mode(x, T, H, R, send_head, rank_prefix_matrix, ORACLE_FP8_AMAX, 0.0f,
                         recv_x8, recv_scales, NULL);
}

/* ------------------------------------------------------------------------ */
/* Combine  ([GCU] combine_forward / dispatch_backward; [HR] Combining with  */
/* Handle Reuse)                                                             */
/* ------------------------------------------------------------------------ */

/* For each token t the rows row(t,r) of its distinct buckets are visited in
 * first-occurrence order over k = 0..K-1.  Row r is scaled by
 *   w(t,r) = 1                                  if gate_weights is NULL
 *          = sum over k with b(topk_idx[t,k]) == r of gate_weights[t,k]
 *            (fp32 adds from +0.0f, ascending k)  otherwise
 * and accumulated from +0.0f as acc = fmaf(w, y[row], acc); out = bf16(acc).
 * If recv_topk_weights is given, combined_topk_weights[t,k] is the fp32 sum
 * (from +0.0f, same visit order) of recv_topk_weights[row(t,r), k]. */
void oracle_combine(const uint16_t *y, int64_t T, int64_t H,
                    const int64_t *topk_idx, int K, int E, int R,
                    const int32_t *send_head, const int32_t *rank_prefix_matrix,
                    const float *gate_weights, const float *recv_topk_weights,
                    uint16_t *out, float *combined_topk_weights)
{
    int P = E / R;
    float *acc = (float *)malloc((size_t)(H ? H : 1) * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) acc[h] = 0.0f;
        if (combined_topk_weights)
            for (int k = 0; k < K; ++k) combined_topk_weights[t * K + k] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) continue;
            int r = (int)(e / P);
            int seen = 0;
            for (int k2 = 0; k2 < k; ++k2) {
                int64_t e2 = topk_idx[t * K + k2];
                if (e2 >= 0 && (int)(e2 / P) == r) seen = 1;
            }
            if (seen) continue;
            float w = 1.0f;
            if (gate_weights) {
                w = 0.0f;
                for (int k2 = 0; k2 < K; ++k2) {
                    int64_t e2 = topk_idx[t * K + k2];
                    if (e2 >= 0 && (int)(e2 / P) == r) w = w + gate_weights[t * K + k2];
                }
            }
            int64_t row = bucket_base(rank_prefix_matrix, r) + send_head[t * R + r];
            for (int64_t h = 0; h < H; ++h)
                acc[h] = fmaf(w, oracle_bf16_to_f32(y[row * H + h]), acc[h]);
            if (combined_topk_weights && recv_topk_weights)
                for (int k2 = 0; k2 < K; ++k2)
                    combined_topk_weights[t * K + k2] =
                        combined_topk_weights[t * K + k2] + recv_topk_weights[row * K + k2];
        }
        for (int64_t h = 0; h < H; ++h) out[t * H + h] = oracle_bf16_round(acc[h]);
    }
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Low-latency layout  ([GCU] low-latency example; [HK] Two-Phase Kernel)    */
/* ------------------------------------------------------------------------ */

/* Per-expert fixed-capacity slots.  For expert e let L_e be the ascending list
 * of tokens that chose e.  recv_count[e] = |L_e|; src_idx[e][s] = L_e[s]
 * (-1 past the count); recv_x[e][s] = x[L_e[s]]; slot_of[t][k] = position of t
 * in L_{topk_idx[t,k]} (-1 for an empty slot).  Requires every |L_e| <= cap;
 * returns -1 otherwise.  recv_x rows past the count are left untouched. */
int oracle_ll_dispatch(const uint16_t *x, int64_t T, int64_t H,
                       const int64_t *topk_idx, int K, int E, int64_t cap,
                       uint16_t *recv_x, int32_t *recv_count, int32_t *src_idx,
                       int32_t *slot_of)
{
    for (int e = 0; e < E; ++e) recv_count[e] = 0;
    for (int64_t i = 0; i < (int64_t)E * cap; ++i) src_idx[i] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) { slot_of[t * K + k] = -1; continue; }
            int64_t s = recv_count[e];
            if (s >= cap) return -1;
            slot_of[t * K + k] = (int32_t)s;
            src_idx[e * cap + s] = (int32_t)t;
            if (recv_x)
                for (int64_t h = 0; h < H; ++h) recv_x[(e * cap + s) * H + h] = x[t * H + h];
            recv_count[e] = (int32_t)(s + 1);
        }
    }
    return 0;
}

/* out[t] = bf16( fmaf chain over k = 0..K-1 of topk_weights[t,k] * y[e_k][slot_of[t,k]] )
 * from +0.0f, skipping empty slots. */
void oracle_ll_combine(const uint16_t *y, int64_t cap, int64_t H,
                       const int64_t *topk_idx, const float *topk_weights, int64_t T, int K,
                       const int32_t *slot_of, uint16_t *out)
{
    float *acc = (float *)malloc((size_t)(H ? H : 1) * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) acc[h] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) continue;
            int64_t row = e * cap + slot_of[t * K + k];
            float w = topk_weights[t * K + k];
            for (int64_t h = 0; h < H; ++h)
                acc[h] = fmaf(w, oracle_bf16_to_f32(y[row * H + h]), acc[h]);
        }
        for (int64_t h = 0; h < H; ++h) out[t * H + h] = oracle_bf16_round(acc[h]);
    }
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs (for the codec sweeps in the tests)             */
/* ------------------------------------------------------------------------ */

void oracle_bf16_round_array(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(in[i]);
}

void oracle_e4m3_encode_array(const float *in, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(in[i]);
}
