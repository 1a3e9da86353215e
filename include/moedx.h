/*
 * moedx — MoE dispatch layout, token pack, handle reuse and combine on one
 * MI355X (gfx950).  C ABI of libmoedx.so.
 *
 * One GPU's share of an expert-parallel all-to-all: the "ranks" of the pages
 * are logical ranks, i.e. buckets of experts that all live in this GPU's HBM
 * (expert e belongs to bucket e / (num_experts / num_ranks)).  Nothing here
 * moves data between GPUs.
 *
 * Source pages (the calls below follow their problem statement):
 *   [EO]  "How DeepEP Achieves Communication-Computation Overlapping with
 *          EventOverlap" — events, previous_event, async_finish, the comm stream
 *   [HK]  "How DeepEP Enables Hook-Based Overlapping Without SM Occupation"
 *          — low-latency dispatch/combine and their stream choice
 *   [GCU] EnflameTechnology/DeepEP README — get_dispatch_layout, dispatch,
 *          combine and low-latency usage examples, FP8 dispatch notes
 *   [HR]  "How DeepEP Optimizes Handle Reuse for Repeated Dispatches"
 *          — handle contents and the cached-layout fast path
 *
 * Conventions for every call:
 *   - Returns MOEDX_OK (0) or a negative MOEDX_E* code; moedx_last_error()
 *     gives a thread-local message.  No C++ exception crosses the ABI, and bad
 *     arguments never abort the process.
 *   - Arguments are validated on the host before anything is enqueued; a call
 *     that returns an error has enqueued nothing.
 *   - Pointers named "dev" or documented as device memory are caller-owned
 *     device allocations; the library never frees them.  Row-major layouts.
 *   - bf16 data is passed as uint16_t bit patterns; FP8 codes as uint8_t
 *     (OCP E4M3FN).
 *   - Execution: see moedx_exec.  Kernels run on the caller's stream unless
 *     MOEDX_ON_CTX_STREAM is set.
 *   - A ctx is not thread-safe (one host thread at a time).  Calls are stream
 *     ordered; of the calls that may overlap on one ctx from different
 *     streams, moedx_create says which share the ctx's scratch.
 */
#ifndef MOEDX_H
#define MOEDX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define MOEDX_API __attribute__((visibility("default")))
#else
#define MOEDX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
enum {
    MOEDX_OK = 0,
    MOEDX_EINVAL = -1,     /* bad argument (shape, null pointer, range) */
    MOEDX_ENOMEM = -2,     /* host or device allocation failed (setup calls only) */
    MOEDX_EHIP = -3,       /* a HIP runtime call failed */
    MOEDX_ECAPACITY = -4,  /* a buffer or workspace is smaller than required */
    MOEDX_ESTATE = -5      /* handle used against a different shape or mode */
};

/* ---- flags --------------------------------------------------------------- */
enum {
    /* Run on the ctx's own stream after it waits for the caller's stream
     * (allocate_on_comm_stream / the comm stream, [EO] C++ Backend
     * Implementation; [GCU] dispatch_forward). */
    MOEDX_ON_CTX_STREAM = 1u,
    /* With done == NULL: return without blocking and without an event; later
     * work on the same stream is ordered after the op by the stream itself. */
    MOEDX_ASYNC = 2u
};

enum { /* moedx_dispatch quant */
    MOEDX_QUANT_NONE = 0,           /* recv_x is bf16 [rows, H] */
    MOEDX_QUANT_FP8_E4M3_1X128 = 1  /* recv_x is E4M3FN [rows, H], recv_scales fp32 [rows, H/128] */
};

typedef struct moedx_ctx moedx_ctx;
typedef struct moedx_event moedx_event;
typedef struct moedx_handle moedx_handle;

/* How a call is ordered and completed ([EO] Propagation Through EP Operations).
 *   stream : the caller's stream (0 = the null stream).
 *   prev   : if non-NULL, the op first waits for this event (previous_event).
 *   done   : if non-NULL, *done receives a new event recorded after the op and
 *            the call returns without blocking (async_finish=True); the caller
 *            destroys it.  If NULL, the call blocks until the op has finished
 *            (async_finish=False), unless MOEDX_ASYNC is set.
 *   flags  : MOEDX_ON_CTX_STREAM | MOEDX_ASYNC.
 * Passing a NULL moedx_exec* means {0, NULL, NULL, 0, NULL, NULL}. */
typedef struct moedx_exec {
    hipStream_t stream;
    const moedx_event *prev;
    moedx_event **done;
    uint32_t flags;
    /* Optional events from moedx_event_create: stamped when the op's kernel
     * starts and when it ends (kernel-accurate timing; every op launches one
     * kernel).  An op that launches no kernel (no token) records both on the
     * stream instead. */
    moedx_event *kernel_start;
    moedx_event *kernel_stop;
} moedx_exec;

/* Kernel launch counters of a ctx (the cached path launches no layout or
 * scan kernel, [HR] Performance Contract and Constraints). */
typedef struct moedx_stats {
    int64_t layout_launches;
    int64_t pack_launches;
    int64_t pack_fp8_launches;
    int64_t combine_launches;
    int64_t ll_dispatch_launches;
    int64_t ll_combine_launches;
    int64_t host_syncs;
    /* scans of a handle from get_dispatch_layout's outputs (moedx_dispatch_prepare
     * given them): no layout kernel runs for such a handle */
    int64_t scan_launches;
} moedx_stats;

/* Which device array of a handle moedx_handle_tensor returns
 * ([HR] What the Handle Contains, plus the layout outputs of [GCU]). */
enum {
    MOEDX_T_RANK_PREFIX_MATRIX = 0,         /* int32 [R], inclusive prefix of per-bucket counts */
    MOEDX_T_CHANNEL_PREFIX_MATRIX = 1,      /* int32 [R, C], inclusive prefix over channels */
    MOEDX_T_RECV_CHANNEL_PREFIX_MATRIX = 2, /* int32 [R, C], exclusive prefix over channels */
    MOEDX_T_RECV_SRC_IDX = 3,               /* int32 [N] (N rows valid), source token of each row;
                                               written by the first moedx_dispatch on the handle */
    MOEDX_T_IS_TOKEN_IN_RANK = 4,           /* uint8 [T, R], 0/1 */
    MOEDX_T_SEND_HEAD = 5,                  /* int32 [T, R], position in bucket or -1;
                                               written by the first moedx_dispatch on the handle */
    MOEDX_T_NUM_TOKENS_PER_RANK = 6,        /* int32 [R] */
    MOEDX_T_NUM_TOKENS_PER_EXPERT = 7,      /* int32 [E] */
    MOEDX_T_NUM_RECV = 8,                   /* int32 [1], N on the device */
    MOEDX_T_LL_SRC_IDX = 9,                 /* int32 [E, cap], low-latency handle */
    MOEDX_T_LL_SLOT_OF = 10                 /* int32 [T, K], low-latency handle */
};

/* ---- setup --------------------------------------------------------------- */

/* Message of the last error on this thread ("" if none). */
MOEDX_API const char *moedx_last_error(void);

/* Create a context on `device` (the Buffer of [GCU] / [HR]).
 * num_experts % num_ranks must be 0 ([GCU] low-latency example asserts it);
 * num_ranks in [1, 64]; num_experts in [1, 1024]; num_channels >= 1 is the
 * number of contiguous token ranges the layout reports per bucket (the
 * channel unit of channel_prefix_matrix); max_tokens bounds T for every call
 * and sizes the ctx's scratch.  Allocates the ctx stream (default priority),
 * a small device scratch and a pinned host buffer; flags must be 0.
 * moedx_get_dispatch_layout and moedx_dispatch_prepare of one ctx share the
 * scratch's completion counter (and get_dispatch_layout its counters and
 * partials): they must not run concurrently with each other (issue them on
 * one stream, or order them with events); the first moedx_dispatch of a
 * handle that borrowed a layout's partials (moedx_dispatch_prepare) counts as
 * part of that layout here, and when it runs on another stream than the
 * layout, the ctx's next get_dispatch_layout waits for it by itself.  Every
 * other call (dispatch, combine, handle_finish, the low-latency calls) leaves
 * that scratch alone and may overlap with anything whose buffers it does not
 * share. */
MOEDX_API int moedx_create(moedx_ctx **out, int device, int num_experts, int num_ranks,
                           int num_channels, int max_tokens, uint32_t flags);
MOEDX_API int moedx_destroy(moedx_ctx *ctx);
MOEDX_API int moedx_ctx_stats(const moedx_ctx *ctx, moedx_stats *out);
/* The ctx's own stream (for MOEDX_ON_CTX_STREAM users). */
MOEDX_API int moedx_ctx_stream(const moedx_ctx *ctx, hipStream_t *out);
/* Use the caller's `stream` (not the null stream; default priority) as the
 * ctx's own stream from now on: the comm stream of [EO] may then be one the
 * caller's runtime owns and keeps alive (a memory pool that records its
 * streams on blocks, for instance, needs them valid when a block is freed,
 * which may be after moedx_destroy).  Waits for the previous ctx stream to
 * drain and destroys it if moedx_create made it; the caller keeps `stream`
 * alive for the ctx's lifetime, and moedx_destroy does not destroy it. */
MOEDX_API int moedx_ctx_set_stream(moedx_ctx *ctx, hipStream_t stream);

/* ---- events ([EO] CUDA Event Capture in Buffer; Explicit Stream Waiting) -- */

/* Record a new event on `stream` (Buffer.capture()).  Timing-capable. */
MOEDX_API int moedx_event_record(moedx_event **out, hipStream_t stream);
/* A new, not yet recorded, timing-capable event (for moedx_exec.kernel_start /
 * kernel_stop). */
MOEDX_API int moedx_event_create(moedx_event **out);
/* Make `stream` wait for the event without blocking the host
 * (current_stream_wait()). */
MOEDX_API int moedx_event_wait(const moedx_event *ev, hipStream_t stream);
/* Block the host until the event has completed. */
MOEDX_API int moedx_event_synchronize(const moedx_event *ev);
/* Milliseconds between two recorded, completed events. */
MOEDX_API int moedx_event_elapsed_ms(const moedx_event *start, const moedx_event *end, float *ms);
MOEDX_API int moedx_event_destroy(moedx_event *ev);

/* ---- dispatch layout ([GCU] normal-kernel example, get_dispatch_layout) --- */

/* From topk_idx (device int64 [T, K]; -1 = empty slot; every other id in
 * [0, E) and distinct within a token) compute, into caller device buffers:
 *   num_tokens_per_rank   int32 [R]   tokens routed to each bucket (once per bucket)
 *   num_tokens_per_expert int32 [E]   (token, slot) pairs per expert
 *   is_token_in_rank      uint8 [T,R] 1 iff a valid slot's expert is in bucket r
 * num_tokens_per_rdma_rank has no counterpart (one GPU, no RDMA domain).
 * Ids outside [-1, E) are a caller error; the kernels ignore such slots.
 * T in [0, max_tokens], K in [1, 16]. */
MOEDX_API int moedx_get_dispatch_layout(moedx_ctx *ctx, const int64_t *topk_idx, int T, int K,
                                        int32_t *num_tokens_per_rank,
                                        int32_t *num_tokens_per_expert,
                                        uint8_t *is_token_in_rank, const moedx_exec *exec);

/* get_dispatch_layout for callers that cannot allocate (code under HIP graph
 * capture, serving loops or harnesses that forbid allocation): the same
 * outputs as moedx_get_dispatch_layout, for E experts in R buckets, without a
 * ctx.  It allocates nothing: its E + R counters (8 bytes each) live in a
 * static device array of 16 KiB inside the library (one per GPU, held until
 * the process ends), which holds them for every E and R accepted here (a
 * request past it would return MOEDX_ECAPACITY).  Runs on the current device,
 * on `stream` (a stream of that device), and returns without waiting.  Calls
 * on one GPU share that array: two calls that overlap (on different streams,
 * or from different threads) race and give wrong results; order them.
 * R in [1, 64], E in [1, 1024], E % R == 0, K in [1, 16], T in [0, 2^24];
 * other errors as moedx_get_dispatch_layout. */
MOEDX_API int moedx_get_dispatch_layout_static(const int64_t *topk_idx, int T, int K, int E, int R,
                                               int32_t *num_tokens_per_rank,
                                               int32_t *num_tokens_per_expert,
                                               uint8_t *is_token_in_rank, hipStream_t stream);

/* ---- handle: layout + receive positions ([HR] Handle Creation) ----------- */

/* Device bytes a handle for T tokens, K slots and the given capacity needs.
 * capacity_rows = 0 selects exact mode, > 0 capacity mode (moedx_dispatch_prepare). */
MOEDX_API int moedx_handle_workspace_bytes(const moedx_ctx *ctx, int T, int K,
                                           int64_t capacity_rows, size_t *bytes);

/* Run the layout and the scan for topk_idx (device int64 [T, K]) into a handle
 * whose device arrays live in `workspace` (caller device memory, at least
 * moedx_handle_workspace_bytes bytes, 256-byte aligned, kept alive by the
 * caller until moedx_handle_destroy).  The handle holds the arrays listed for
 * moedx_handle_tensor plus the bucket of every slot.
 *
 * Reuse of get_dispatch_layout's outputs (the normal-kernel example of [GCU]
 * passes num_tokens_per_rank, is_token_in_rank and num_tokens_per_expert from
 * get_dispatch_layout into dispatch): when num_tokens_per_expert (device int32
 * [E]) and is_token_in_rank (device uint8 [T, R], nonzero = member; may be
 * NULL only when T == 0) are given, no layout runs: one scan kernel takes the
 * bucket membership from is_token_in_rank, the slot buckets from topk_idx,
 * and copies the expert totals (moedx_stats.scan_launches counts it instead
 * of layout_launches).  They must be the layout of this topk_idx (the scan
 * trusts them).  num_tokens_per_rank (device int32 [R]) may be passed with
 * them, as the pages' call does; the bucket totals are recomputed by the scan,
 * so it is not read.  Alignment: num_tokens_per_expert 4 bytes,
 * is_token_in_rank 4 bytes when R % 4 == 0.  All three NULL: the layout runs.
 * When they are exactly the outputs (same pointers, T and K) of this ctx's
 * last moedx_get_dispatch_layout, in capacity mode where a first dispatch
 * finishes the handle in its own launch (below), not even the scan runs: the
 * handle borrows the partial counts, token masks and slot buckets that
 * get_dispatch_layout left in the ctx's scratch, and its first moedx_dispatch
 * or moedx_dispatch_fp8 builds the handle from them.
 * Any other first use, a
 * later prepare that borrows the same layout, or the ctx's next
 * moedx_get_dispatch_layout first copies them into the handle (one small
 * kernel, counted as a scan).  See moedx_create for ordering the next layout
 * after the first pack.  Destroying the ctx before the handle's first use
 * leaves the handle unusable (MOEDX_ESTATE).
 *
 * Receive rows are bucket-major and, inside a bucket, in ascending token order
 * (channel order, then token order inside a channel); N = total rows.
 *   capacity_rows == 0 (exact mode): the host waits for N and the per-expert
 *     counts ([GCU]: the CPU waits for the received-count signal) and
 *     moedx_handle_num_recv / moedx_handle_recv_tokens_per_expert work.
 *   capacity_rows  > 0 (capacity mode, num_worst_tokens of [GCU]): no host
 *     wait; capacity_rows must be >= T * min(K, R) so that every row fits;
 *     N stays on the device (MOEDX_T_NUM_RECV).  For T <= 4096 and R a
 *     multiple of 4 up to 16 only the layout's per-token outputs and partial
 *     counts run here; the prefixes, totals and N (rank and channel prefix
 *     matrices, num_tokens_per_rank/expert, MOEDX_T_NUM_RECV) are written on
 *     the stream of the handle's first moedx_dispatch or moedx_dispatch_fp8
 *     (by its pack kernel, in the same launch), moedx_combine (one small
 *     kernel before it) or moedx_handle_finish:
 *     read them after that call.  In exact mode the call blocks on the host
 *     even when exec->done is given.
 * *out receives a new handle (moedx_handle_destroy frees it). */
MOEDX_API int moedx_dispatch_prepare(moedx_ctx *ctx, const int64_t *topk_idx, int T, int K,
                                     const int32_t *num_tokens_per_rank,
                                     const uint8_t *is_token_in_rank,
                                     const int32_t *num_tokens_per_expert, void *workspace,
                                     size_t workspace_bytes, int64_t capacity_rows,
                                     moedx_handle **out, const moedx_exec *exec);

/* N on the host; exact-mode handles only (MOEDX_ESTATE otherwise). */
MOEDX_API int moedx_handle_num_recv(const moedx_handle *h, int64_t *n);
/* Per-expert receive counts (num_recv_tokens_per_expert_list) on the host,
 * host_counts int32 [E]; exact-mode handles only. */
MOEDX_API int moedx_handle_recv_tokens_per_expert(const moedx_handle *h, int32_t *host_counts);
/* Device pointer and shape of one handle array (MOEDX_T_*).  shape[1] is 1 for
 * vectors.  For MOEDX_T_RECV_SRC_IDX shape[0] is N in exact mode and the
 * capacity in capacity mode (rows past N are unspecified). */
MOEDX_API int moedx_handle_tensor(const moedx_handle *h, int which, const void **dev,
                                  int64_t shape[2]);
/* Write a capacity-mode handle's prefixes, totals and N (the prefix matrices
 * and counts of [HR] What the Handle Contains) now, on exec's stream, instead
 * of on the handle's first dispatch or combine (moedx_dispatch_prepare).  No
 * kernel runs when they are already written or enqueued (exact mode, or after
 * a first use).  Normal handles only. */
MOEDX_API int moedx_handle_finish(moedx_ctx *ctx, const moedx_handle *h,
                                  const moedx_exec *exec);
MOEDX_API int moedx_handle_destroy(moedx_handle *h);

/* ---- dispatch (token pack) ([GCU] dispatch_forward; [HR] Fast Path) ------- */

/* Copy every token row x[t] (device [T, H], bf16) to its receive rows.
 *   quant = MOEDX_QUANT_NONE: recv_x bf16 [rows, H], bit-exact copies.
 *   quant = MOEDX_QUANT_FP8_E4M3_1X128: per 1x128 block of each token,
 *     s = max(amax, 1e-4) / 448 and codes E4M3FN(x / s) (IEEE fp32 division,
 *     round to nearest even, saturating at +/-448); recv_x uint8 [rows, H],
 *     recv_scales fp32 [rows, H/128] (FP8 dispatch with per-group scales,
 *     [GCU] feature notes).  H % 128 == 0.
 * rows = N in exact mode, capacity_rows in capacity mode (rows >= N untouched).
 * First dispatch: topk_idx [T,K] and topk_weights [T,K] (fp32) may be given
 *   together with recv_topk_idx int64 [rows, K] (local expert id e - r*P, or -1
 *   when slot k's expert is not in the row's bucket) and recv_topk_weights fp32
 *   [rows, K] (the weight, or +0.0f); topk_idx must equal the one the handle
 *   was prepared from.
 * Cached dispatch (handle reuse): topk_idx, topk_weights, recv_topk_idx and
 *   recv_topk_weights are all NULL; only rows move, no layout or scan kernel
 *   runs.  Valid only while the routing is unchanged ([HR] Performance
 *   Contract and Constraints).
 * H % 8 == 0 (16-byte rows); T must equal the handle's T. */
MOEDX_API int moedx_dispatch(moedx_ctx *ctx, const moedx_handle *h, const void *x, int T, int H,
                             int quant, const int64_t *topk_idx, const float *topk_weights,
                             void *recv_x, float *recv_scales, int64_t *recv_topk_idx,
                             float *recv_topk_weights, const moedx_exec *exec);

/* FP8 dispatch options ([GCU] feature notes: FP8 dispatch supports
 * round_scale, power-of-two scales, and use_ue8m0, the UE8M0 scale format; a
 * single per-tensor scale may be given with fp8_quant_scale, exclusive with
 * use_ue8m0; FP8 dispatch of an already-quantised (codes, scales) input).
 * For each 1x128 block with a' = max(amax, 1e-4):
 *   MOEDX_FP8_SCALE_AMAX   s = a' / 448 (IEEE fp32); scales fp32
 *   MOEDX_FP8_SCALE_POW2   s = the smallest power of two >= a' / 448; scales fp32
 *   MOEDX_FP8_SCALE_UE8M0  s as POW2; scales uint8, log2(s) + 127 (0xFF: inf)
 *   MOEDX_FP8_SCALE_TENSOR s = tensor_scale for every block; no scales written
 * codes = E4M3FN(x / s) (IEEE fp32 quotient, nearest even, saturating at
 * +/-448, NaN -> 0x7F).  A block holding inf has s = inf. */
enum {
    MOEDX_FP8_SCALE_AMAX = 0,
    MOEDX_FP8_SCALE_POW2 = 1,
    MOEDX_FP8_SCALE_UE8M0 = 2,
    MOEDX_FP8_SCALE_TENSOR = 3
};

typedef struct moedx_fp8 {
    int scale_mode;        /* MOEDX_FP8_SCALE_* */
    int prequantized;      /* 1: x already holds E4M3FN codes uint8 [T, H] */
    float tensor_scale;    /* MOEDX_FP8_SCALE_TENSOR: positive, in [2^-126, 2^126) */
    const void *x_scales;  /* prequantized: the scales of x, in the scale_mode's format
                              ([T, H/128] fp32 or uint8); NULL for TENSOR */
} moedx_fp8;

/* FP8 dispatch with options: recv_x uint8 [rows, H]; recv_scales [rows, H/128]
 * in the scale_mode's format (NULL for MOEDX_FP8_SCALE_TENSOR).  Quantising:
 * x is bf16 [T, H] and codes / scales follow the definition above.
 * Pre-quantised (prequantized = 1): the code rows and scale rows of x are
 * copied unchanged to every receive row of their token.  Handle rows, capacity
 * mode and cached use behave as in moedx_dispatch; recv_topk_* are not
 * produced.  H % 128 == 0.  Errors: MOEDX_EINVAL for an unknown mode, a
 * tensor_scale out of range, x_scales missing or given where unused, NULL or
 * misaligned buffers (x, recv_x 16-byte); MOEDX_ESTATE for a handle of another
 * ctx or another T. */
MOEDX_API int moedx_dispatch_fp8(moedx_ctx *ctx, const moedx_handle *h, const void *x, int T, int H,
                                 const moedx_fp8 *fp8, uint8_t *recv_x, void *recv_scales,
                                 const moedx_exec *exec);

/* ---- combine ([GCU] combine_forward, dispatch_backward; [HR] Combining) --- */

/* out[t] (bf16 [T, H]) = bf16_rne( sum over t's distinct buckets r, in
 * first-occurrence order over k, of w(t,r) * y[row(t,r)] ), accumulated in fp32
 * with fused multiply-adds from +0.0f, where y is bf16 [rows, H] laid out like
 * recv_x and
 *   w(t,r) = 1                                        if gate_weights is NULL,
 *   w(t,r) = sum of gate_weights[t,k] over k with expert in r (fp32, ascending k).
 * If recv_topk_weights (fp32 [rows, K]) is given, combined_topk_weights
 * (fp32 [T, K]) = the sum of recv_topk_weights[row(t,r), k] over the same
 * visited rows, in the same order (the weight payload of dispatch_backward).
 * H % 8 == 0. */
MOEDX_API int moedx_combine(moedx_ctx *ctx, const moedx_handle *h, const uint16_t *y, int H,
                            const float *gate_weights, const float *recv_topk_weights,
                            uint16_t *out, float *combined_topk_weights, const moedx_exec *exec);

/* ---- low-latency path ([GCU] low-latency example; [HK]) ------------------- */

/* Device bytes of a low-latency handle (src_idx [E, cap] + slot_of [T, K]). */
MOEDX_API int moedx_ll_workspace_bytes(const moedx_ctx *ctx, int T, int K,
                                       int num_max_dispatch_tokens_per_rank, size_t *bytes);

/* Per-expert fixed-capacity dispatch.  cap = num_max_dispatch_tokens_per_rank,
 * T <= cap.  For expert e, L_e = ascending list of tokens that chose e:
 *   recv_count[e] = |L_e| (int32 [E]), recv_x[e][s] = x[L_e[s]]
 *   (bf16 [E, cap, H]; slots past the count untouched), and in the handle
 *   src_idx[e][s] = L_e[s] and slot_of[t][k] = position of t in L_{topk_idx[t,k]}
 *   (-1 for an empty slot).  Runs as a single kernel launch.
 * recv_x == NULL defers the receive (return_recv_hook=True of the low-latency
 *   example: the rows arrive only when the hook runs): counts and the handle
 *   are written, rows are not, and x is not read; moedx_ll_dispatch_recv then
 *   copies the rows.
 * Errors: MOEDX_ECAPACITY when T > cap or the workspace is too small;
 * MOEDX_EINVAL when E * cap exceeds 2^31 - 1 rows, H % 8 != 0, a pointer is
 * NULL or misaligned (x, recv_x 16-byte; workspace 256-byte). */
MOEDX_API int moedx_ll_dispatch(moedx_ctx *ctx, const uint16_t *x, const int64_t *topk_idx,
                                int T, int K, int H, int num_max_dispatch_tokens_per_rank,
                                uint16_t *recv_x, int32_t *recv_count, void *workspace,
                                size_t workspace_bytes, moedx_handle **out,
                                const moedx_exec *exec);

/* The deferred receive of a moedx_ll_dispatch called with recv_x == NULL (the
 * hook of [GCU]'s low-latency example, "How DeepEP Enables Hook-Based
 * Overlapping Without SM Occupation"): recv_x[e][slot_of[t][k]] = x[t] for
 * every filled slot.  x, topk_idx and H as given to that dispatch; one kernel
 * launch.  Errors: MOEDX_EINVAL for a handle that is not low-latency, H % 8
 * != 0, NULL or misaligned pointers (16-byte). */
MOEDX_API int moedx_ll_dispatch_recv(moedx_ctx *ctx, const moedx_handle *h, const uint16_t *x,
                                     const int64_t *topk_idx, int H, uint16_t *recv_x,
                                     const moedx_exec *exec);

/* out[t] (bf16 [T, H]) = bf16_rne( fmaf chain over k = 0..K-1, from +0.0f, of
 * topk_weights[t,k] * y[e_k][slot_of[t,k]] ), y bf16 [E, cap, H]; empty slots
 * skipped. topk_idx / topk_weights [T, K] as given to moedx_ll_dispatch. */
MOEDX_API int moedx_ll_combine(moedx_ctx *ctx, const uint16_t *y, const int64_t *topk_idx,
                               const float *topk_weights, const moedx_handle *h, int H,
                               uint16_t *out, const moedx_exec *exec);

#ifdef __cplusplus
}
#endif

#endif /* MOEDX_H */
