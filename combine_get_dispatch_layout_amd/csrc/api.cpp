// C ABI of libmoedx.so: validation, contexts, handles, events and launches.
//
// The calls follow the problem statement of the pages: get_dispatch_layout,
// dispatch with or without a cached handle, combine, and the low-latency pair
// (EnflameTechnology/DeepEP README usage examples), ordered by events in the
// way "How DeepEP Achieves Communication-Computation Overlapping with
// EventOverlap" describes (previous_event, async_finish, the comm stream).
//
// Every argument is checked on the host before anything is enqueued, and no
// C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "launch.h"
#include "moedx.h"

using namespace moedx;

struct moedx_event {
    hipEvent_t ev;
};

struct moedx_ctx {
    int device;
    int E, R, P, C, max_tokens;
    BucketDiv bucket;        // e / P as a multiply and shift on the device
    hipStream_t stream;      // the ctx's own stream (default priority)
    bool owns_stream;        // made by moedx_create (else the caller's, moedx_ctx_set_stream)
    hipEvent_t order_event;  // orders the ctx stream after the caller's
    void* scratch;           // the handle layouts' ticket + get_dispatch_layout's counters
    size_t scratch_bytes;    //   and the partials it leaves for a handle to borrow
    unsigned int* ticket;    // zero between layout launches
    unsigned long long* acc; // [E + R] counters of get_dispatch_layout, zero between launches
    // What the last get_dispatch_layout left: the partials a handle scanned
    // from its outputs would hold ([max_tokens] masks, [max_tokens, 16] slot
    // buckets, [ceil(max_tokens/64), R] group counts, [C + 1, R] channel
    // partials, [E] expert totals), and which call that was.
    uint64_t* lay_mask;
    int8_t* lay_slot_bucket;
    int32_t* lay_group_cnt;
    int32_t* lay_chan_part;
    int32_t* lay_experts;
    struct {
        bool valid;
        const int64_t* topk_idx;
        const uint8_t* is_token_in_rank;
        const int32_t* num_tokens_per_expert;
        int T, K;
        hipStream_t stream;  // where that layout ran
    } last;
    moedx_handle* pending;   // the handle borrowing those partials, before its first pack
    hipEvent_t borrow_done;  // recorded after a first pack that read them on another stream
    bool borrow_armed;       // borrow_done recorded since the last layout
    int32_t* pinned;         // host readback: [0] = N, [1..E] = per-expert counts
    moedx_stats stats;
};

enum HandleKind { kNormal = 1, kLowLatency = 2 };

struct moedx_handle {
    HandleKind kind;
    int T, K, E, R, P, C;
    int64_t capacity;  // 0 = exact mode
    int64_t n_host;    // exact mode only
    std::vector<int32_t> per_expert_host;
    mutable bool rows_written;  // send_head / recv_src_idx filled by a dispatch
    bool experts_given;         // prepared from get_dispatch_layout's outputs: the expert
                                // totals were copied, the tiles' expert partials never exist
    // Borrowing the partials that ctx's last get_dispatch_layout left in its
    // scratch (prepared from exactly those outputs): set until the first pack
    // reads them, or until they are copied into the handle's own arrays.
    mutable moedx_ctx* borrow_ctx;
    mutable hipEvent_t adopted;  // recorded after a copy enqueued on another op's stream
    bool orphaned;               // its borrow_ctx was destroyed first: nothing to finish from
    // Capacity mode: prepared with the layout's partials only; the first
    // dispatch or combine finishes the prefixes (or launches the finishing
    // step first).
    mutable bool prefixes_pending;
    // device arrays inside the caller's workspace
    uint8_t* is_token_in_rank;
    uint64_t* token_mask;
    int8_t* slot_bucket;
    int32_t* num_tokens_per_rank;
    int32_t* num_tokens_per_expert;
    int32_t* rank_prefix_matrix;
    int32_t* channel_prefix_matrix;
    int32_t* recv_channel_prefix_matrix;
    int32_t* group_prefix;
    int32_t* send_head;
    int32_t* recv_src_idx;
    int32_t* num_recv;
    int32_t* group_cnt;
    int32_t* chan_part;
    int32_t* tile_expert;
    // low-latency
    int cap;
    int32_t* ll_src_idx;
    int32_t* ll_slot_of;
};

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MOEDX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_OR_FAIL(call)                                  \
    do {                                                   \
        hipError_t e_ = (call);                            \
        if (e_ != hipSuccess) return hip_fail(e_, #call);  \
    } while (0)

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Carves consecutive 256-byte-aligned regions out of one workspace.
struct Carver {
    char* base;
    size_t off = 0;
    template <typename T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += align256(count * sizeof(T));
        return p;
    }
};

// Lays out a normal handle's device arrays; with base == nullptr it only sizes.
size_t carve_normal(moedx_handle* h, char* base, int T, int K, int E, int R, int C,
                    int64_t rows) {
    Carver cv{base};
    const int nt = num_tiles(T);
    moedx_handle tmp;
    moedx_handle* d = h ? h : &tmp;
    const int ng = num_groups(T);
    d->is_token_in_rank = cv.take<uint8_t>((size_t)T * R);
    d->token_mask = cv.take<uint64_t>((size_t)T);
    d->slot_bucket = cv.take<int8_t>((size_t)T * K);
    d->num_tokens_per_rank = cv.take<int32_t>(R);
    // N, then the per-expert counts: exact mode reads both back with one copy
    d->num_recv = cv.take<int32_t>(1 + (size_t)E);
    d->num_tokens_per_expert = d->num_recv + 1;
    d->rank_prefix_matrix = cv.take<int32_t>(R);
    d->channel_prefix_matrix = cv.take<int32_t>((size_t)R * C);
    d->recv_channel_prefix_matrix = cv.take<int32_t>((size_t)R * C);
    d->group_prefix = cv.take<int32_t>((size_t)std::max(ng, 1) * R);
    d->send_head = cv.take<int32_t>((size_t)T * R);
    d->recv_src_idx = cv.take<int32_t>((size_t)std::max<int64_t>(rows, 1));
    d->group_cnt = cv.take<int32_t>((size_t)std::max(ng, 1) * R);
    d->chan_part = cv.take<int32_t>((size_t)(C + 1) * R);
    d->tile_expert = cv.take<int32_t>((size_t)std::max(nt, 1) * E);
    return cv.off;
}

size_t carve_ll(moedx_handle* h, char* base, int T, int K, int E, int cap) {
    Carver cv{base};
    moedx_handle tmp;
    moedx_handle* d = h ? h : &tmp;
    d->ll_src_idx = cv.take<int32_t>((size_t)E * cap);
    d->ll_slot_of = cv.take<int32_t>((size_t)std::max(T, 1) * K);
    return cv.off;
}

// Worst-case receive rows: each token lands in at most min(K, R) buckets.
int64_t worst_rows(int T, int K, int R) { return (int64_t)T * std::min(K, R); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Stream choice and the previous_event wait; see moedx_exec.
struct Exec {
    hipStream_t caller = nullptr;
    hipStream_t run = nullptr;
    moedx_event** done = nullptr;
    bool async = false;
    hipEvent_t start = nullptr;  // stamped at the op's kernel start
    hipEvent_t stop = nullptr;   // stamped at the op's kernel end
    Launch launch() const { return Launch{run, start, stop, 0u}; }
    // An op that launches no kernel still completes its timing events.
    hipError_t no_kernel() const {
        hipError_t e = hipSuccess;
        if (start) e = hipEventRecord(start, run);
        if (e == hipSuccess && stop) e = hipEventRecord(stop, run);
        return e;
    }
};

int exec_begin(moedx_ctx* ctx, const moedx_exec* ex, Exec* out) {
    if (ex && (ex->flags & ~uint32_t(MOEDX_ON_CTX_STREAM | MOEDX_ASYNC)))
        return fail(MOEDX_EINVAL, "unknown moedx_exec flags 0x%x", ex->flags);
    out->caller = ex ? ex->stream : nullptr;
    out->done = ex ? ex->done : nullptr;
    out->async = ex && (ex->flags & MOEDX_ASYNC);
    out->start = (ex && ex->kernel_start) ? ex->kernel_start->ev : nullptr;
    out->stop = (ex && ex->kernel_stop) ? ex->kernel_stop->ev : nullptr;
    const bool on_ctx = ex && (ex->flags & MOEDX_ON_CTX_STREAM);
    out->run = on_ctx ? ctx->stream : out->caller;
    HIP_OR_FAIL(hipSetDevice(ctx->device));
    if (ex && ex->prev) HIP_OR_FAIL(hipStreamWaitEvent(out->run, ex->prev->ev, 0));
    if (on_ctx) {
        HIP_OR_FAIL(hipEventRecord(ctx->order_event, out->caller));
        HIP_OR_FAIL(hipStreamWaitEvent(out->run, ctx->order_event, 0));
    }
    return MOEDX_OK;
}

int exec_end(const Exec& ex) {
    if (ex.done) {
        moedx_event* ev = new (std::nothrow) moedx_event;
        if (!ev) return fail(MOEDX_ENOMEM, "event allocation failed");
        hipError_t e = hipEventCreateWithFlags(&ev->ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            delete ev;
            return hip_fail(e, "hipEventCreateWithFlags");
        }
        e = hipEventRecord(ev->ev, ex.run);
        if (e != hipSuccess) {
            (void)hipEventDestroy(ev->ev);
            delete ev;
            return hip_fail(e, "hipEventRecord");
        }
        *ex.done = ev;
        return MOEDX_OK;
    }
    if (!ex.async) HIP_OR_FAIL(hipStreamSynchronize(ex.run));
    return MOEDX_OK;
}

int check_ctx(const moedx_ctx* ctx) {
    if (!ctx) return fail(MOEDX_EINVAL, "ctx is NULL");
    return MOEDX_OK;
}

int check_tokens(const moedx_ctx* ctx, int T, int K) {
    if (T < 0 || T > ctx->max_tokens)
        return fail(MOEDX_EINVAL, "T=%d outside [0, max_tokens=%d]", T, ctx->max_tokens);
    if (K < 1 || K > kMaxTopk) return fail(MOEDX_EINVAL, "K=%d outside [1, %d]", K, kMaxTopk);
    return MOEDX_OK;
}

}  // namespace

// Every row kernel runs one wave per (token, slice of 64 or more chunks of 16
// bytes); keep the wave count inside a 32-bit index.
static int check_waves(int T, int H) {
    const int64_t slices = (int64_t)(H / 8 + 63) / 64;
    if ((int64_t)T * slices > ((int64_t)1 << 30))
        return fail(MOEDX_EINVAL, "T=%d x H=%d exceeds the supported row count", T, H);
    return MOEDX_OK;
}

// The layout kernel's arguments for a handle: every handle array is written.
// Only a launch whose workgroups take tickets (the layout kernel that finishes
// in its last workgroup) gets the ctx's counter; the partials-only layout, the
// finishing step alone and the first pack leave it untouched, so they may run
// while a get_dispatch_layout or prepare of the same ctx is counting.
static LayoutArgs handle_layout_args(const moedx_ctx* ctx, const moedx_handle* h,
                                     const int64_t* topk_idx, bool takes_tickets) {
    LayoutArgs a{};
    a.topk_idx = topk_idx;
    a.T = h->T;
    a.K = h->K;
    a.E = h->E;
    a.R = h->R;
    a.P = h->P;
    a.bucket = ctx->bucket;
    a.C = h->C;
    a.per = h->T > 0 ? (h->T + h->C - 1) / h->C : 1;
    a.per_div = make_fastdiv((uint32_t)a.per);
    a.is_token_in_rank = h->is_token_in_rank;
    a.token_mask = h->token_mask;
    a.slot_bucket = h->slot_bucket;
    a.num_tokens_per_rank = h->num_tokens_per_rank;
    a.num_tokens_per_expert = h->num_tokens_per_expert;
    a.rank_prefix_matrix = h->rank_prefix_matrix;
    a.num_recv = h->num_recv;
    a.group_prefix = h->group_prefix;
    a.channel_prefix_matrix = h->channel_prefix_matrix;
    a.recv_channel_prefix_matrix = h->recv_channel_prefix_matrix;
    a.group_cnt = h->group_cnt;
    a.chan_part = h->chan_part;
    a.tile_expert = h->experts_given ? nullptr : h->tile_expert;
    a.itr_in = nullptr;
    a.experts_in = nullptr;
    a.ticket = takes_tickets ? ctx->ticket : nullptr;
    return a;
}

// A handle prepared with the layout's partials only gets its prefixes from the
// finishing step, launched here on the op's stream ahead of the op's kernel.
static int finish_pending(moedx_ctx* ctx, const moedx_handle* h, hipStream_t run) {
    if (!h->prefixes_pending) return MOEDX_OK;
    HIP_OR_FAIL(launch_layout_finish(handle_layout_args(ctx, h, nullptr, false),
                                     Launch{run, nullptr, nullptr, 0u}));
    (h->experts_given ? ctx->stats.scan_launches : ctx->stats.layout_launches) += 1;
    h->prefixes_pending = false;
    return MOEDX_OK;
}

// ---- the allocation-free layout ---------------------------------------------
//
// moedx_get_dispatch_layout_static keeps what moedx_get_dispatch_layout keeps
// in a ctx's scratch (the E + R counters of the totals) in this file-scope
// device array instead: every GPU the library runs on holds its own copy,
// from the code object's load until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory): the first call on a device takes the device address with
// hipGetSymbolAddress and keeps it per device.
constexpr size_t kStaticScratchBytes = size_t(16) << 10;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
unsigned char* g_static_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The static scratch a layout of E experts in R buckets uses: its counters.
size_t static_layout_bytes(int E, int R) { return (size_t)(E + R) * 8; }

}  // namespace

// A borrowing handle's partials copied from its ctx's scratch into its own
// arrays, on `run`: the handle becomes one scanned from the layout's outputs
// whose prefixes are still pending.  `elsewhere`: the copy runs on the stream
// of another op (a layout about to overwrite the scratch); the handle's next
// op then waits for it.
static int settle_borrow(moedx_handle* h, hipStream_t run, bool elsewhere) {
    moedx_ctx* c = h->borrow_ctx;
    if (!c) return MOEDX_OK;
    AdoptArgs a{};
    a.mask_src = c->lay_mask;
    a.slot_bucket_src = c->lay_slot_bucket;
    a.group_cnt_src = c->lay_group_cnt;
    a.chan_part_src = c->lay_chan_part;
    a.experts_src = c->lay_experts;
    a.token_mask = h->token_mask;
    a.is_token_in_rank = h->is_token_in_rank;
    a.slot_bucket = h->slot_bucket;
    a.group_cnt = h->group_cnt;
    a.chan_part = h->chan_part;
    a.num_tokens_per_expert = h->num_tokens_per_expert;
    a.T = h->T;
    a.K = h->K;
    a.R = h->R;
    a.E = h->E;
    a.n_group_cnt = num_groups(h->T) * h->R;
    a.n_chan_part = (h->C + 1) * h->R;
    HIP_OR_FAIL(launch_adopt(a, Launch{run, nullptr, nullptr, 0u}));
    c->stats.scan_launches += 1;
    if (elsewhere) {
        if (!h->adopted) HIP_OR_FAIL(hipEventCreateWithFlags(&h->adopted, hipEventDisableTiming));
        HIP_OR_FAIL(hipEventRecord(h->adopted, run));
    }
    c->pending = nullptr;
    h->borrow_ctx = nullptr;
    return MOEDX_OK;
}

// Before an op reads a handle: a borrowed layout is copied in (on the op's own
// stream), and a copy enqueued on another stream is waited for.
static int handle_ready(const moedx_handle* hc, hipStream_t run) {
    moedx_handle* h = const_cast<moedx_handle*>(hc);
    if (h->orphaned)
        return fail(MOEDX_ESTATE, "the ctx whose layout this handle borrowed was destroyed "
                                  "before the handle's first use");
    if (int rc = settle_borrow(h, run, false)) return rc;
    if (h->adopted) {
        HIP_OR_FAIL(hipStreamWaitEvent(run, h->adopted, 0));
        (void)hipEventDestroy(h->adopted);
        h->adopted = nullptr;
    }
    return MOEDX_OK;
}

// A first pack that also finishes a partials-only capacity-mode handle
// (launch_pack_bf16_first, launch_pack_fp8_first).  For a handle that borrowed
// a layout's partials, the pack reads them from that ctx's scratch and writes
// the handle's per-token arrays (ht); any other handle is made ready first.
struct FirstPack {
    LayoutArgs la;
    HandleTokens ht;
    moedx_ctx* borrowed_from;
};

static int first_pack_begin(moedx_ctx* ctx, const moedx_handle* h, const int64_t* topk_idx,
                            hipStream_t run, FirstPack* fp) {
    fp->la = handle_layout_args(ctx, h, topk_idx, false);
    fp->ht = HandleTokens{};
    fp->borrowed_from = h->borrow_ctx;
    moedx_ctx* bc = fp->borrowed_from;
    if (bc) {
        fp->la.group_cnt = bc->lay_group_cnt;
        fp->la.chan_part = bc->lay_chan_part;
        fp->la.token_mask = bc->lay_mask;
        fp->la.tile_expert = nullptr;
        fp->la.experts_in = bc->lay_experts;
        fp->ht = HandleTokens{h->token_mask, h->is_token_in_rank, h->slot_bucket,
                              bc->lay_slot_bucket};
        return MOEDX_OK;
    }
    return handle_ready(h, run);  // also refuses an orphaned borrower
}

// After the first pack is enqueued on `run`: the handle is finished and, for a
// borrower, the ctx's next layout waits for this pack when it ran on another
// stream than that layout (on one stream, the stream orders them).
static int first_pack_end(const moedx_handle* h, const FirstPack& fp, hipStream_t run) {
    h->prefixes_pending = false;
    h->rows_written = true;
    moedx_ctx* bc = fp.borrowed_from;
    if (bc) {
        if (run != bc->last.stream) {
            HIP_OR_FAIL(hipEventRecord(bc->borrow_done, run));
            bc->borrow_armed = true;
        }
        bc->pending = nullptr;
        h->borrow_ctx = nullptr;
    }
    return MOEDX_OK;
}

extern "C" {

const char* moedx_last_error(void) { return g_err; }

int moedx_create(moedx_ctx** out, int device, int num_experts, int num_ranks, int num_channels,
                 int max_tokens, uint32_t flags) {
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = nullptr;
    if (flags != 0) return fail(MOEDX_EINVAL, "flags must be 0");
    if (num_ranks < 1 || num_ranks > kMaxRanks)
        return fail(MOEDX_EINVAL, "num_ranks=%d outside [1, %d]", num_ranks, kMaxRanks);
    if (num_experts < 1 || num_experts > kMaxExperts)
        return fail(MOEDX_EINVAL, "num_experts=%d outside [1, %d]", num_experts, kMaxExperts);
    if (num_experts % num_ranks != 0)
        return fail(MOEDX_EINVAL, "num_experts=%d is not a multiple of num_ranks=%d", num_experts,
                    num_ranks);
    if (num_channels < 1) return fail(MOEDX_EINVAL, "num_channels=%d < 1", num_channels);
    if (max_tokens < 0 || max_tokens > (1 << 24))
        return fail(MOEDX_EINVAL, "max_tokens=%d outside [0, 2^24]", max_tokens);
    if (device < 0) return fail(MOEDX_EINVAL, "device=%d < 0", device);

    moedx_ctx* c = new (std::nothrow) moedx_ctx();
    if (!c) return fail(MOEDX_ENOMEM, "ctx allocation failed");
    c->device = device;
    c->E = num_experts;
    c->R = num_ranks;
    c->P = num_experts / num_ranks;
    c->bucket = bucket_div(num_experts, c->P);
    if (c->bucket.mul == 0) {
        delete c;
        return fail(MOEDX_EINVAL, "no exact multiply-shift for num_experts / num_ranks");
    }
    c->C = num_channels;
    c->max_tokens = max_tokens;
    const size_t mt = (size_t)std::max(max_tokens, 1);
    const size_t ng = (size_t)std::max(num_groups(max_tokens), 1);
    const size_t off_mask = 256 + align256((size_t)(num_experts + num_ranks) * 8);
    const size_t off_sb = off_mask + align256(mt * 8);
    const size_t off_gc = off_sb + align256(mt * kMaxTopk);
    const size_t off_cp = off_gc + align256(ng * num_ranks * 4);
    const size_t off_ex = off_cp + align256((size_t)(num_channels + 1) * num_ranks * 4);
    c->scratch_bytes = off_ex + align256((size_t)num_experts * 4);
    hipError_t e = hipSetDevice(device);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking);
    if (e == hipSuccess) c->owns_stream = true;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->order_event, hipEventDisableTiming);
    if (e == hipSuccess) e = hipMalloc(&c->scratch, c->scratch_bytes);
    // the ticket and the counters start at 0 (and every launch leaves them there)
    if (e == hipSuccess) e = hipMemset(c->scratch, 0, c->scratch_bytes);
    if (e == hipSuccess) {
        char* p = static_cast<char*>(c->scratch);
        c->ticket = reinterpret_cast<unsigned int*>(p);
        c->acc = reinterpret_cast<unsigned long long*>(p + 256);
        c->lay_mask = reinterpret_cast<uint64_t*>(p + off_mask);
        c->lay_slot_bucket = reinterpret_cast<int8_t*>(p + off_sb);
        c->lay_group_cnt = reinterpret_cast<int32_t*>(p + off_gc);
        c->lay_chan_part = reinterpret_cast<int32_t*>(p + off_cp);
        c->lay_experts = reinterpret_cast<int32_t*>(p + off_ex);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->borrow_done, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&c->pinned), (size_t)(num_experts + 1) * 4,
                          hipHostMallocDefault);
    if (e != hipSuccess) {
        int rc = hip_fail(e, "moedx_create");
        moedx_destroy(c);
        return rc;
    }
    *out = c;
    return MOEDX_OK;
}

int moedx_destroy(moedx_ctx* ctx) {
    if (!ctx) return MOEDX_OK;
    if (ctx->pending) {  // it can no longer be finished
        ctx->pending->borrow_ctx = nullptr;
        ctx->pending->orphaned = true;
    }
    (void)hipSetDevice(ctx->device);
    if (ctx->stream) (void)hipStreamSynchronize(ctx->stream);
    if (ctx->scratch) (void)hipFree(ctx->scratch);
    if (ctx->pinned) (void)hipHostFree(ctx->pinned);
    if (ctx->order_event) (void)hipEventDestroy(ctx->order_event);
    if (ctx->borrow_done) (void)hipEventDestroy(ctx->borrow_done);
    if (ctx->stream && ctx->owns_stream) (void)hipStreamDestroy(ctx->stream);
    delete ctx;
    return MOEDX_OK;
}

int moedx_ctx_stats(const moedx_ctx* ctx, moedx_stats* out) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = ctx->stats;
    return MOEDX_OK;
}

int moedx_ctx_set_stream(moedx_ctx* ctx, hipStream_t stream) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!stream) return fail(MOEDX_EINVAL, "stream is NULL (the null stream cannot be the ctx's own)");
    if (stream == ctx->stream) return MOEDX_OK;
    HIP_OR_FAIL(hipSetDevice(ctx->device));
    HIP_OR_FAIL(hipStreamSynchronize(ctx->stream));  // nothing of the old stream is left behind
    if (ctx->owns_stream) HIP_OR_FAIL(hipStreamDestroy(ctx->stream));
    ctx->stream = stream;
    ctx->owns_stream = false;
    return MOEDX_OK;
}

int moedx_ctx_stream(const moedx_ctx* ctx, hipStream_t* out) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = ctx->stream;
    return MOEDX_OK;
}

// ---- events -----------------------------------------------------------------

int moedx_event_record(moedx_event** out, hipStream_t stream) {
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = nullptr;
    moedx_event* ev = new (std::nothrow) moedx_event;
    if (!ev) return fail(MOEDX_ENOMEM, "event allocation failed");
    hipError_t e = hipEventCreate(&ev->ev);
    if (e == hipSuccess) e = hipEventRecord(ev->ev, stream);
    if (e != hipSuccess) {
        (void)hipEventDestroy(ev->ev);
        delete ev;
        return hip_fail(e, "moedx_event_record");
    }
    *out = ev;
    return MOEDX_OK;
}

int moedx_event_create(moedx_event** out) {
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = nullptr;
    moedx_event* ev = new (std::nothrow) moedx_event;
    if (!ev) return fail(MOEDX_ENOMEM, "event allocation failed");
    hipError_t e = hipEventCreate(&ev->ev);
    if (e != hipSuccess) {
        delete ev;
        return hip_fail(e, "moedx_event_create");
    }
    *out = ev;
    return MOEDX_OK;
}

int moedx_event_wait(const moedx_event* ev, hipStream_t stream) {
    if (!ev) return fail(MOEDX_EINVAL, "event is NULL");
    HIP_OR_FAIL(hipStreamWaitEvent(stream, ev->ev, 0));
    return MOEDX_OK;
}

int moedx_event_synchronize(const moedx_event* ev) {
    if (!ev) return fail(MOEDX_EINVAL, "event is NULL");
    HIP_OR_FAIL(hipEventSynchronize(ev->ev));
    return MOEDX_OK;
}

int moedx_event_elapsed_ms(const moedx_event* start, const moedx_event* end, float* ms) {
    if (!start || !end || !ms) return fail(MOEDX_EINVAL, "NULL argument");
    HIP_OR_FAIL(hipEventElapsedTime(ms, start->ev, end->ev));
    return MOEDX_OK;
}

int moedx_event_destroy(moedx_event* ev) {
    if (!ev) return MOEDX_OK;
    (void)hipEventDestroy(ev->ev);
    delete ev;
    return MOEDX_OK;
}

// ---- layout -----------------------------------------------------------------

int moedx_get_dispatch_layout(moedx_ctx* ctx, const int64_t* topk_idx, int T, int K,
                              int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                              uint8_t* is_token_in_rank, const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (int rc = check_tokens(ctx, T, K)) return rc;
    if ((T > 0 && (!topk_idx || !is_token_in_rank)) || !num_tokens_per_rank ||
        !num_tokens_per_expert)
        return fail(MOEDX_EINVAL, "NULL device pointer");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    // The scratch is about to be rewritten: a handle still borrowing it gets
    // its copy first, and a first pack that read it must have finished.
    if (ctx->pending) {
        if (int rc = settle_borrow(ctx->pending, ex.run, true)) return rc;
    }
    if (ctx->borrow_armed) {
        HIP_OR_FAIL(hipStreamWaitEvent(ex.run, ctx->borrow_done, 0));
        ctx->borrow_armed = false;
    }
    LayoutArgs a{};
    a.topk_idx = topk_idx;
    a.T = T;
    a.K = K;
    a.E = ctx->E;
    a.R = ctx->R;
    a.P = ctx->P;
    a.bucket = ctx->bucket;
    a.C = ctx->C;
    a.per = T > 0 ? (T + ctx->C - 1) / ctx->C : 1;
    a.per_div = make_fastdiv((uint32_t)a.per);
    a.is_token_in_rank = is_token_in_rank;
    a.num_tokens_per_rank = num_tokens_per_rank;
    a.num_tokens_per_expert = num_tokens_per_expert;
    // the partials a handle prepared from these outputs borrows
    a.token_mask = ctx->lay_mask;
    a.slot_bucket = ctx->lay_slot_bucket;
    a.group_cnt = ctx->lay_group_cnt;
    a.chan_part = ctx->lay_chan_part;
    a.experts_copy = ctx->lay_experts;
    ctx->last.valid = false;
    HIP_OR_FAIL(launch_layout_totals(a, ctx->acc, ex.launch()));
    ctx->stats.layout_launches += 1;
    ctx->last.valid = true;
    ctx->last.topk_idx = topk_idx;
    ctx->last.is_token_in_rank = is_token_in_rank;
    ctx->last.num_tokens_per_expert = num_tokens_per_expert;
    ctx->last.T = T;
    ctx->last.K = K;
    ctx->last.stream = ex.run;
    return exec_end(ex);
}

int moedx_get_dispatch_layout_static(const int64_t* topk_idx, int T, int K, int E, int R,
                                     int32_t* num_tokens_per_rank,
                                     int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                     hipStream_t stream) {
    if (R < 1 || R > kMaxRanks) return fail(MOEDX_EINVAL, "R=%d outside [1, %d]", R, kMaxRanks);
    if (E < 1 || E > kMaxExperts)
        return fail(MOEDX_EINVAL, "E=%d outside [1, %d]", E, kMaxExperts);
    if (E % R != 0) return fail(MOEDX_EINVAL, "E=%d is not a multiple of R=%d", E, R);
    if (K < 1 || K > kMaxTopk) return fail(MOEDX_EINVAL, "K=%d outside [1, %d]", K, kMaxTopk);
    if (T < 0 || T > (1 << 24)) return fail(MOEDX_EINVAL, "T=%d outside [0, 2^24]", T);
    if ((T > 0 && (!topk_idx || !is_token_in_rank)) || !num_tokens_per_rank ||
        !num_tokens_per_expert)
        return fail(MOEDX_EINVAL, "NULL device pointer");
    const size_t need = static_layout_bytes(E, R);
    if (need > kStaticScratchBytes)  // not reached within the bounds above
        return fail(MOEDX_ECAPACITY,
                    "E=%d, R=%d need %zu bytes of the static scratch, which holds %zu "
                    "(use moedx_get_dispatch_layout with a ctx)",
                    E, R, need, kStaticScratchBytes);
    const BucketDiv bucket = bucket_div(E, E / R);
    if (bucket.mul == 0) return fail(MOEDX_EINVAL, "no exact multiply-shift for E / R");
    int dev = 0;
    HIP_OR_FAIL(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOEDX_EINVAL, "device %d >= %d", dev, kMaxDevices);
    const Launch L{stream, nullptr, nullptr, 0u};
    unsigned char* base = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        if (!g_static_ptr[dev]) {  // once per device, with that device current
            void* p = nullptr;
            HIP_OR_FAIL(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
            if (!p) return fail(MOEDX_EHIP, "hipGetSymbolAddress gave no address");
            // The counters must start at zero (every launch leaves them
            // there): cleared on this stream ahead of the first layout.  The
            // address is kept only once the clear is enqueued.
            HIP_OR_FAIL(launch_zero_words(static_cast<uint32_t*>(p), (int)(kStaticScratchBytes / 4), L));
            g_static_ptr[dev] = static_cast<unsigned char*>(p);
        }
        base = g_static_ptr[dev];
    }
    LayoutArgs a{};
    a.topk_idx = topk_idx;
    a.T = T;
    a.K = K;
    a.E = E;
    a.R = R;
    a.P = E / R;
    a.bucket = bucket;
    a.C = 1;
    a.per = T > 0 ? T : 1;
    a.per_div = make_fastdiv((uint32_t)a.per);
    a.is_token_in_rank = is_token_in_rank;
    a.num_tokens_per_rank = num_tokens_per_rank;
    a.num_tokens_per_expert = num_tokens_per_expert;
    HIP_OR_FAIL(launch_layout_totals(a, reinterpret_cast<unsigned long long*>(base), L));
    return MOEDX_OK;
}

// ---- handle -----------------------------------------------------------------

int moedx_handle_workspace_bytes(const moedx_ctx* ctx, int T, int K, int64_t capacity_rows,
                                 size_t* bytes) {
    if (int rc = check_ctx(ctx)) return rc;
    if (int rc = check_tokens(ctx, T, K)) return rc;
    if (!bytes) return fail(MOEDX_EINVAL, "bytes is NULL");
    if (capacity_rows < 0) return fail(MOEDX_EINVAL, "capacity_rows < 0");
    const int64_t rows = capacity_rows > 0 ? capacity_rows : worst_rows(T, K, ctx->R);
    *bytes = carve_normal(nullptr, nullptr, T, K, ctx->E, ctx->R, ctx->C, rows);
    return MOEDX_OK;
}

int moedx_dispatch_prepare(moedx_ctx* ctx, const int64_t* topk_idx, int T, int K,
                           const int32_t* num_tokens_per_rank, const uint8_t* is_token_in_rank,
                           const int32_t* num_tokens_per_expert, void* workspace,
                           size_t workspace_bytes, int64_t capacity_rows, moedx_handle** out,
                           const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = nullptr;
    if (int rc = check_tokens(ctx, T, K)) return rc;
    if ((T > 0 && !topk_idx) || !workspace) return fail(MOEDX_EINVAL, "NULL device pointer");
    // From layout outputs: num_tokens_per_expert, with is_token_in_rank (which
    // an empty batch need not name); num_tokens_per_rank only together with them.
    const bool from_layout = num_tokens_per_expert != nullptr;
    if (from_layout ? (T > 0 && !is_token_in_rank) : (is_token_in_rank || num_tokens_per_rank))
        return fail(MOEDX_EINVAL,
                    "is_token_in_rank and num_tokens_per_expert go together, and "
                    "num_tokens_per_rank is given only with them");
    if (from_layout && (!aligned4(num_tokens_per_expert) ||
                        ((ctx->R & 3) == 0 && !aligned4(is_token_in_rank))))
        return fail(MOEDX_EINVAL, "layout outputs are misaligned (int32: 4 bytes; "
                                  "is_token_in_rank rows of a multiple of 4 buckets: 4 bytes)");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(MOEDX_EINVAL, "workspace is not 256-byte aligned");
    if (capacity_rows < 0) return fail(MOEDX_EINVAL, "capacity_rows < 0");
    const int64_t worst = worst_rows(T, K, ctx->R);
    if (capacity_rows > 0 && capacity_rows < worst)
        return fail(MOEDX_ECAPACITY, "capacity_rows=%lld < T*min(K,R)=%lld",
                    (long long)capacity_rows, (long long)worst);
    const int64_t rows = capacity_rows > 0 ? capacity_rows : worst;
    const size_t need = carve_normal(nullptr, nullptr, T, K, ctx->E, ctx->R, ctx->C, rows);
    if (workspace_bytes < need)
        return fail(MOEDX_ECAPACITY, "workspace_bytes=%zu < %zu", workspace_bytes, need);

    moedx_handle* h = new (std::nothrow) moedx_handle();
    if (!h) return fail(MOEDX_ENOMEM, "handle allocation failed");
    h->kind = kNormal;
    h->T = T;
    h->K = K;
    h->E = ctx->E;
    h->R = ctx->R;
    h->P = ctx->P;
    h->C = ctx->C;
    h->capacity = capacity_rows;
    h->n_host = -1;
    h->experts_given = from_layout;
    carve_normal(h, static_cast<char*>(workspace), T, K, ctx->E, ctx->R, ctx->C, rows);

    Exec ex;
    int rc = exec_begin(ctx, exec, &ex);
    hipError_t e = hipSuccess;
    // Capacity mode, where a first dispatch (bf16, FP8 or pre-quantised) can
    // finish the prefixes in its own launch: the partials only, and the first
    // dispatch (or combine) on the handle finishes them.  Elsewhere the layout
    // kernel writes every prefix itself.
    const bool partials = capacity_rows > 0 && T > 0 && pack_first_fits(T, h->R, h->E, h->C);
    // Given exactly the outputs of this ctx's last get_dispatch_layout, the
    // handle borrows the partials that call left in the ctx's scratch: nothing
    // runs now, and the first pack finishes the handle from them.
    const bool borrow = partials && from_layout && ctx->last.valid &&
                        ctx->last.topk_idx == topk_idx &&
                        ctx->last.is_token_in_rank == is_token_in_rank &&
                        ctx->last.num_tokens_per_expert == num_tokens_per_expert &&
                        ctx->last.T == T && ctx->last.K == K;
    if (rc == MOEDX_OK && borrow) {
        if (ctx->pending) rc = settle_borrow(ctx->pending, ex.run, true);  // one borrower at a time
        if (rc == MOEDX_OK) {
            e = ex.no_kernel();
            if (e != hipSuccess) rc = hip_fail(e, "event record");
        }
        h->prefixes_pending = true;
    } else if (rc == MOEDX_OK) {
        LayoutArgs a = handle_layout_args(ctx, h, topk_idx, !partials);
        if (from_layout) {  // the scan of the given layout outputs
            a.itr_in = is_token_in_rank;
            a.experts_in = num_tokens_per_expert;
        }
        e = partials ? launch_layout_partials(a, ex.launch()) : launch_layout(a, ex.launch());
        h->prefixes_pending = partials;
        if (e != hipSuccess) rc = hip_fail(e, "layout launch");
        if (rc == MOEDX_OK)
            (from_layout ? ctx->stats.scan_launches : ctx->stats.layout_launches) += 1;
    }
    if (rc == MOEDX_OK && capacity_rows == 0) {
        // Exact mode: the host waits for N and the per-expert counts.
        e = hipMemcpyAsync(ctx->pinned, h->num_recv, (size_t)(1 + h->E) * 4,
                           hipMemcpyDeviceToHost, ex.run);
        if (e == hipSuccess) e = hipStreamSynchronize(ex.run);
        if (e != hipSuccess) {
            rc = hip_fail(e, "exact-mode count readback");
        } else {
            ctx->stats.host_syncs += 1;
            h->n_host = ctx->pinned[0];
            h->per_expert_host.assign(ctx->pinned + 1, ctx->pinned + 1 + h->E);
        }
    }
    if (rc == MOEDX_OK) rc = exec_end(ex);
    if (rc != MOEDX_OK) {
        delete h;
        return rc;
    }
    if (borrow) {
        h->borrow_ctx = ctx;
        ctx->pending = h;
    }
    *out = h;
    return MOEDX_OK;
}

int moedx_handle_num_recv(const moedx_handle* h, int64_t* n) {
    if (!h || !n) return fail(MOEDX_EINVAL, "NULL argument");
    if (h->kind != kNormal || h->capacity != 0)
        return fail(MOEDX_ESTATE, "N is on the host only for exact-mode normal handles");
    *n = h->n_host;
    return MOEDX_OK;
}

int moedx_handle_recv_tokens_per_expert(const moedx_handle* h, int32_t* host_counts) {
    if (!h || !host_counts) return fail(MOEDX_EINVAL, "NULL argument");
    if (h->kind != kNormal || h->capacity != 0)
        return fail(MOEDX_ESTATE, "counts are on the host only for exact-mode normal handles");
    std::memcpy(host_counts, h->per_expert_host.data(), (size_t)h->E * 4);
    return MOEDX_OK;
}

int moedx_handle_tensor(const moedx_handle* h, int which, const void** dev, int64_t shape[2]) {
    if (!h || !dev || !shape) return fail(MOEDX_EINVAL, "NULL argument");
    const void* p = nullptr;
    int64_t s0 = 0, s1 = 1;
    if (h->kind == kNormal) {
        switch (which) {
            case MOEDX_T_RANK_PREFIX_MATRIX: p = h->rank_prefix_matrix; s0 = h->R; break;
            case MOEDX_T_CHANNEL_PREFIX_MATRIX:
                p = h->channel_prefix_matrix; s0 = h->R; s1 = h->C; break;
            case MOEDX_T_RECV_CHANNEL_PREFIX_MATRIX:
                p = h->recv_channel_prefix_matrix; s0 = h->R; s1 = h->C; break;
            case MOEDX_T_RECV_SRC_IDX:
                p = h->recv_src_idx; s0 = h->capacity > 0 ? h->capacity : h->n_host; break;
            case MOEDX_T_IS_TOKEN_IN_RANK: p = h->is_token_in_rank; s0 = h->T; s1 = h->R; break;
            case MOEDX_T_SEND_HEAD: p = h->send_head; s0 = h->T; s1 = h->R; break;
            case MOEDX_T_NUM_TOKENS_PER_RANK: p = h->num_tokens_per_rank; s0 = h->R; break;
            case MOEDX_T_NUM_TOKENS_PER_EXPERT: p = h->num_tokens_per_expert; s0 = h->E; break;
            case MOEDX_T_NUM_RECV: p = h->num_recv; s0 = 1; break;
            default: return fail(MOEDX_EINVAL, "tensor %d is not part of a normal handle", which);
        }
    } else {
        switch (which) {
            case MOEDX_T_LL_SRC_IDX: p = h->ll_src_idx; s0 = h->E; s1 = h->cap; break;
            case MOEDX_T_LL_SLOT_OF: p = h->ll_slot_of; s0 = h->T; s1 = h->K; break;
            default:
                return fail(MOEDX_EINVAL, "tensor %d is not part of a low-latency handle", which);
        }
    }
    *dev = p;
    shape[0] = s0;
    shape[1] = s1;
    return MOEDX_OK;
}

int moedx_handle_finish(moedx_ctx* ctx, const moedx_handle* h, const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kNormal) return fail(MOEDX_EINVAL, "a normal handle is required");
    if (h->E != ctx->E || h->R != ctx->R || h->C != ctx->C)
        return fail(MOEDX_ESTATE, "handle was prepared on a ctx with a different E/R/C");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    if (int rc = handle_ready(h, ex.run)) return rc;
    if (h->prefixes_pending) {
        HIP_OR_FAIL(launch_layout_finish(handle_layout_args(ctx, h, nullptr, false), ex.launch()));
        (h->experts_given ? ctx->stats.scan_launches : ctx->stats.layout_launches) += 1;
        h->prefixes_pending = false;
    } else {
        HIP_OR_FAIL(ex.no_kernel());
    }
    return exec_end(ex);
}

int moedx_handle_destroy(moedx_handle* h) {
    if (!h) return MOEDX_OK;
    if (h->borrow_ctx && h->borrow_ctx->pending == h) h->borrow_ctx->pending = nullptr;
    if (h->adopted) (void)hipEventDestroy(h->adopted);
    delete h;
    return MOEDX_OK;
}

// ---- dispatch / combine -------------------------------------------------------

int moedx_dispatch(moedx_ctx* ctx, const moedx_handle* h, const void* x, int T, int H, int quant,
                   const int64_t* topk_idx, const float* topk_weights, void* recv_x,
                   float* recv_scales, int64_t* recv_topk_idx, float* recv_topk_weights,
                   const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kNormal) return fail(MOEDX_EINVAL, "a normal handle is required");
    if (T != h->T) return fail(MOEDX_ESTATE, "T=%d differs from the handle's T=%d", T, h->T);
    if (h->E != ctx->E || h->R != ctx->R || h->C != ctx->C)
        return fail(MOEDX_ESTATE, "handle was prepared on a ctx with a different E/R/C");
    if (H < 8 || H % 8 != 0) return fail(MOEDX_EINVAL, "H=%d must be a positive multiple of 8", H);
    if (int rc = check_waves(T, H)) return rc;
    if (quant != MOEDX_QUANT_NONE && quant != MOEDX_QUANT_FP8_E4M3_1X128)
        return fail(MOEDX_EINVAL, "unknown quant mode %d", quant);
    if (quant == MOEDX_QUANT_FP8_E4M3_1X128 && H % 128 != 0)
        return fail(MOEDX_EINVAL, "FP8 dispatch needs H %% 128 == 0 (H=%d)", H);
    if (T > 0 && (!x || !recv_x)) return fail(MOEDX_EINVAL, "NULL device pointer");
    if ((T > 0) && (!aligned16(x) || !aligned16(recv_x)))
        return fail(MOEDX_EINVAL, "x and recv_x must be 16-byte aligned");
    if (quant == MOEDX_QUANT_FP8_E4M3_1X128 && T > 0 && !recv_scales)
        return fail(MOEDX_EINVAL, "FP8 dispatch needs recv_scales");
    if (quant == MOEDX_QUANT_NONE && recv_scales)
        return fail(MOEDX_EINVAL, "recv_scales is only produced by FP8 dispatch");
    const bool reuse = (topk_idx == nullptr);
    if (T > 0 && reuse && (topk_weights || recv_topk_idx || recv_topk_weights))
        return fail(MOEDX_EINVAL,
                    "cached dispatch takes no topk_weights and produces no recv_topk_*");
    if (!reuse && (recv_topk_weights && !topk_weights))
        return fail(MOEDX_EINVAL, "recv_topk_weights needs topk_weights");
    if (!reuse && !recv_topk_idx && recv_topk_weights)
        return fail(MOEDX_EINVAL, "recv_topk_weights needs recv_topk_idx");
    if (quant == MOEDX_QUANT_FP8_E4M3_1X128 && (recv_topk_idx || recv_topk_weights))
        return fail(MOEDX_EINVAL, "FP8 dispatch does not produce recv_topk_*");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    const RowMap rm{h->token_mask, h->group_prefix, h->rank_prefix_matrix, h->num_tokens_per_rank,
                    h->R, h->T, h->capacity > 0 ? h->capacity : h->n_host};
    // The first dispatch on a handle also writes send_head and recv_src_idx.
    const HandleRows hr = h->rows_written ? HandleRows{nullptr, nullptr}
                                          : HandleRows{h->send_head, h->recv_src_idx};
    if (T > 0 && h->prefixes_pending && pack_first_fits(T, h->R, h->E, h->C)) {
        // One launch finishes the handle and packs the rows.
        FirstPack fp;
        if (int rc = first_pack_begin(ctx, h, topk_idx, ex.run, &fp)) return rc;
        if (quant == MOEDX_QUANT_NONE) {
            HIP_OR_FAIL(launch_pack_bf16_first(fp.la, fp.ht, x, H, h->capacity, hr, recv_x,
                                               topk_weights, recv_topk_idx, recv_topk_weights,
                                               ex.launch()));
            ctx->stats.pack_launches += 1;
        } else {
            HIP_OR_FAIL(launch_pack_fp8_first(fp.la, fp.ht, x, H, h->capacity, hr, recv_x,
                                              recv_scales, MOEDX_FP8_SCALE_AMAX, 0.0f,
                                              ex.launch()));
            ctx->stats.pack_fp8_launches += 1;
        }
        if (int rc = first_pack_end(h, fp, ex.run)) return rc;
        return exec_end(ex);
    }
    if (int rc = handle_ready(h, ex.run)) return rc;
    if (int rc = finish_pending(ctx, h, ex.run)) return rc;
    if (T == 0) {
        HIP_OR_FAIL(ex.no_kernel());
    } else if (quant == MOEDX_QUANT_NONE) {
        HIP_OR_FAIL(launch_pack_bf16(x, T, H, rm, hr, recv_x, topk_idx, topk_weights, h->K, h->E,
                                     h->P, ctx->bucket, recv_topk_idx, recv_topk_weights,
                                     ex.launch()));
        ctx->stats.pack_launches += 1;
    } else {
        HIP_OR_FAIL(launch_pack_fp8(x, T, H, rm, hr, recv_x, recv_scales, MOEDX_FP8_SCALE_AMAX,
                                    0.0f, ex.launch()));
        ctx->stats.pack_fp8_launches += 1;
    }
    h->rows_written = true;
    return exec_end(ex);
}

int moedx_dispatch_fp8(moedx_ctx* ctx, const moedx_handle* h, const void* x, int T, int H,
                       const moedx_fp8* fp8, uint8_t* recv_x, void* recv_scales,
                       const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kNormal) return fail(MOEDX_EINVAL, "a normal handle is required");
    if (T != h->T) return fail(MOEDX_ESTATE, "T=%d differs from the handle's T=%d", T, h->T);
    if (h->E != ctx->E || h->R != ctx->R || h->C != ctx->C)
        return fail(MOEDX_ESTATE, "handle was prepared on a ctx with a different E/R/C");
    if (!fp8) return fail(MOEDX_EINVAL, "fp8 options are NULL");
    const int mode = fp8->scale_mode;
    if (mode < MOEDX_FP8_SCALE_AMAX || mode > MOEDX_FP8_SCALE_TENSOR)
        return fail(MOEDX_EINVAL, "unknown FP8 scale mode %d", mode);
    if (H < 128 || H % 128 != 0)
        return fail(MOEDX_EINVAL, "FP8 dispatch needs H %% 128 == 0 (H=%d)", H);
    if (int rc = check_waves(T, H)) return rc;
    const bool tensor = mode == MOEDX_FP8_SCALE_TENSOR;
    if (tensor) {
        const float s = fp8->tensor_scale;
        // a positive normal scale whose reciprocal is normal too
        if (!(s >= 0x1p-126f && s < 0x1p126f))
            return fail(MOEDX_EINVAL, "tensor_scale=%g outside [2^-126, 2^126)", (double)s);
    }
    if (fp8->prequantized && !tensor && !fp8->x_scales)
        return fail(MOEDX_EINVAL, "pre-quantised input needs x_scales");
    if ((!fp8->prequantized || tensor) && fp8->x_scales)
        return fail(MOEDX_EINVAL, "x_scales is read only for pre-quantised input with scales");
    if (T > 0 && (!x || !recv_x)) return fail(MOEDX_EINVAL, "NULL device pointer");
    if (T > 0 && (!aligned16(x) || !aligned16(recv_x)))
        return fail(MOEDX_EINVAL, "x and recv_x must be 16-byte aligned");
    if (T > 0 && !tensor && !recv_scales) return fail(MOEDX_EINVAL, "recv_scales is NULL");
    if (tensor && recv_scales)
        return fail(MOEDX_EINVAL, "a per-tensor scale writes no recv_scales");
    if ((T > 0 && !tensor && !aligned4(recv_scales)) ||
        (fp8->x_scales && mode != MOEDX_FP8_SCALE_UE8M0 && !aligned4(fp8->x_scales)))
        return fail(MOEDX_EINVAL, "fp32 scales must be 4-byte aligned");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    const RowMap rm{h->token_mask, h->group_prefix, h->rank_prefix_matrix, h->num_tokens_per_rank,
                    h->R, h->T, h->capacity > 0 ? h->capacity : h->n_host};
    const HandleRows hr = h->rows_written ? HandleRows{nullptr, nullptr}
                                          : HandleRows{h->send_head, h->recv_src_idx};
    const int sb = tensor ? 0 : (H / 128) * (mode == MOEDX_FP8_SCALE_UE8M0 ? 1 : 4);
    if (T > 0 && h->prefixes_pending && pack_first_fits(T, h->R, h->E, h->C)) {
        // One launch finishes the handle and quantises (or copies) and packs the rows.
        FirstPack fp;
        if (int rc = first_pack_begin(ctx, h, nullptr, ex.run, &fp)) return rc;
        if (fp8->prequantized) {
            HIP_OR_FAIL(launch_pack_bytes_first(fp.la, fp.ht, x, fp8->x_scales, H, sb, h->capacity,
                                                hr, recv_x, recv_scales, ex.launch()));
        } else {
            HIP_OR_FAIL(launch_pack_fp8_first(fp.la, fp.ht, x, H, h->capacity, hr, recv_x,
                                              recv_scales, mode, fp8->tensor_scale, ex.launch()));
        }
        ctx->stats.pack_fp8_launches += 1;
        if (int rc = first_pack_end(h, fp, ex.run)) return rc;
        return exec_end(ex);
    }
    if (int rc = handle_ready(h, ex.run)) return rc;
    if (int rc = finish_pending(ctx, h, ex.run)) return rc;
    if (T == 0) {
        HIP_OR_FAIL(ex.no_kernel());
    } else if (fp8->prequantized) {
        HIP_OR_FAIL(launch_pack_bytes(x, fp8->x_scales, T, H, sb, rm, hr, recv_x, recv_scales,
                                      ex.launch()));
        ctx->stats.pack_fp8_launches += 1;
    } else {
        HIP_OR_FAIL(launch_pack_fp8(x, T, H, rm, hr, recv_x, recv_scales, mode,
                                    fp8->tensor_scale, ex.launch()));
        ctx->stats.pack_fp8_launches += 1;
    }
    h->rows_written = true;
    return exec_end(ex);
}

int moedx_combine(moedx_ctx* ctx, const moedx_handle* h, const uint16_t* y, int H,
                  const float* gate_weights, const float* recv_topk_weights, uint16_t* out,
                  float* combined_topk_weights, const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kNormal) return fail(MOEDX_EINVAL, "a normal handle is required");
    if (h->E != ctx->E || h->R != ctx->R || h->C != ctx->C)
        return fail(MOEDX_ESTATE, "handle was prepared on a ctx with a different E/R/C");
    if (H < 8 || H % 8 != 0) return fail(MOEDX_EINVAL, "H=%d must be a positive multiple of 8", H);
    if (int rc = check_waves(h->T, H)) return rc;
    // y may be NULL only when there is provably no receive row (exact mode, N = 0)
    const bool no_rows = h->capacity == 0 && h->n_host == 0;
    if (h->T > 0 && (!out || (!y && !no_rows))) return fail(MOEDX_EINVAL, "NULL device pointer");
    if (h->T > 0 && (!aligned16(y) || !aligned16(out)))
        return fail(MOEDX_EINVAL, "y and out must be 16-byte aligned");
    if (h->T > 0 && (combined_topk_weights != nullptr) != (recv_topk_weights != nullptr))
        return fail(MOEDX_EINVAL,
                    "recv_topk_weights and combined_topk_weights go together");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    const RowMap rm{h->token_mask, h->group_prefix, h->rank_prefix_matrix, h->num_tokens_per_rank,
                    h->R, h->T, h->capacity > 0 ? h->capacity : h->n_host};
    if (int rc = handle_ready(h, ex.run)) return rc;
    if (int rc = finish_pending(ctx, h, ex.run)) return rc;
    if (h->T == 0) {
        HIP_OR_FAIL(ex.no_kernel());
    } else {
        HIP_OR_FAIL(launch_combine(y, h->T, H, h->K, rm, h->slot_bucket, gate_weights,
                                   recv_topk_weights, out, combined_topk_weights, ex.launch()));
        ctx->stats.combine_launches += 1;
    }
    return exec_end(ex);
}

// ---- low-latency ----------------------------------------------------------------

int moedx_ll_workspace_bytes(const moedx_ctx* ctx, int T, int K,
                             int num_max_dispatch_tokens_per_rank, size_t* bytes) {
    if (int rc = check_ctx(ctx)) return rc;
    if (int rc = check_tokens(ctx, T, K)) return rc;
    if (!bytes) return fail(MOEDX_EINVAL, "bytes is NULL");
    if (num_max_dispatch_tokens_per_rank < 1)
        return fail(MOEDX_EINVAL, "num_max_dispatch_tokens_per_rank < 1");
    *bytes = carve_ll(nullptr, nullptr, T, K, ctx->E, num_max_dispatch_tokens_per_rank);
    return MOEDX_OK;
}

int moedx_ll_dispatch(moedx_ctx* ctx, const uint16_t* x, const int64_t* topk_idx, int T, int K,
                      int H, int num_max_dispatch_tokens_per_rank, uint16_t* recv_x,
                      int32_t* recv_count, void* workspace, size_t workspace_bytes,
                      moedx_handle** out, const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!out) return fail(MOEDX_EINVAL, "out is NULL");
    *out = nullptr;
    if (int rc = check_tokens(ctx, T, K)) return rc;
    const int cap = num_max_dispatch_tokens_per_rank;
    if (cap < 1) return fail(MOEDX_EINVAL, "num_max_dispatch_tokens_per_rank < 1");
    if (T > cap)
        return fail(MOEDX_ECAPACITY, "T=%d exceeds num_max_dispatch_tokens_per_rank=%d", T, cap);
    if ((int64_t)ctx->E * cap > INT32_MAX)
        return fail(MOEDX_EINVAL,
                    "num_experts * num_max_dispatch_tokens_per_rank exceeds 2^31 - 1");
    if (H < 8 || H % 8 != 0) return fail(MOEDX_EINVAL, "H=%d must be a positive multiple of 8", H);
    // recv_x == NULL defers the rows to moedx_ll_dispatch_recv (x is then unused)
    if (!recv_count || !workspace || (T > 0 && (!topk_idx || (recv_x && !x))))
        return fail(MOEDX_EINVAL, "NULL device pointer");
    if (T > 0 && recv_x && (!aligned16(x) || !aligned16(recv_x)))
        return fail(MOEDX_EINVAL, "x and recv_x must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(MOEDX_EINVAL, "workspace is not 256-byte aligned");
    const size_t need = carve_ll(nullptr, nullptr, T, K, ctx->E, cap);
    if (workspace_bytes < need)
        return fail(MOEDX_ECAPACITY, "workspace_bytes=%zu < %zu", workspace_bytes, need);
    moedx_handle* h = new (std::nothrow) moedx_handle();
    if (!h) return fail(MOEDX_ENOMEM, "handle allocation failed");
    h->kind = kLowLatency;
    h->T = T;
    h->K = K;
    h->E = ctx->E;
    h->R = ctx->R;
    h->P = ctx->P;
    h->C = ctx->C;
    h->cap = cap;
    carve_ll(h, static_cast<char*>(workspace), T, K, ctx->E, cap);
    Exec ex;
    int rc = exec_begin(ctx, exec, &ex);
    if (rc == MOEDX_OK) {
        hipError_t e = launch_ll_dispatch(x, topk_idx, T, K, H, h->E, cap, recv_x, recv_count,
                                          h->ll_src_idx, h->ll_slot_of, ex.launch());
        if (e != hipSuccess) rc = hip_fail(e, "ll dispatch launch");
    }
    if (rc == MOEDX_OK) {
        ctx->stats.ll_dispatch_launches += 1;
        rc = exec_end(ex);
    }
    if (rc != MOEDX_OK) {
        delete h;
        return rc;
    }
    *out = h;
    return MOEDX_OK;
}

int moedx_ll_dispatch_recv(moedx_ctx* ctx, const moedx_handle* h, const uint16_t* x,
                           const int64_t* topk_idx, int H, uint16_t* recv_x,
                           const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kLowLatency) return fail(MOEDX_EINVAL, "a low-latency handle is required");
    if (h->E != ctx->E) return fail(MOEDX_ESTATE, "handle was made on a ctx with a different E");
    if (H < 8 || H % 8 != 0) return fail(MOEDX_EINVAL, "H=%d must be a positive multiple of 8", H);
    if (h->T > 0 && (!x || !topk_idx || !recv_x)) return fail(MOEDX_EINVAL, "NULL device pointer");
    if (h->T > 0 && (!aligned16(x) || !aligned16(recv_x)))
        return fail(MOEDX_EINVAL, "x and recv_x must be 16-byte aligned");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    if (h->T == 0) {
        HIP_OR_FAIL(ex.no_kernel());
    } else {
        HIP_OR_FAIL(launch_ll_recv(x, topk_idx, h->ll_slot_of, h->T, h->K, H, h->E, h->cap, recv_x,
                                   ex.launch()));
        ctx->stats.ll_dispatch_launches += 1;
    }
    return exec_end(ex);
}

int moedx_ll_combine(moedx_ctx* ctx, const uint16_t* y, const int64_t* topk_idx,
                     const float* topk_weights, const moedx_handle* h, int H, uint16_t* out,
                     const moedx_exec* exec) {
    if (int rc = check_ctx(ctx)) return rc;
    if (!h || h->kind != kLowLatency) return fail(MOEDX_EINVAL, "a low-latency handle is required");
    if (h->E != ctx->E) return fail(MOEDX_ESTATE, "handle was made on a ctx with a different E");
    if (H < 8 || H % 8 != 0) return fail(MOEDX_EINVAL, "H=%d must be a positive multiple of 8", H);
    if (h->T > 0 && (!y || !topk_idx || !topk_weights || !out))
        return fail(MOEDX_EINVAL, "NULL device pointer");
    if (h->T > 0 && (!aligned16(y) || !aligned16(out)))
        return fail(MOEDX_EINVAL, "y and out must be 16-byte aligned");
    Exec ex;
    if (int rc = exec_begin(ctx, exec, &ex)) return rc;
    if (h->T == 0) {
        HIP_OR_FAIL(ex.no_kernel());
    } else {
        HIP_OR_FAIL(launch_ll_combine(y, topk_idx, topk_weights, h->ll_slot_of, h->T, h->K, H,
                                      h->E, h->cap, out, ex.launch()));
        ctx->stats.ll_combine_launches += 1;
    }
    return exec_end(ex);
}

}  // extern "C"
