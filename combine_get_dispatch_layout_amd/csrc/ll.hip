// Low-latency dispatch and combine kernels for gfx950.
//
// The low-latency example of the EnflameTechnology/DeepEP README (and the
// two-phase kernel on "How DeepEP Enables Hook-Based Overlapping Without SM
// Occupation") receives tokens into per-expert slots of a fixed capacity,
// num_max_dispatch_tokens_per_rank, and returns per-expert counts; the
// low-latency combine weights each expert's output row by the token's top-k
// weight.  Slots are filled in ascending token order, so slot positions are a
// pure function of the routing.
//
// Decode batches are small (the README recommends fewer than 256 tokens), so
// the dispatch is a single launch: each workgroup owns one token (or a slice
// of its row) and finds the token's slot in every chosen expert by counting,
// with wave ballots, the earlier tokens that chose the same expert.  That is
// O(T*K) reads per workgroup, all from L2, and saves a separate count kernel;
// one extra workgroup of the same launch writes the per-expert counts.  The
// row chunk is loaded before the counting so the two latencies overlap, and
// the combine issues the loads of up to 8 slot rows before its first FMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

#ifndef MOEDX_LL_TARGET_WG
#define MOEDX_LL_TARGET_WG 512  // dispatch workgroups a small batch is spread over
#endif
#ifndef MOEDX_LL_COMBINE_TARGET_WG
#define MOEDX_LL_COMBINE_TARGET_WG 1024  // combine workgroups
#endif
#ifndef MOEDX_LL_MIN_CHUNKS
#define MOEDX_LL_MIN_CHUNKS 64  // fewest 16-byte chunks of a row per workgroup
#endif

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.  Both
// results are computed and one is selected (no branch per value).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

constexpr int kCountBatch = 4;  // earlier entries each thread loads per pass
constexpr int kVisitBatch = 8;  // slot rows whose loads one combine pass issues together

// grid = T * slices (+1): workgroup b < T * slices handles token b / slices,
// row slice b % slices; the extra last workgroup writes every expert's count.
// cnt[k] += entries among v (kCountBatch per thread) equal to lane k's expert.
__device__ __forceinline__ void count_matches(const int64_t (&v)[kCountBatch], int64_t ek, int K,
                                              int32_t (&cnt)[kMaxTopk]) {
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        if (k < K) {
            const int64_t e = __builtin_amdgcn_readlane((int)ek, k);
#pragma unroll
            for (int b = 0; b < kCountBatch; ++b) cnt[k] += __popcll(__ballot(v[b] == e && e >= 0));
        }
    }
}

__global__ __launch_bounds__(kThreads) void ll_dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx, int T, int K, int H8,
    int E, int cap, int slices, u32x4* __restrict__ recv_x, int32_t* __restrict__ recv_count,
    int32_t* __restrict__ src_idx, int32_t* __restrict__ slot_of) {
    __shared__ int32_t wave_cnt[kWaves][kMaxTopk];
    __shared__ int32_t hist[kMaxExperts];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    if ((int)blockIdx.x == T * slices) {  // counts: a histogram of every valid entry
        for (int e = tid; e < E; e += kThreads) hist[e] = 0;
        __syncthreads();
        for (int i = tid; i < T * K; i += kThreads) {
            const int64_t e = topk_idx[i];
            if (e >= 0 && e < E) atomicAdd(&hist[(int)e], 1);
        }
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) recv_count[e] = hist[e];
        return;
    }
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    // This slice's chunk range of x[t].
    const int c0 = (int)((int64_t)H8 * slice / slices);
    const int c1 = (int)((int64_t)H8 * (slice + 1) / slices);
    const u32x4* src = x + (int64_t)t * H8;

    // Lane k < K: the token's k-th entry as loaded (validity is applied after
    // every load below is issued, so that nothing waits for it before then).
    int64_t e_raw = -1;
    if (lane < K) e_raw = topk_idx[(int64_t)t * K + lane];
    // Slot of (t, k) = earlier (token, slot) entries naming the same expert:
    // each pass loads kCountBatch entries per thread, then one ballot per
    // (entry, k) counts the matches of 64 entries at once.
    const int n_before = t * K;
    int64_t v[kCountBatch];
#pragma unroll
    for (int b = 0; b < kCountBatch; ++b) {
        const int i = b * kThreads + tid;
        v[b] = i < n_before ? topk_idx[i] : -2;
    }
    // The first chunk of this thread's part of the row goes out after the first
    // pass's entries, as a streaming buffer load (no branch; nothing past c1 or
    // without recv_x is read), so that its latency overlaps the counting and
    // the counting waits for its own loads only.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(src + c0), (short)0, recv_x != nullptr ? (c1 - c0) * 16 : 0,
        0x00020000);
    const u32x4 first = __builtin_amdgcn_raw_buffer_load_b128(xr, tid * 16, 0, 2);
    __builtin_amdgcn_sched_barrier(0);  // keep every use of the loads above below it
    // Lane k holds the token's k-th expert (-1 when empty or out of range).
    const int64_t ek = (e_raw >= 0 && e_raw < E) ? e_raw : -1;
    int32_t cnt[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) cnt[k] = 0;
    // The first pass outside the loop: its waits then leave the row load out.
    count_matches(v, ek, K, cnt);
    for (int i0 = kThreads * kCountBatch; i0 < n_before; i0 += kThreads * kCountBatch) {
#pragma unroll
        for (int b = 0; b < kCountBatch; ++b) {
            const int i = i0 + b * kThreads + tid;
            v[b] = i < n_before ? topk_idx[i] : -2;
        }
        count_matches(v, ek, K, cnt);
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (k < K) wave_cnt[wave][k] = cnt[k];
    }
    __syncthreads();
    // lane k: the slot, or -1 when the entry is empty or past the capacity
    int slot = -1;
    if (lane < K) {
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += wave_cnt[w][lane];
        slot = (ek >= 0 && sum < cap) ? sum : -1;
    }
    if (slice == 0 && wave == 0 && lane < K) {
        slot_of[(int64_t)t * K + lane] = slot;
        if (slot >= 0) src_idx[ek * cap + slot] = t;
    }
    const uint64_t dests = __ballot(slot >= 0);
    // slot row of lane k, as a row index of recv_x [E * cap, H]
    const int row_l = slot >= 0 ? (int)ek * cap + slot : 0;

    // Rows: this slice's chunk range of x[t] to every chosen expert's slot
    // (none when the receive is deferred to ll_recv_kernel).
    if (recv_x == nullptr) return;
    for (int c = c0 + tid; c < c1; c += kThreads) {
        const u32x4 v = c == c0 + tid ? first : __builtin_nontemporal_load(src + c);
        uint64_t m = dests;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(row_l, k);
            __builtin_nontemporal_store(v, recv_x + row * H8 + c);
        }
    }
}

// The deferred receive of a low-latency dispatch: grid = T * slices; the
// token's rows go to the slots the dispatch recorded in slot_of.
__global__ __launch_bounds__(kThreads) void ll_recv_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const int32_t* __restrict__ slot_of, int K, int H8, int E, int cap, int slices,
    u32x4* __restrict__ recv_x) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    int row_l = -1;
    if (lane < K) {
        const int64_t e = topk_idx[(int64_t)t * K + lane];
        const int s = slot_of[(int64_t)t * K + lane];
        if (e >= 0 && e < E && s >= 0 && s < cap) row_l = (int)e * cap + s;
    }
    const uint64_t dests = __ballot(row_l >= 0);
    const int c0 = (int)((int64_t)H8 * slice / slices);
    const int c1 = (int)((int64_t)H8 * (slice + 1) / slices);
    const u32x4* src = x + (int64_t)t * H8;
    for (int c = c0 + (int)threadIdx.x; c < c1; c += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + c);
        uint64_t m = dests;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(row_l, k);
            __builtin_nontemporal_store(v, recv_x + row * H8 + c);
        }
    }
}

// grid = T * slices; each thread owns 16-byte chunks of one token's output and
// sums the token's slot rows in k order (fp32 fused multiply-adds from +0.0).
__global__ __launch_bounds__(kThreads) void ll_combine_kernel(
    const u32x4* __restrict__ y, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, const int32_t* __restrict__ slot_of, int K, int H8,
    int E, int cap, int slices, u32x4* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    // lane k: row index of slot k in y [E * cap, H], its weight, whether valid
    int row_l = 0;
    float w_l = 0.0f;
    bool ok = false;
    if (lane < K) {
        const int64_t e = topk_idx[(int64_t)t * K + lane];
        const int s = slot_of[(int64_t)t * K + lane];
        ok = e >= 0 && e < E && s >= 0 && s < cap;
        row_l = ok ? (int)e * cap + s : 0;
        w_l = topk_weights[(int64_t)t * K + lane];
    }
    const uint64_t valid = __ballot(ok);
    const int c0 = (int)((int64_t)H8 * slice / slices);
    const int c1 = (int)((int64_t)H8 * (slice + 1) / slices);
    for (int c = c0 + (int)threadIdx.x; c < c1; c += kThreads) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += kVisitBatch) {
            // every load of the pass is issued before the first FMA; a slot
            // that is empty (or past K) reads row 0 and adds nothing
            u32x4 v[kVisitBatch];
            float wt[kVisitBatch];
            bool use[kVisitBatch];
#pragma unroll
            for (int b = 0; b < kVisitBatch; ++b) {
                const int k = min(k0 + b, K - 1);
                use[b] = k0 + b < K && ((valid >> k) & 1);
                const int64_t row = __builtin_amdgcn_readlane(row_l, k);
                wt[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), k));
                v[b] = __builtin_nontemporal_load(y + row * H8 + c);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < kVisitBatch; ++b) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = __builtin_fmaf(wt[b], bf16_lo(v[b][j]), acc[2 * j]);
                    const float hi = __builtin_fmaf(wt[b], bf16_hi(v[b][j]), acc[2 * j + 1]);
                    acc[2 * j] = use[b] ? lo : acc[2 * j];
                    acc[2 * j + 1] = use[b] ? hi : acc[2 * j + 1];
                }
            }
        }
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = bf16_bits(acc[2 * j]) | (bf16_bits(acc[2 * j + 1]) << 16);
        __builtin_nontemporal_store(o, out + (int64_t)t * H8 + c);
    }
}

__global__ __launch_bounds__(kThreads) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Enough workgroups per token that a small decode batch still spreads over
// the 256 compute units, and at least 64 chunks per workgroup.
int ll_slices(int T, int H8, int target_wg) {
    int s = 1;
    while (s < 16 && (int64_t)T * s < target_wg && H8 / (s * 2) >= MOEDX_LL_MIN_CHUNKS) s *= 2;
    return s;
}

}  // namespace

hipError_t launch_ll_dispatch(const void* x, const int64_t* topk_idx, int T, int K, int H, int E,
                              int cap, void* recv_x, int32_t* recv_count, int32_t* src_idx,
                              int32_t* slot_of, const Launch& L) {
    if (T == 0) {  // no token: every count is zero
        return launch_kernel(zero_i32_kernel, dim3((E + kThreads - 1) / kThreads), dim3(kThreads),
                             L,
                             recv_count, E);
    }
    const int H8 = H / 8;
    const int slices = ll_slices(T, H8, MOEDX_LL_TARGET_WG);
    return launch_kernel(ll_dispatch_kernel, dim3(T * slices + 1), dim3(kThreads), L,
                         static_cast<const u32x4*>(x), topk_idx, T, K, H8, E, cap, slices,
                         static_cast<u32x4*>(recv_x), recv_count, src_idx, slot_of);
}

hipError_t launch_ll_recv(const void* x, const int64_t* topk_idx, const int32_t* slot_of, int T,
                          int K, int H, int E, int cap, void* recv_x, const Launch& L) {
    const int H8 = H / 8;
    const int slices = ll_slices(T, H8, MOEDX_LL_COMBINE_TARGET_WG);
    return launch_kernel(ll_recv_kernel, dim3(T * slices), dim3(kThreads), L,
                         static_cast<const u32x4*>(x), topk_idx, slot_of, K, H8, E, cap, slices,
                         static_cast<u32x4*>(recv_x));
}

hipError_t launch_ll_combine(const void* y, const int64_t* topk_idx, const float* topk_weights,
                             const int32_t* slot_of, int T, int K, int H, int E, int cap, void* out,
                             const Launch& L) {
    const int H8 = H / 8;
    const int slices = ll_slices(T, H8, MOEDX_LL_COMBINE_TARGET_WG);
    return launch_kernel(ll_combine_kernel, dim3(T * slices), dim3(kThreads), L,
                         static_cast<const u32x4*>(y), topk_idx, topk_weights, slot_of, K, H8, E,
                         cap, slices, static_cast<u32x4*>(out));
}

}  // namespace moedx
