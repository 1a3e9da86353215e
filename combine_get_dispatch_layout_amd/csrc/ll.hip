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
// O(T*K) reads per workgroup, all from L2, and saves a separate count kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// grid = T * slices; workgroup b handles token b / slices, row slice b % slices.
__global__ __launch_bounds__(kThreads) void ll_dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx, int T, int K, int H8,
    int E, int cap, int slices, u32x4* __restrict__ recv_x, int32_t* __restrict__ recv_count,
    int32_t* __restrict__ src_idx, int32_t* __restrict__ slot_of) {
    __shared__ int32_t wave_cnt[kWaves][kMaxTopk];
    __shared__ int32_t s_slot[kMaxTopk];
    __shared__ int32_t s_expert[kMaxTopk];
    __shared__ int32_t hist[kMaxExperts];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;

    // This token's experts (uniform; invalid ids become -1).
    int64_t ek[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
        int64_t e = (k < K) ? topk_idx[(int64_t)t * K + k] : -1;
        ek[k] = (e >= 0 && e < E) ? e : -1;
    }
    // Count earlier (token, slot) entries naming each of those experts.
    int32_t cnt[kMaxTopk];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) cnt[k] = 0;
    const int n_before = t * K;
    for (int i0 = 0; i0 < n_before; i0 += kThreads) {
        const int i = i0 + tid;
        const int64_t v = (i < n_before) ? topk_idx[i] : -2;
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) {
            if (k < K) cnt[k] += __popcll(__ballot(v == ek[k] && ek[k] >= 0));
        }
    }
    if ((tid & 63) == 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (k < K) wave_cnt[wave][k] = cnt[k];
    }
    __syncthreads();
    if (tid < K) {
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += wave_cnt[w][tid];
        s_slot[tid] = s;
    }
    if (tid == 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k)
            if (k < K) s_expert[k] = (int32_t)ek[k];
    }
    __syncthreads();

    if (slice == 0 && tid < K) {
        const int e = s_expert[tid];
        const int s = s_slot[tid];
        const bool ok = e >= 0 && s < cap;
        slot_of[(int64_t)t * K + tid] = ok ? s : -1;
        if (ok) src_idx[(int64_t)e * cap + s] = t;
    }

    // Rows: this slice's chunk range of x[t] to every chosen expert's slot.
    const int c0 = (int)((int64_t)H8 * slice / slices);
    const int c1 = (int)((int64_t)H8 * (slice + 1) / slices);
    const u32x4* src = x + (int64_t)t * H8;
    for (int c = c0 + tid; c < c1; c += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + c);
        for (int k = 0; k < K; ++k) {
            const int e = s_expert[k];
            const int s = s_slot[k];
            if (e >= 0 && s < cap)
                __builtin_nontemporal_store(v, recv_x + ((int64_t)e * cap + s) * H8 + c);
        }
    }

    // The last token's first slice also writes every expert's count.
    if (t == T - 1 && slice == 0) {
        for (int e = tid; e < E; e += kThreads) hist[e] = 0;
        __syncthreads();
        for (int i = tid; i < T * K; i += kThreads) {
            const int64_t e = topk_idx[i];
            if (e >= 0 && e < E) atomicAdd(&hist[(int)e], 1);
        }
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) recv_count[e] = hist[e];
    }
}

// grid = T * slices; each thread owns 16-byte chunks of one token's output.
__global__ __launch_bounds__(kThreads) void ll_combine_kernel(
    const u32x4* __restrict__ y, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, const int32_t* __restrict__ slot_of, int T, int K,
    int H8, int E, int cap, int slices, u32x4* __restrict__ out) {
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    const int c0 = (int)((int64_t)H8 * slice / slices);
    const int c1 = (int)((int64_t)H8 * (slice + 1) / slices);
    for (int c = c0 + threadIdx.x; c < c1; c += kThreads) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int64_t e = topk_idx[(int64_t)t * K + k];
            const int s = slot_of[(int64_t)t * K + k];
            if (e < 0 || e >= E || s < 0 || s >= cap) continue;
            const float w = topk_weights[(int64_t)t * K + k];
            const u32x4 v = __builtin_nontemporal_load(y + (e * cap + s) * H8 + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] = __builtin_fmaf(w, bf16_lo(v[j]), acc[2 * j]);
                acc[2 * j + 1] = __builtin_fmaf(w, bf16_hi(v[j]), acc[2 * j + 1]);
            }
        }
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16_bits(acc[2 * j]) | (bf16_bits(acc[2 * j + 1]) << 16);
        __builtin_nontemporal_store(o, out + (int64_t)t * H8 + c);
    }
}

__global__ __launch_bounds__(kThreads) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Enough workgroups per token that a small decode batch still spreads over
// the 256 compute units, and at least 64 chunks per workgroup.
int ll_slices(int T, int H8) {
    int s = 1;
    while (s < 16 && (int64_t)T * s < 1024 && H8 / (s * 2) >= 64) s *= 2;
    return s;
}

}  // namespace

hipError_t launch_ll_dispatch(const void* x, const int64_t* topk_idx, int T, int K, int H, int E,
                              int cap, void* recv_x, int32_t* recv_count, int32_t* src_idx,
                              int32_t* slot_of, const Launch& L) {
    if (T == 0) {  // no token: every count is zero
        return launch_kernel(zero_i32_kernel, dim3((E + kThreads - 1) / kThreads), dim3(kThreads), L,
                             recv_count, E);
    }
    const int H8 = H / 8;
    const int slices = ll_slices(T, H8);
    return launch_kernel(ll_dispatch_kernel, dim3(T * slices), dim3(kThreads), L,
                         static_cast<const u32x4*>(x), topk_idx, T, K, H8, E, cap, slices,
                         static_cast<u32x4*>(recv_x), recv_count, src_idx, slot_of);
}

hipError_t launch_ll_combine(const void* y, const int64_t* topk_idx, const float* topk_weights,
                             const int32_t* slot_of, int T, int K, int H, int E, int cap, void* out,
                             const Launch& L) {
    const int H8 = H / 8;
    const int slices = ll_slices(T, H8);
    return launch_kernel(ll_combine_kernel, dim3(T * slices), dim3(kThreads), L,
                         static_cast<const u32x4*>(y), topk_idx, topk_weights, slot_of, T, K, H8,
                         E, cap, slices, static_cast<u32x4*>(out));
}

}  // namespace moedx
