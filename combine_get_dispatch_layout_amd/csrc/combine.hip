// Combine kernel for gfx950: the weighted gather-reduce of receive rows back
// to token order.
//
// combine_forward in the normal-kernel example of the EnflameTechnology/DeepEP
// README reduces the rows a token was sent to back into one row, and its
// dispatch_backward reduces the top-k weight payload the same way; the
// handle-reuse page ("Combining with Handle Reuse") runs it from the cached
// handle.  Here each token gathers the rows of its distinct buckets, in the
// order those buckets first occur among its top-k slots, scales each by the
// bucket's summed gate weight and accumulates in fp32 with fused multiply-adds
// from +0.0, then rounds once to bf16 (nearest even).
//
// Design (HBM-bound, no MFMA): one wavefront per (token, slice of 64 * CPL
// 16-byte chunks of its row); many small waves keep more gathers in flight than
// a few long ones (measured: a wave per token slice sustains ~10% more read
// bandwidth than a wave per token).  The wave locates the token's rows itself
// (rows.h); lanes 0..K-1 hold the slots, and first occurrence and the
// per-bucket weight come from lane reads, so every visited row, its weight and
// its address are wave-uniform.  The visit order is fixed, so the result does
// not depend on the launch shape.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "rows.h"

#ifndef MOEDX_COMBINE_CPL
#define MOEDX_COMBINE_CPL 2  // 16-byte chunks per lane; a wave covers 64 * CPL chunks
#endif
#ifndef MOEDX_COMBINE_VISIT_BATCH
#define MOEDX_COMBINE_VISIT_BATCH 4  // visited rows whose loads are issued together
#endif
#ifndef MOEDX_COMBINE_ROWS_FROM_SEND_HEAD
#define MOEDX_COMBINE_ROWS_FROM_SEND_HEAD 0  // rows from send_head instead of the token masks
#endif
#ifndef MOEDX_COMBINE_NT_LOAD
#define MOEDX_COMBINE_NT_LOAD 1
#endif
#ifndef MOEDX_COMBINE_NT_STORE
#define MOEDX_COMBINE_NT_STORE 1
#endif

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;
constexpr int kCPL = MOEDX_COMBINE_CPL;
constexpr int kVB = MOEDX_COMBINE_VISIT_BATCH;

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

__device__ __forceinline__ u32x4 load_row(const u32x4* p) {
#if MOEDX_COMBINE_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

__device__ __forceinline__ void store_row(u32x4 v, u32x4* p) {
#if MOEDX_COMBINE_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__global__ __launch_bounds__(256) void combine_kernel(
    const u32x4* __restrict__ y, int T, int H8, int K, RowMap rm,
    const int8_t* __restrict__ slot_bucket, const float* __restrict__ gate_weights,
    const float* __restrict__ recv_topk_weights, u32x4* __restrict__ out,
    float* __restrict__ combined_topk_weights, int slices, const int32_t* __restrict__ send_head) {
    constexpr int CPL = kCPL;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
    const int t = w / slices;
    const int part = w - t * slices;
    if (t >= T) return;
#if MOEDX_COMBINE_ROWS_FROM_SEND_HEAD
    TokenRows d;
    {
        int row = -1;
        if (lane < rm.R) {
            const int pos = send_head[(int64_t)t * rm.R + lane];
            const int64_t r64 = pos >= 0 ? (int64_t)rm.rank_prefix_matrix[lane] -
                                               rm.num_tokens_per_rank[lane] + pos
                                         : -1;
            row = r64 < rm.rows ? (int)r64 : -1;
        }
        d.row = row;
        d.dest = __ballot(row >= 0);
    }
#else
    const TokenRows d = token_rows(rm, t, lane);
#endif

    int rk = -1;
    float wk = 0.0f;
    if (lane < K) {
        rk = slot_bucket[(int64_t)t * K + lane];
        if (gate_weights) wk = gate_weights[(int64_t)t * K + lane];
    }
    // A slot is visited if it is the first slot of its bucket; its weight is the
    // sum, in ascending slot order from +0.0, of the gate weights of its bucket.
    bool first = rk >= 0;
    float om = 0.0f;
    for (int kk = 0; kk < K; ++kk) {
        const int r2 = __builtin_amdgcn_readlane(rk, kk);
        const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), kk));
        if (r2 == rk) {
            if (kk < lane) first = false;
            om = om + w2;
        }
    }
    if (!gate_weights) om = 1.0f;
    // lane k (a visited slot) holds the row of its bucket
    int vrow = -1;
    {
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int row_r = __builtin_amdgcn_readlane(d.row, r);
            if (first && rk == r) vrow = row_r;
        }
    }
    const uint64_t visits = __ballot(first && vrow >= 0);

    // This wave's chunks; lanes past the row end read a valid chunk and store nothing.
    const int c_begin = part * CPL * 64;
    const int c_end = min(c_begin + CPL * 64, H8);
    u32x4* dst = out + (int64_t)t * H8;
    int cs[CPL];
    bool act[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = c_begin + i * 64 + lane;
        act[i] = c < c_end;
        cs[i] = act[i] ? c : c_begin;
    }
    float acc[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    uint64_t m = visits;
    int k_last = visits ? __builtin_ctzll(visits) : 0;
    while (m) {
        // kVB visited rows per batch: every load is issued before the first FMA
        // (a batch past the last visit re-reads that visit's row and adds nothing).
        const u32x4* src[kVB];
        float wt[kVB];
        bool use[kVB];
#pragma unroll
        for (int b = 0; b < kVB; ++b) {
            use[b] = m != 0;
            if (use[b]) {
                k_last = __builtin_ctzll(m);
                m &= m - 1;
            }
            src[b] = y + (int64_t)__builtin_amdgcn_readlane(vrow, k_last) * H8;
            wt[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(om), k_last));
        }
        u32x4 v[kVB][CPL];
#pragma unroll
        for (int b = 0; b < kVB; ++b)
#pragma unroll
            for (int i = 0; i < CPL; ++i) v[b][i] = load_row(src[b] + cs[i]);
        __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its FMAs
        // Branch-free: an unused slot of the batch computes and discards its FMA,
        // so no control flow separates the loads from one another.
#pragma unroll
        for (int b = 0; b < kVB; ++b) {
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = __builtin_fmaf(wt[b], bf16_lo(v[b][i][j]), acc[i][2 * j]);
                    const float hi = __builtin_fmaf(wt[b], bf16_hi(v[b][i][j]), acc[i][2 * j + 1]);
                    acc[i][2 * j] = use[b] ? lo : acc[i][2 * j];
                    acc[i][2 * j + 1] = use[b] ? hi : acc[i][2 * j + 1];
                }
        }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (!act[i]) continue;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = bf16_bits(acc[i][2 * j]) | (bf16_bits(acc[i][2 * j + 1]) << 16);
        store_row(o, dst + cs[i]);
    }

    if (part == 0 && combined_topk_weights != nullptr && recv_topk_weights != nullptr &&
        lane < K) {
        float s = 0.0f;
        uint64_t m = visits;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t r = __builtin_amdgcn_readlane(vrow, k);
            s = s + recv_topk_weights[r * K + lane];
        }
        combined_topk_weights[(int64_t)t * K + lane] = s;
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int T, int H, int K, const RowMap& rm,
                          const int8_t* slot_bucket, const float* gate_weights,
                          const float* recv_topk_weights, void* out,
                          float* combined_topk_weights, const int32_t* send_head,
                          const Launch& L) {
    const int H8 = H / 8;
    const int slices = (H8 + kCPL * 64 - 1) / (kCPL * 64);
    const dim3 grid((int)(((int64_t)T * slices + kWavesPerBlock - 1) / kWavesPerBlock));
    return launch_kernel(combine_kernel, grid, dim3(256), L, static_cast<const u32x4*>(y), T, H8, K,
                         rm, slot_bucket, gate_weights, recv_topk_weights,
                         static_cast<u32x4*>(out), combined_topk_weights, slices, send_head);
}

}  // namespace moedx
