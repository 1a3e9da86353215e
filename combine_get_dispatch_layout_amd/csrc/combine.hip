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
// (rows.h); lanes 0..K-1 hold the slots, and for each bucket of the token one
// ballot names its slots: the first is the visit, and the bucket's weight is
// the sum over them in ascending order, so every visited row, its weight and
// its address are wave-uniform.  Visits go in batches of 4, then 2, then 1,
// each batch's loads issued before its first FMA, so no row is read twice.
// The visit order is fixed, so the result does not depend on the launch
// shape.  The row addresses wait for the token's metadata loads, so the
// workgroups are ordered by xcd_run_block: each XCD takes runs of 16
// consecutive workgroups (about 4.6 tokens of a 7168-wide row), and a token's
// slot buckets, gate weights and group masks are mostly read from the L2 of
// the XCD that needs them.  Measured against the plain order (one process,
// interleaved repetitions): 4096 x 7168 combine 48.2 against 49.3 us, 16384 x
// 4096 140.2 against 144.1 us, the skewed 8192 x 7168 combine unchanged; the
// packs, whose row loads do not wait for their lookup, ran as fast or slower
// under every run length (the capped cached pack up to 11% slower).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "rows.h"
#include "xcd.h"

#ifndef MOEDX_COMBINE_CPL
#define MOEDX_COMBINE_CPL 1  // 16-byte chunks per lane; a wave covers 64 * CPL chunks
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

constexpr int kCPL = MOEDX_COMBINE_CPL;
constexpr int kCombineRunLog2 = 4;  // runs of 16 workgroups per XCD

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

// What locates one item's rows, loaded before they are needed: lane i holds
// the token mask of token (group start + i); lane r < R the group prefix of
// bucket r; lane k < K the bucket of slot k and its gate weight.
struct ItemLoads {
    uint64_t gm;
    int pfx;
    int rk;
    float wk;
};

__device__ __forceinline__ ItemLoads item_loads(const RowMap& rm, const int8_t* slot_bucket,
                                                const float* gate_weights, int K, int t,
                                                int lane) {
    ItemLoads a;
    const int tj = (t & ~63) + lane;
    a.gm = tj < rm.T ? rm.token_mask[tj] : 0ull;
    a.pfx = lane < rm.R ? rm.group_prefix[(int64_t)(t >> 6) * rm.R + lane] : 0;
    a.rk = lane < K ? (int)slot_bucket[(int64_t)t * K + lane] : -1;
    a.wk = (lane < K && gate_weights) ? gate_weights[(int64_t)t * K + lane] : 0.0f;
    return a;
}

// The token's visits: bucket r of the token is visited at its first slot k0
// (the visit order is ascending k0); lane k0 holds the bucket's row and its
// weight, the sum of the bucket's slot weights in ascending slot order from
// +0.0 (1 without gate weights).  Rows follow rows.h; a row outside the
// receive buffer (impossible for a consistent handle) is dropped.
struct Visits {
    uint64_t lanes;
    int row;
    float w;
};

__device__ __forceinline__ Visits item_visits(const ItemLoads& a, int base, int64_t rows, int t,
                                              int lane, bool weighted) {
    const int j = t & 63;
    const uint64_t mine = readlane64(a.gm, j);
    const uint64_t below = (j == 0) ? 0ull : (~0ull >> (64 - j));
    Visits v{0ull, -1, 0.0f};
    uint64_t m = mine;
    while (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
        const int pfx = __builtin_amdgcn_readlane(a.pfx, r);
        const int b = __builtin_amdgcn_readlane(base, r);
        const int64_t row = (int64_t)b + pfx + __popcll(__ballot((a.gm >> r) & 1u) & below);
        const uint64_t slots = __ballot(a.rk == r);
        if (slots == 0 || row < 0 || row >= rows) continue;
        float w = 0.0f;
        for (uint64_t s = slots; s; s &= s - 1)
            w = w + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a.wk),
                                                             __builtin_ctzll(s)));
        const int k0 = __builtin_ctzll(slots);
        v.lanes |= 1ull << k0;
        if (lane == k0) {
            v.row = (int)row;
            v.w = weighted ? w : 1.0f;
        }
    }
    return v;
}

// The next NB visits of *m (in order): their rows' loads are all issued,
// then the FMAs run in visit order; the visits are taken off *m.
template <int NB, int CPL>
__device__ __forceinline__ void visit_batch(const u32x4* __restrict__ y, int H8, const int* cs,
                                            const Visits& vs, uint64_t* m, float (*acc)[8]) {
    const u32x4* src[NB];
    float wt[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int k = __builtin_ctzll(*m);
        *m &= *m - 1;
        src[b] = y + (int64_t)__builtin_amdgcn_readlane(vs.row, k) * H8;
        wt[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vs.w), k));
    }
    u32x4 v[NB][CPL];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < CPL; ++i) v[b][i] = load_row(src[b] + cs[i]);
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its FMAs
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[i][2 * j] = __builtin_fmaf(wt[b], bf16_lo(v[b][i][j]), acc[i][2 * j]);
                acc[i][2 * j + 1] = __builtin_fmaf(wt[b], bf16_hi(v[b][i][j]), acc[i][2 * j + 1]);
            }
}

// One wave per (token, slice of 64 * CPL chunks of its row).
__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const u32x4* __restrict__ y, int T, int H8, int K, RowMap rm,
    const int8_t* __restrict__ slot_bucket, const float* __restrict__ gate_weights,
    const float* __restrict__ recv_topk_weights, u32x4* __restrict__ out,
    float* __restrict__ combined_topk_weights, RowSplit rs) {
    constexpr int CPL = kCPL;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(
        xcd_run_block<kCombineRunLog2>((int)blockIdx.x, (int)gridDim.x) * kRowWavesPerBlock +
        (int)(threadIdx.x >> 6));
    const int t = (int)rs.div.div((uint32_t)w);
    const int part = w - t * rs.split;
    if (t >= T) return;
    // Every lookup load goes out before the first wait: bucket r's base is
    // formed only after the item's loads are issued.
    int rp = 0, cnt = 0;
    if (lane < rm.R) {
        rp = rm.rank_prefix_matrix[lane];
        cnt = rm.num_tokens_per_rank[lane];
    }
    const ItemLoads ld = item_loads(rm, slot_bucket, gate_weights, K, t, lane);
    const Visits vs = item_visits(ld, rp - cnt, rm.rows, t, lane, gate_weights != nullptr);

    // This wave's chunks; lanes past the row end read a valid chunk and store nothing.
    const int c_begin = part * CPL * 64;
    const int c_end = min(c_begin + CPL * 64, H8);
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
    // Batches of 4 visits, then one of 2 and one of 1 as needed: every load of
    // a batch is issued before its first FMA and no row is read twice.
    uint64_t m = vs.lanes;
    while (__popcll(m) >= 4) visit_batch<4, CPL>(y, H8, cs, vs, &m, acc);
    if (__popcll(m) >= 2) visit_batch<2, CPL>(y, H8, cs, vs, &m, acc);
    if (m) visit_batch<1, CPL>(y, H8, cs, vs, &m, acc);
    u32x4* dst = out + (int64_t)t * H8;
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
        for (uint64_t mm = vs.lanes; mm; mm &= mm - 1) {
            const int64_t r = __builtin_amdgcn_readlane(vs.row, __builtin_ctzll(mm));
            s = s + recv_topk_weights[r * K + lane];
        }
        combined_topk_weights[(int64_t)t * K + lane] = s;
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int T, int H, int K, const RowMap& rm,
                          const int8_t* slot_bucket, const float* gate_weights,
                          const float* recv_topk_weights, void* out,
                          float* combined_topk_weights, const Launch& L) {
    const int H8 = H / 8;
    const int slices = (H8 + kCPL * 64 - 1) / (kCPL * 64);
    const int64_t blocks = row_blocks(T, slices);
    const u32x4* ys = static_cast<const u32x4*>(y);
    u32x4* os = static_cast<u32x4*>(out);
    return launch_kernel(combine_kernel, dim3((int)blocks), dim3(kRowThreads), L, ys, T, H8, K, rm,
                         slot_bucket, gate_weights, recv_topk_weights, os, combined_topk_weights,
                         make_row_split(H8, slices));
}

}  // namespace moedx
