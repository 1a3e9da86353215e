// Dispatch layout kernels for gfx950 (wave64); the two layout phases are in
// layout_core.h.
//   layout_kernel<false>: one launch computes the layout and every prefix.
//   layout_kernel<true>:  the partials and per-token outputs only, for a
//     capacity-mode handle whose first dispatch finishes it (no fence, ticket
//     or finishing step on this launch's path).
//   layout_finish_kernel: the finishing step alone, one workgroup, for a
//     handle whose first use is not a dispatch that finishes it itself.
// With kFromLayout the same launches scan a handle from get_dispatch_layout's
// outputs (is_token_in_rank, num_tokens_per_expert) instead of computing them:
// the dispatch of the normal-kernel example passes them in.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "layout_core.h"

namespace moedx {

namespace {

using FullLds = LayoutShared<8192, 2048>;  // 32 KB of group prefixes, 8 KB of channel partials

// kMaxR: 0 computes the layout from topk_idx; 8, 16 or 64 scans a handle from
// given layout outputs with up to that many buckets.
template <bool kPartialsOnly, int kMaxR>
__global__ __launch_bounds__(kTile) void layout_kernel(LayoutArgs a) {
    __shared__ FullLds s;
    TileToken tk;
    if (layout_tile<(kMaxR > 0), (kMaxR > 0 ? kMaxR : kMaxRanks)>(a, (int)blockIdx.x,
                                                                   (int)gridDim.x, s, &tk,
                                                                   kPartialsOnly)) {
        if (!layout_finish(a, (int)gridDim.x, s, &tk)) {
            const int t = (int)blockIdx.x * kTile + (int)threadIdx.x;
            if (t < a.T) layout_token_outputs(a, t, tk);
        }
    }
}

__global__ __launch_bounds__(kTile) void layout_finish_kernel(LayoutArgs a, int ntiles) {
    __shared__ FullLds s;
    layout_finish(a, ntiles, s, (const TileToken*)nullptr);
}

// get_dispatch_layout's outputs alone (the mask and the two count vectors):
// no prefix is needed, so the totals come from one round of counting atomics
// instead of partials, a fence, a ticket and a reload.  Each workgroup counts
// its 256 tokens per expert and per bucket in LDS and adds every count to a
// 64-bit accumulator as (1 << 32) + count, the high half counting arrivals;
// the workgroup whose add sees the last arrival holds the total, writes it
// and sets the accumulator back to zero for the next launch.  Every launch
// leaves the accumulators at zero; two launches on one accumulator array must
// not overlap.
struct TotalsLds {
    int32_t hist[kMaxExperts];
    int32_t bucket[kMaxRanks];
};

template <int NS>
__global__ __launch_bounds__(kTile) void layout_totals_kernel(LayoutArgs a,
                                                              unsigned long long* __restrict__ acc,
                                                              unsigned int ntiles) {
    __shared__ TotalsLds s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int T = a.T, K = a.K, E = a.E, R = a.R;
    const int t = (int)blockIdx.x * kTile + tid;
    for (int e = tid; e < E; e += kTile) s.hist[e] = 0;
    if (tid < R) s.bucket[tid] = 0;
    __syncthreads();
    TileToken tk;
    tk.mask = 0;
#pragma unroll
    for (int w = 0; w < kMaxTopk / 4; ++w) tk.sb[w] = 0xffffffffu;
    if (t < T) tk.mask = tile_slots<NS, true>(a, a.topk_idx + (int64_t)t * K, s, &tk);
    // tokens of this wave per bucket: lane r keeps bucket r's count
    int32_t cnt = 0;
    for (int r = 0; r < R; ++r) {
        const int c = __popcll(__ballot((tk.mask >> r) & 1u));
        cnt = lane == r ? c : cnt;
    }
    if (lane < R && cnt) atomicAdd(&s.bucket[lane], cnt);
    // With a ctx: the group and channel partials a handle scanned from these
    // outputs would hold, left in the ctx's scratch with the token masks and
    // slot buckets (layout_token_outputs), so that a dispatch prepared from
    // this layout can finish its handle in its first pack.
    if (a.group_cnt)
        group_partials(a, (int)blockIdx.x * kLayoutWaves + (tid >> 6), tk.mask, lane,
                       a.chan_part != nullptr);
    if (t < T) layout_token_outputs(a, t, tk);
    __syncthreads();
    const unsigned long long arrive = 1ull << 32;
    for (int i = tid; i < E + R; i += kTile) {
        const uint32_t v = (uint32_t)(i < E ? s.hist[i] : s.bucket[i - E]);
        const unsigned long long old = atomicAdd(acc + i, arrive | v);
        if ((unsigned int)(old >> 32) == ntiles - 1) {  // the last arrival: the total
            const int32_t total = (int32_t)((uint32_t)old + v);
            if (i < E) {
                a.num_tokens_per_expert[i] = total;
                if (a.experts_copy) a.experts_copy[i] = total;
            } else {
                a.num_tokens_per_rank[i - E] = total;
            }
            atomicExch(acc + i, 0ull);
        }
    }
}

// One thread per token copies its mask, is_token_in_rank row and slot
// buckets; the small partial arrays are copied by the first threads.
__global__ __launch_bounds__(kTile) void adopt_kernel(AdoptArgs a) {
    const int i = blockIdx.x * kTile + threadIdx.x;
    if (i < a.T) {
        const uint64_t m = a.mask_src[i];
        a.token_mask[i] = m;
        for (int r = 0; r < a.R; ++r)
            a.is_token_in_rank[(int64_t)i * a.R + r] = (uint8_t)((m >> r) & 1u);
        for (int k = 0; k < a.K; ++k)
            a.slot_bucket[(int64_t)i * a.K + k] = a.slot_bucket_src[(int64_t)i * a.K + k];
    }
    const int n = gridDim.x * kTile;
    for (int j = i; j < a.n_group_cnt; j += n) a.group_cnt[j] = a.group_cnt_src[j];
    for (int j = i; j < a.n_chan_part; j += n) a.chan_part[j] = a.chan_part_src[j];
    for (int j = i; j < a.E; j += n) a.num_tokens_per_expert[j] = a.experts_src[j];
}

__global__ __launch_bounds__(kTile) void zero_words_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * kTile + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

BucketDiv bucket_div(int E, int P) {
    // Smallest shift whose rounded-up reciprocal is exact on [0, E) and keeps
    // e * mul inside 32 bits.
    for (uint32_t shift = 0; shift < 32; ++shift) {
        const uint64_t mul = (((uint64_t)1 << shift) + (uint64_t)P - 1) / (uint64_t)P;
        if (mul * (uint64_t)E >= ((uint64_t)1 << 32)) break;
        bool exact = true;
        for (int e = 0; e < E && exact; ++e) exact = (int)(((uint64_t)e * mul) >> shift) == e / P;
        if (exact) return BucketDiv{(uint32_t)mul, shift};
    }
    return BucketDiv{0u, 0u};  // not reached for E <= 1024
}

namespace {

template <bool kPartialsOnly>
hipError_t launch_layout_kind(const LayoutArgs& a, const Launch& L) {
    const dim3 grid(num_tiles(a.T) > 0 ? num_tiles(a.T) : 1), block(kTile);
    if (a.experts_in == nullptr) return launch_kernel(layout_kernel<kPartialsOnly, 0>, grid, block, L, a);
    if (a.R <= 8) return launch_kernel(layout_kernel<kPartialsOnly, 8>, grid, block, L, a);
    if (a.R <= 16) return launch_kernel(layout_kernel<kPartialsOnly, 16>, grid, block, L, a);
    return launch_kernel(layout_kernel<kPartialsOnly, kMaxRanks>, grid, block, L, a);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, const Launch& L) {
    return launch_layout_kind<false>(a, L);
}

hipError_t launch_layout_partials(const LayoutArgs& a, const Launch& L) {
    return launch_layout_kind<true>(a, L);
}

hipError_t launch_layout_finish(const LayoutArgs& a, const Launch& L) {
    const int nt = num_tiles(a.T);
    return launch_kernel(layout_finish_kernel, dim3(1), dim3(kTile), L, a, nt > 0 ? nt : 1);
}

hipError_t launch_layout_totals(const LayoutArgs& a, unsigned long long* acc, const Launch& L) {
    const int nt = num_tiles(a.T) > 0 ? num_tiles(a.T) : 1;
    if (a.K <= kMaxTopk / 2)
        return launch_kernel(layout_totals_kernel<kMaxTopk / 2>, dim3(nt), dim3(kTile), L, a, acc,
                             (unsigned int)nt);
    return launch_kernel(layout_totals_kernel<kMaxTopk>, dim3(nt), dim3(kTile), L, a, acc,
                         (unsigned int)nt);
}

hipError_t launch_adopt(const AdoptArgs& a, const Launch& L) {
    const int nt = num_tiles(a.T) > 0 ? num_tiles(a.T) : 1;
    return launch_kernel(adopt_kernel, dim3(nt), dim3(kTile), L, a);
}

hipError_t launch_zero_words(uint32_t* p, int n, const Launch& L) {
    return launch_kernel(zero_words_kernel, dim3((n + kTile - 1) / kTile), dim3(kTile), L, p, n);
}

}  // namespace moedx
