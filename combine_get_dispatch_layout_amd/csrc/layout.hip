// Dispatch layout kernel for gfx950 (wave64): one launch computes the layout
// and every prefix the receive side needs.
//
// The layout is what get_dispatch_layout returns in the normal-kernel example
// of the EnflameTechnology/DeepEP README: tokens per bucket, tokens per expert
// and the token-by-bucket mask.  For a handle it also yields the fields listed
// under "What the Handle Contains" on the handle-reuse page that do not depend
// on the row data: rank_prefix_matrix, channel_prefix_matrix and
// recv_channel_prefix_matrix, all on the device (no host prefix sum).
//
// Each workgroup takes a tile of 256 tokens, one per lane.  Bucket membership
// of a wave's 64 tokens (a "group") is one 64-bit ballot per bucket, so group
// counts, and the counts from a group's start to any channel boundary inside
// it, are popcounts of registers the wave already holds; expert counts go
// through an LDS histogram.  The last workgroup to finish (an atomic ticket;
// no workgroup ever waits on another) turns the group counts into exclusive
// per-bucket prefixes with wave shuffles, and derives the bucket totals and
// offsets, the expert totals and the channel prefixes.  A receive position is
// then base[r] + group_prefix[g][r] + a popcount inside the group, which the
// pack and combine kernels evaluate for themselves.  Every value is a pure
// function of the routing; no atomic decides an order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

namespace {

constexpr int kWaves = kTile / 64;
constexpr int kPerThread = 16;  // groups per finishing thread per pass
constexpr int kBatch = 16;      // loads issued together for the expert totals
constexpr int kLdsGroups = 8192;  // LDS slots for group prefixes (32 KB)
constexpr int kLdsChan = 2048;    // LDS slots for channel-boundary partials (8 KB)

// Channel c starts at token b_c = min(c * per, T), c = 0..C (b_C = T).
__device__ __forceinline__ int64_t boundary(int c, int per, int T) {
    const int64_t b = (int64_t)c * per;
    return b < T ? b : T;
}

__global__ __launch_bounds__(kTile) void layout_kernel(LayoutArgs a) {
    __shared__ int32_t hist[kMaxExperts];
    __shared__ int32_t s_gp[kLdsGroups];   // group prefixes, when ng * R fits
    __shared__ int32_t s_chan[kLdsChan];   // channel-boundary partials, when (C+1) * R fits
    __shared__ int32_t s_total[kMaxRanks];
    __shared__ int32_t s_base[kMaxRanks];
    __shared__ unsigned int s_ticket;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int T = a.T, K = a.K, E = a.E, R = a.R;
    const bool with_channels = a.channel_prefix_matrix != nullptr;

    // ---- phase 1: this tile's tokens ----------------------------------------
    // The small partials the finishing workgroup reads are stored first and
    // published (fence + ticket) before the large per-token outputs, so the
    // fence only waits for them.
    const int t = blockIdx.x * kTile + tid;
    uint64_t mask = 0;
    int64_t ids[kMaxTopk];
    if (T > 0) {
        for (int e = tid; e < E; e += kTile) hist[e] = 0;
        __syncthreads();
        if (t < T) {
            const int64_t* row = a.topk_idx + (int64_t)t * K;
#pragma unroll
            for (int k = 0; k < kMaxTopk; ++k) ids[k] = (k < K) ? row[k] : -1;
#pragma unroll
            for (int k = 0; k < kMaxTopk; ++k) {
                if (k >= K) break;
                const int64_t e = ids[k];
                if (e >= 0 && e < E) {  // ids outside [0, E) are treated as empty slots
                    mask |= 1ull << a.bucket.of((int)e);
                    atomicAdd(&hist[(int)e], 1);
                }
            }
        }
        // Group (one wave = 64 tokens) counts of every bucket; lane r keeps bucket r.
        const int g = blockIdx.x * kWaves + wave;
        const int g_begin = g * kGroup;
        if (g_begin < T) {
            int32_t my_cnt = 0;
            for (int r = 0; r < R; ++r) {
                const int c = __popcll(__ballot((mask >> r) & 1u));
                if (lane == r) my_cnt = c;
            }
            if (lane < R) a.group_cnt[(int64_t)g * R + lane] = my_cnt;
            // Channel boundaries inside this group: count from the group start.
            if (with_channels) {
                int c = (int)((g_begin + a.per - 1) / a.per);
                for (; c <= a.C; ++c) {
                    const int64_t b = boundary(c, a.per, T);
                    if (b >= T || b >= g_begin + kGroup) break;
                    const int off = (int)(b - g_begin);
                    const uint64_t below = off == 0 ? 0ull : (~0ull >> (64 - off));
                    int32_t part = 0;
                    for (int r = 0; r < R; ++r) {
                        const int n = __popcll(__ballot((mask >> r) & 1u) & below);
                        if (lane == r) part = n;
                    }
                    if (lane < R) a.chan_part[(int64_t)c * R + lane] = part;
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += kTile) a.tile_expert[(int64_t)blockIdx.x * E + e] = hist[e];
    }

    // ---- phase 2: publish the partials; the last workgroup finishes the job ----
    // Release at device scope: the partials are visible to every XCD's L2
    // before the ticket moves.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) s_ticket = atomicAdd(a.ticket, 1u);

    // The per-token outputs (not read by the finishing step).
    if (t < T) {
        uint8_t* out = a.is_token_in_rank + (int64_t)t * R;
        if ((R & 3) == 0) {
            for (int r = 0; r < R; r += 4)
                *reinterpret_cast<uint32_t*>(out + r) =
                    (uint32_t)((mask >> r) & 1u) | ((uint32_t)((mask >> (r + 1)) & 1u) << 8) |
                    ((uint32_t)((mask >> (r + 2)) & 1u) << 16) |
                    ((uint32_t)((mask >> (r + 3)) & 1u) << 24);
        } else {
            for (int r = 0; r < R; ++r) out[r] = (uint8_t)((mask >> r) & 1u);
        }
        if (a.token_mask) a.token_mask[t] = mask;
        if (a.slot_bucket) {
#pragma unroll
            for (int k = 0; k < kMaxTopk; ++k) {
                if (k >= K) break;
                const int64_t e = ids[k];
                a.slot_bucket[(int64_t)t * K + k] =
                    (e >= 0 && e < E) ? (int8_t)a.bucket.of((int)e) : (int8_t)-1;
            }
        }
    }
    __syncthreads();
    if (s_ticket != gridDim.x - 1) return;
    // Acquire: drop stale lines before reading the other workgroups' partials.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    const int ng = num_groups(T);
    const int nt = T > 0 ? (int)gridDim.x : 0;

    // Expert totals: issue these loads first; they overlap the group scan.
    const int per_e = E >= kTile ? 1 : kTile / E;
    int32_t esum[kMaxExperts / kTile];  // one partial per expert this thread sums
#pragma unroll
    for (int q = 0; q < kMaxExperts / kTile; ++q) {
        esum[q] = 0;
        const int i = tid + q * kTile;
        if (i >= E * per_e) continue;
        const int e = i % E, part = i / E;
        for (int j = part; j < nt; j += per_e * kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int jj = j + u * per_e;
                v[u] = jj < nt ? a.tile_expert[(int64_t)jj * E + e] : 0;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) esum[q] += v[u];
        }
    }

    // Channel-boundary partial counts (written in phase 1) staged in LDS.
    const int nb = with_channels ? (a.C + 1) * R : 0;
    const bool cp_in_lds = nb <= kLdsChan;
    if (cp_in_lds)
        for (int i = tid; i < nb; i += kTile) s_chan[i] = a.chan_part[i];

    // Exclusive prefix over groups per bucket.  Bucket r owns L consecutive
    // lanes of one wave (L a power of two, L * R <= 256); each lane takes G
    // consecutive groups per pass and the L lanes combine their sums with a
    // shuffle scan.  Prefixes also go to LDS when they fit, for the channel step.
    int L = 64;
    while (L * R > kTile) L >>= 1;
    int G = (ng + L - 1) / L;
    if (G > kPerThread) G = kPerThread;
    if (G < 1) G = 1;
    const bool gp_in_lds = ng * R <= kLdsGroups;
    const bool scan_thread = tid < L * R;
    const int sr = tid / L, sj = tid % L;
    int32_t carry = 0;
    if (scan_thread) {
        for (int pass = 0; pass < ng; pass += L * G) {
            const int g0 = pass + sj * G;
            int32_t v[kPerThread];
#pragma unroll
            for (int u = 0; u < kPerThread; ++u)
                v[u] = (u < G && g0 + u < ng) ? a.group_cnt[(int64_t)(g0 + u) * R + sr] : 0;
            int32_t mine = 0;
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) mine += v[u];
            int32_t incl = mine;
            for (int d = 1; d < L; d <<= 1) {
                const int32_t n = __shfl_up(incl, d, L);
                if (sj >= d) incl += n;
            }
            int32_t run = carry + incl - mine;
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) {
                const int gg = g0 + u;
                if (u < G && gg < ng) {
                    if (a.group_prefix) a.group_prefix[(int64_t)gg * R + sr] = run;
                    if (gp_in_lds) s_gp[gg * R + sr] = run;
                }
                run += v[u];
            }
            carry += __shfl(incl, L - 1, L);
        }
        if (sj == 0) s_total[sr] = carry;
    }
    // Expert partials meet in LDS.
    for (int e = tid; e < E; e += kTile) hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxExperts / kTile; ++q) {
        const int i = tid + q * kTile;
        if (i < E * per_e) {
            if (per_e == 1) hist[i] = esum[q];
            else atomicAdd(&hist[i % E], esum[q]);
        }
    }
    if (tid == 0) {
        int32_t run = 0;
        for (int r = 0; r < R; ++r) {
            s_base[r] = run;
            run += s_total[r];
        }
    }
    __syncthreads();
    if (tid < R) {
        a.num_tokens_per_rank[tid] = s_total[tid];
        if (a.rank_prefix_matrix) a.rank_prefix_matrix[tid] = s_base[tid] + s_total[tid];
        if (a.num_recv && tid == R - 1) *a.num_recv = s_base[tid] + s_total[tid];
    }
    for (int e = tid; e < E; e += kTile) a.num_tokens_per_expert[e] = hist[e];
    // Channel prefixes, one (boundary, bucket) pair per thread:
    // excl(b, r) = group_prefix[b / 64][r] + (count from the group start to b).
    for (int i = tid; i < nb; i += kTile) {
        const int c = i / R, r = i % R;
        const int64_t b = boundary(c, a.per, T);
        int32_t val;
        if (b >= T) {
            val = s_total[r];
        } else {
            const int g = (int)(b / kGroup);
            const int32_t gp = gp_in_lds ? s_gp[g * R + r] : a.group_prefix[(int64_t)g * R + r];
            val = gp + (cp_in_lds ? s_chan[i] : a.chan_part[i]);
        }
        if (c < a.C) a.recv_channel_prefix_matrix[r * a.C + c] = val;
        if (c > 0) a.channel_prefix_matrix[r * a.C + c - 1] = val;
    }
    if (tid == 0) atomicExch(a.ticket, 0u);
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

hipError_t launch_layout(const LayoutArgs& a, const Launch& L) {
    const int nt = num_tiles(a.T);
    return launch_kernel(layout_kernel, dim3(nt > 0 ? nt : 1), dim3(kTile), L, a);
}

}  // namespace moedx
