// Dispatch layout and scan kernels for gfx950 (wave64).
//
// The layout is what get_dispatch_layout returns in the normal-kernel example
// of the EnflameTechnology/DeepEP README: tokens per bucket, tokens per expert
// and the token-by-bucket mask.  The scan produces the handle fields listed
// under "What the Handle Contains" on the handle-reuse page (rank and channel
// prefix matrices, recv_src_idx, send_head), on the device, so that no host
// prefix sum is needed.
//
// Both kernels give one token to each lane and 256 tokens to a workgroup (a
// "tile").  Bucket membership of a wave's 64 tokens is a 64-bit ballot per
// bucket; popcounts give per-wave counts and mbcnt gives each lane's position,
// so every position is a pure function of the routing: no atomics decide an
// order, and the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

namespace {

constexpr int kWaves = kTile / 64;

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t count_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(kTile) void layout_tiles_kernel(
    const int64_t* __restrict__ topk_idx, int T, int K, int E, int R, int P,
    uint8_t* __restrict__ is_token_in_rank, int8_t* __restrict__ slot_bucket,
    int32_t* __restrict__ tile_rank, int32_t* __restrict__ tile_expert) {
    __shared__ int32_t hist[kMaxExperts];
    __shared__ int32_t wave_cnt[kWaves][kMaxRanks];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int t = blockIdx.x * kTile + tid;

    for (int e = tid; e < E; e += kTile) hist[e] = 0;
    __syncthreads();

    uint64_t mask = 0;
    if (t < T) {
        const int64_t* row = topk_idx + (int64_t)t * K;
        int64_t ids[kMaxTopk];
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) ids[k] = (k < K) ? row[k] : -1;
#pragma unroll
        for (int k = 0; k < kMaxTopk; ++k) {
            if (k >= K) break;
            const int64_t e = ids[k];
            int8_t b = -1;
            if (e >= 0 && e < E) {  // ids outside [0,E) are treated as empty slots
                const int r = (int)e / P;
                mask |= 1ull << r;
                atomicAdd(&hist[(int)e], 1);
                b = (int8_t)r;
            }
            if (slot_bucket) slot_bucket[(int64_t)t * K + k] = b;
        }
        uint8_t* out = is_token_in_rank + (int64_t)t * R;
        for (int r = 0; r < R; ++r) out[r] = (uint8_t)((mask >> r) & 1u);
    }

    for (int r = 0; r < R; ++r) {
        const uint64_t b = __ballot((mask >> r) & 1u);
        if ((tid & 63) == 0) wave_cnt[wave][r] = __popcll(b);
    }
    __syncthreads();
    if (tid < R) {
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += wave_cnt[w][tid];
        tile_rank[(int64_t)blockIdx.x * R + tid] = s;
    }
    for (int e = tid; e < E; e += kTile) tile_expert[(int64_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(kTile) void layout_reduce_kernel(
    const int32_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_expert, int ntiles,
    int R, int E, int32_t* __restrict__ num_tokens_per_rank,
    int32_t* __restrict__ num_tokens_per_expert) {
    const int i = blockIdx.x * kTile + threadIdx.x;
    if (i < R) {
        int32_t s = 0;
        for (int j = 0; j < ntiles; ++j) s += tile_rank[(int64_t)j * R + i];
        num_tokens_per_rank[i] = s;
    } else if (i < R + E) {
        const int e = i - R;
        int32_t s = 0;
        for (int j = 0; j < ntiles; ++j) s += tile_expert[(int64_t)j * E + e];
        num_tokens_per_expert[e] = s;
    }
}

// One workgroup per tile of 256 tokens (at least one workgroup, so that an
// empty batch still writes its zero counts and prefixes).
__global__ __launch_bounds__(kTile) void scan_kernel(
    const uint8_t* __restrict__ is_token_in_rank, int T, int R, int C, int per, int E, int ntiles,
    const int32_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_expert, ScanOut out) {
    __shared__ int32_t s_before[kMaxRanks];  // rows of bucket r owned by earlier tiles
    __shared__ int32_t s_total[kMaxRanks];   // rows of bucket r overall
    __shared__ int32_t s_base[kMaxRanks];    // first row of bucket r
    __shared__ int32_t wave_cnt[kWaves][kMaxRanks];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int tile = blockIdx.x;

    if (tid < R) {
        int32_t before = 0, total = 0;
        for (int j = 0; j < ntiles; ++j) {
            const int32_t v = tile_rank[(int64_t)j * R + tid];
            total += v;
            before += (j < tile) ? v : 0;
        }
        s_before[tid] = before;
        s_total[tid] = total;
    }
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0;
        for (int r = 0; r < R; ++r) {
            s_base[r] = run;
            run += s_total[r];
        }
    }
    __syncthreads();

    if (tile == 0 && tid < R) {
        out.num_tokens_per_rank[tid] = s_total[tid];
        out.rank_prefix_matrix[tid] = s_base[tid] + s_total[tid];
        if (tid == R - 1) *out.num_recv = s_base[tid] + s_total[tid];
    }
    for (int e = tile * kTile + tid; e < E; e += gridDim.x * kTile) {
        int32_t s = 0;
        for (int j = 0; j < ntiles; ++j) s += tile_expert[(int64_t)j * E + e];
        out.num_tokens_per_expert[e] = s;
    }
    if (T == 0) {
        for (int i = tid; i < R * C; i += kTile) {
            out.channel_prefix_matrix[i] = 0;
            out.recv_channel_prefix_matrix[i] = 0;
        }
        return;
    }

    const int t = tile * kTile + tid;
    uint64_t mask = 0;
    if (t < T) {
        const uint8_t* row = is_token_in_rank + (int64_t)t * R;
        for (int r = 0; r < R; ++r) mask |= (uint64_t)(row[r] != 0) << r;
    }
    // Pass 1: per-wave counts of every bucket.
    for (int r = 0; r < R; ++r) {
        const uint64_t b = __ballot((mask >> r) & 1u);
        if ((tid & 63) == 0) wave_cnt[wave][r] = __popcll(b);
    }
    __syncthreads();
    if (t >= T) return;

    const int c = t / per;
    const bool chan_start = (t == c * per);
    const int chan_end = min((c + 1) * per, T);
    const bool chan_last = (t == chan_end - 1);
    const bool last_token = (t == T - 1);
    int32_t* sh = out.send_head + (int64_t)t * R;

    // Pass 2: positions.  excl = tokens before t in bucket r.
    for (int r = 0; r < R; ++r) {
        const bool in = (mask >> r) & 1u;
        const uint64_t b = __ballot(in);
        int32_t excl = s_before[r] + (int32_t)count_below(b);
        for (int w = 0; w < wave; ++w) excl += wave_cnt[w][r];
        sh[r] = in ? excl : -1;
        if (in) out.recv_src_idx[s_base[r] + excl] = t;
        if (chan_start) out.recv_channel_prefix_matrix[r * C + c] = excl;
        if (chan_last) out.channel_prefix_matrix[r * C + c] = excl + (in ? 1 : 0);
        if (last_token) {
            for (int c2 = c + 1; c2 < C; ++c2) {  // empty trailing channels
                out.channel_prefix_matrix[r * C + c2] = s_total[r];
                out.recv_channel_prefix_matrix[r * C + c2] = s_total[r];
            }
        }
    }
}

}  // namespace

hipError_t launch_layout_tiles(const int64_t* topk_idx, int T, int K, int E, int R,
                               uint8_t* is_token_in_rank, int8_t* slot_bucket,
                               int32_t* tile_rank, int32_t* tile_expert, hipStream_t stream) {
    const int nt = num_tiles(T);
    if (nt == 0) return hipSuccess;
    layout_tiles_kernel<<<nt, kTile, 0, stream>>>(topk_idx, T, K, E, R, E / R, is_token_in_rank,
                                                  slot_bucket, tile_rank, tile_expert);
    return hipGetLastError();
}

hipError_t launch_layout_reduce(const int32_t* tile_rank, const int32_t* tile_expert, int ntiles,
                                int R, int E, int32_t* num_tokens_per_rank,
                                int32_t* num_tokens_per_expert, hipStream_t stream) {
    const int blocks = (R + E + kTile - 1) / kTile;
    layout_reduce_kernel<<<blocks, kTile, 0, stream>>>(tile_rank, tile_expert, ntiles, R, E,
                                                       num_tokens_per_rank,
                                                       num_tokens_per_expert);
    return hipGetLastError();
}

hipError_t launch_scan(const uint8_t* is_token_in_rank, int T, int R, int C, int E,
                       const int32_t* tile_rank, const int32_t* tile_expert, const ScanOut& out,
                       hipStream_t stream) {
    const int nt = num_tiles(T);
    const int per = T > 0 ? (T + C - 1) / C : 1;
    scan_kernel<<<nt > 0 ? nt : 1, kTile, 0, stream>>>(is_token_in_rank, T, R, C, per, E, nt,
                                                        tile_rank, tile_expert, out);
    return hipGetLastError();
}

}  // namespace moedx
