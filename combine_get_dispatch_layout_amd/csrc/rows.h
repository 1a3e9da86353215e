// Receive-row lookup shared by the pack and combine kernels (device code).
//
// Rows are bucket-major and, inside a bucket, in ascending token order.  For
// token t in 64-token group g = t / 64 and bucket r:
//   row(t, r) = base[r] + group_prefix[g][r] + #{t' in group g, t' < t, bucket r},
// the last term being a popcount of one wavefront ballot over the group's
// token masks.  The whole wave evaluates it for one token; lane r ends up
// holding row(t, r) (or -1), and the token's bucket mask is wave-uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

struct TokenRows {
    int row;        // lane r: row(t, r), or -1 when t does not go to bucket r
    int pos;        // lane r: position of t inside bucket r (send_head), or -1
    uint64_t mask;  // buckets of t (wave-uniform)
    uint64_t dest;  // buckets whose row is valid (wave-uniform; mask, for a consistent handle)
};

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// The loads of a row lookup: the group's token masks and, on lanes r < R,
// what bucket r's base and group prefix are made of (nothing is computed from
// them here, so that no wait sits before the caller's next loads).
struct RowLoads {
    uint64_t gm;  // lane l: token_mask of token 64 g + l (0 past T)
    int rp;       // lane r < R: rank_prefix_matrix[r]
    int cnt;      // lane r < R: num_tokens_per_rank[r]
    int pfx;      // lane r < R: group_prefix[g][r]
};

// Issues the loads only (t wave-uniform, < rm.T); a kernel that issues its
// row loads after this call lets the lookup's wait skip them.
__device__ __forceinline__ RowLoads token_rows_load(const RowMap& rm, int t, int lane) {
    const int g = t >> 6;
    const int tj = (g << 6) + lane;
    RowLoads l;
    l.gm = tj < rm.T ? rm.token_mask[tj] : 0ull;
    l.rp = 0;
    l.cnt = 0;
    l.pfx = 0;
    if (lane < rm.R) {
        l.rp = rm.rank_prefix_matrix[lane];
        l.cnt = rm.num_tokens_per_rank[lane];
        l.pfx = rm.group_prefix[(int64_t)g * rm.R + lane];
    }
    return l;
}

__device__ __forceinline__ TokenRows token_rows_from(const RowMap& rm, const RowLoads& l, int t,
                                                     int lane) {
    const int j = t & 63;
    const uint64_t mine = readlane64(l.gm, j);
    const uint64_t below = (j == 0) ? 0ull : (~0ull >> (64 - j));
    int pos = -1;
    uint64_t m = mine;
    while (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
        const int c = __popcll(__ballot((l.gm >> r) & 1u) & below);
        if (lane == r) pos = l.pfx + c;
    }
    // A row past the receive buffer (impossible for a consistent handle) is
    // dropped rather than written: the kernels stay inside their buffers.
    const int64_t row64 = pos >= 0 ? (int64_t)(l.rp - l.cnt) + pos : -1;
    const int row = (row64 >= 0 && row64 < rm.rows) ? (int)row64 : -1;
    return TokenRows{row, pos, mine, __ballot(row >= 0)};
}

// t must be wave-uniform and < rm.T.
__device__ __forceinline__ TokenRows token_rows(const RowMap& rm, int t, int lane) {
    return token_rows_from(rm, token_rows_load(rm, t, lane), t, lane);
}

}  // namespace moedx
