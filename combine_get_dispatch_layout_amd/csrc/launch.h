// Internal launchers of the gfx950 kernels (host functions; not exported).
// Each launcher enqueues one kernel on `stream` and returns the HIP status of
// the launch.  Shapes have been validated by the C-ABI layer before any call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moedx {

constexpr int kTile = 256;        // tokens per workgroup of the layout and scan kernels
constexpr int kMaxRanks = 64;     // buckets fit one 64-bit wavefront mask
constexpr int kMaxExperts = 1024; // LDS histogram bound
constexpr int kMaxTopk = 16;

inline int num_tiles(int T) { return (T + kTile - 1) / kTile; }

// Layout: per-token bucket mask, is_token_in_rank, bucket of each slot and
// per-tile counts (tile_rank [ntiles, R], tile_expert [ntiles, E]).
hipError_t launch_layout_tiles(const int64_t* topk_idx, int T, int K, int E, int R,
                               uint8_t* is_token_in_rank, int8_t* slot_bucket,
                               int32_t* tile_rank, int32_t* tile_expert, hipStream_t stream);

// Column sums of the per-tile counts: num_tokens_per_rank [R], num_tokens_per_expert [E].
hipError_t launch_layout_reduce(const int32_t* tile_rank, const int32_t* tile_expert, int ntiles,
                                int R, int E, int32_t* num_tokens_per_rank,
                                int32_t* num_tokens_per_expert, hipStream_t stream);

// Scan: counts, prefix matrices, send_head, recv_src_idx and N.
struct ScanOut {
    int32_t* num_tokens_per_rank;
    int32_t* num_tokens_per_expert;
    int32_t* rank_prefix_matrix;
    int32_t* num_recv;
    int32_t* channel_prefix_matrix;
    int32_t* recv_channel_prefix_matrix;
    int32_t* send_head;
    int32_t* recv_src_idx;
};
hipError_t launch_scan(const uint8_t* is_token_in_rank, int T, int R, int C, int E,
                       const int32_t* tile_rank, const int32_t* tile_expert, const ScanOut& out,
                       hipStream_t stream);

// Receive-row lookup shared by pack and combine: row(t,r) = base[r] + send_head[t,r],
// base[r] = rank_prefix_matrix[r] - num_tokens_per_rank[r].
struct RowMap {
    const int32_t* send_head;           // [T, R]
    const int32_t* rank_prefix_matrix;  // [R]
    const int32_t* num_tokens_per_rank; // [R]
    int R;
};

hipError_t launch_pack_bf16(const void* x, int T, int H, const RowMap& rm, void* recv_x,
                            const int64_t* topk_idx, const float* topk_weights, int K, int E, int P,
                            int64_t* recv_topk_idx, float* recv_topk_weights, hipStream_t stream);

hipError_t launch_pack_fp8(const void* x, int T, int H, const RowMap& rm, void* recv_x8,
                           float* recv_scales, hipStream_t stream);

hipError_t launch_combine(const void* y, int T, int H, int K, const RowMap& rm,
                          const int8_t* slot_bucket, const float* gate_weights,
                          const float* recv_topk_weights, void* out,
                          float* combined_topk_weights, hipStream_t stream);

hipError_t launch_ll_dispatch(const void* x, const int64_t* topk_idx, int T, int K, int H, int E,
                              int cap, void* recv_x, int32_t* recv_count, int32_t* src_idx,
                              int32_t* slot_of, hipStream_t stream);

hipError_t launch_ll_combine(const void* y, const int64_t* topk_idx, const float* topk_weights,
                             const int32_t* slot_of, int T, int K, int H, int E, int cap, void* out,
                             hipStream_t stream);

}  // namespace moedx
