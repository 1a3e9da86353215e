// Internal launchers of the gfx950 kernels (host functions; not exported).
// Each launcher enqueues exactly one kernel on L.stream and returns the HIP
// status of the launch.  Shapes have been validated by the C-ABI layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "fastdiv.h"

namespace moedx {

#ifndef MOEDX_LAYOUT_TILE
#define MOEDX_LAYOUT_TILE 256
#endif
constexpr int kTile = MOEDX_LAYOUT_TILE;  // tokens per workgroup of the layout kernel
constexpr int kGroup = 64;         // tokens per receive-position group (one wavefront)
constexpr int kMaxRanks = 64;      // buckets fit one 64-bit mask
constexpr int kMaxExperts = 1024;  // LDS histogram bound
constexpr int kMaxTopk = 16;

__host__ __device__ inline int num_tiles(int T) { return (T + kTile - 1) / kTile; }
__host__ __device__ inline int num_groups(int T) { return (T + kGroup - 1) / kGroup; }

// ---- work order of the row kernels ------------------------------------------
// The pack and combine kernels run one wave per (token, slice of its row), 4
// waves per workgroup; wave index = token * waves_per_token + slice.  The
// packs take it in workgroup order; the combine takes its workgroups in short
// runs per XCD (xcd.h).  Long runs (a 64-token group, or a contiguous range,
// per XCD) were measured slower for both: they spread the rows in flight over
// more of HBM.
#ifndef MOEDX_ROW_WAVES_PER_BLOCK
#define MOEDX_ROW_WAVES_PER_BLOCK 4
#endif
constexpr int kRowWavesPerBlock = MOEDX_ROW_WAVES_PER_BLOCK;
constexpr int kRowThreads = kRowWavesPerBlock * 64;

inline int64_t row_blocks(int T, int waves_per_token) {
    return ((int64_t)T * waves_per_token + kRowWavesPerBlock - 1) / kRowWavesPerBlock;
}

// This wave's index (wave-uniform).
__device__ __forceinline__ int row_wave() {
    return __builtin_amdgcn_readfirstlane(blockIdx.x * kRowWavesPerBlock + (threadIdx.x >> 6));
}

// How a token's row is cut over waves: `split` waves per token; part p covers
// units [p * per, min((p + 1) * per, units)) with per = ceil(units / split).
struct RowSplit {
    FastDiv div;  // wave index / split
    int split;
    int per;
};

inline RowSplit make_row_split(int units, int split) {
    return RowSplit{make_fastdiv((uint32_t)split), split, (units + split - 1) / split};
}

// The wave's token and part (wave-uniform).
__device__ __forceinline__ void row_part(const RowSplit& rs, int* t, int* part) {
    const int w = row_wave();
    *t = (int)rs.div.div((uint32_t)w);
    *part = w - *t * rs.split;
}

// Where a launch goes and, optionally, events stamped with the kernel's own
// start and end (hipExtLaunchKernel), for kernel-accurate timing.  lds_bytes:
// dynamic LDS per workgroup (0 unless a launcher caps its occupancy).
struct Launch {
    hipStream_t stream;
    hipEvent_t start;
    hipEvent_t stop;
    unsigned int lds_bytes;
};

// Dynamic LDS (bytes) that, beside `static_lds` bytes of static LDS, lets at
// most `workgroups_per_cu` workgroups of a kernel share one CU (gfx950: 160 KB
// of LDS per CU, allocated in 512-byte granules).  A row kernel that reads a
// part of a row and writes it out runs faster on some shapes with fewer waves
// in flight per CU; its launcher reserves this much LDS, which the kernel does
// not touch.
unsigned int occupancy_lds(int workgroups_per_cu, unsigned int static_lds);

template <typename Tup, size_t... I>
inline void fill_args(void** argv, Tup& tup, std::index_sequence<I...>) {
    ((argv[I] = static_cast<void*>(&std::get<I>(tup))), ...);
}

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, const Launch& L,
                                Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> tup(static_cast<KArgs>(args)...);
    void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    fill_args(argv, tup, std::index_sequence_for<KArgs...>{});
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv,
                              L.lds_bytes, L.stream, L.start, L.stop, 0);
}

// ---- layout ------------------------------------------------------------------

// Everything the layout kernel reads and writes.  Pointers marked "handle" are
// null for the standalone get_dispatch_layout.
// Bucket of expert e, e / P, as (e * mul) >> shift: exact for every e in
// [0, E) (the host picks mul and shift and checks each e), and a multiply and a
// shift on the device instead of an integer division.
struct BucketDiv {
    uint32_t mul;
    uint32_t shift;
    __device__ __forceinline__ int of(int e) const { return (int)(((uint32_t)e * mul) >> shift); }
};

// mul == 0 when no such pair exists (not the case for E <= 1024).
BucketDiv bucket_div(int E, int P);

struct LayoutArgs {
    const int64_t* topk_idx;  // [T, K]
    int T, K, E, R, P, C, per;
    FastDiv per_div;  // n / per
    BucketDiv bucket;
    uint8_t* is_token_in_rank;             // [T, R]
    uint64_t* token_mask;                  // [T] bucket bit mask (handle)
    int8_t* slot_bucket;                   // [T, K] bucket of each slot or -1 (handle)
    int32_t* num_tokens_per_rank;          // [R]
    int32_t* num_tokens_per_expert;        // [E]
    int32_t* rank_prefix_matrix;           // [R] inclusive (handle)
    int32_t* num_recv;                     // [1] (handle)
    int32_t* group_prefix;                 // [ceil(T/64), R] exclusive, per bucket (handle)
    int32_t* channel_prefix_matrix;        // [R, C] inclusive (handle)
    int32_t* recv_channel_prefix_matrix;   // [R, C] exclusive (handle)
    int32_t* group_cnt;                    // scratch [ceil(T/64), R]
    int32_t* chan_part;                    // scratch [C + 1, R] (handle)
    int32_t* tile_expert;                  // scratch [ceil(T/256), E]; null when the expert
                                           // totals are given (experts_in)
    // A handle prepared from get_dispatch_layout's outputs: the bucket masks
    // come from is_token_in_rank [T, R] and the expert totals from
    // num_tokens_per_expert [E] instead of from topk_idx (null otherwise).
    const uint8_t* itr_in;
    const int32_t* experts_in;
    int32_t* experts_copy;  // get_dispatch_layout: a second copy of the expert totals (or null)
    unsigned int* ticket;                  // zero between launches; null for a launch that
                                           // takes no ticket (finishing step alone, first pack)
};

// With a.experts_in set (and a.itr_in, unless T == 0), the scan of a handle
// from given layout outputs: no expert histogram, masks from is_token_in_rank.
hipError_t launch_layout(const LayoutArgs& a, const Launch& L);

// The partials and per-token outputs of the layout only (handle arrays
// group_cnt, chan_part, tile_expert, is_token_in_rank, token_mask,
// slot_bucket); the prefixes, totals and N are left to a finishing step.
hipError_t launch_layout_partials(const LayoutArgs& a, const Launch& L);

// The finishing step alone (one workgroup) over partials a previous
// launch_layout_partials wrote.
hipError_t launch_layout_finish(const LayoutArgs& a, const Launch& L);

// get_dispatch_layout's outputs only (is_token_in_rank and the per-bucket and
// per-expert totals; a.token_mask / a.slot_bucket written when non-null):
// acc is E + R zeroed 64-bit accumulators, zero again when the launch ends.
hipError_t launch_layout_totals(const LayoutArgs& a, unsigned long long* acc, const Launch& L);

// Zero n 32-bit words with a kernel (capturable, unlike a memset node).
hipError_t launch_zero_words(uint32_t* p, int n, const Launch& L);

// ---- receive rows ------------------------------------------------------------

// row(t, r) = base[r] + group_prefix[t / 64][r] + (tokens of t's 64-token group
// before t that go to bucket r), base[r] = rank_prefix_matrix[r] - count[r].
struct RowMap {
    const uint64_t* token_mask;           // [T]
    const int32_t* group_prefix;          // [ceil(T/64), R]
    const int32_t* rank_prefix_matrix;    // [R]
    const int32_t* num_tokens_per_rank;   // [R]
    int R;
    int T;
    int64_t rows;  // rows of the receive buffer; a row at or past it is never touched
};

// First-dispatch outputs that complete the handle (null on a cached dispatch).
struct HandleRows {
    int32_t* send_head;     // [T, R]
    int32_t* recv_src_idx;  // [rows]
};

// Per-token handle arrays that a first pack writes when its handle borrowed
// the partials of a get_dispatch_layout left in a ctx's scratch (all null
// otherwise): each token's bucket mask and is_token_in_rank row, and its slot
// buckets copied from slot_bucket_src.
struct HandleTokens {
    uint64_t* token_mask;        // [T]
    uint8_t* is_token_in_rank;   // [T, R]
    int8_t* slot_bucket;         // [T, K]
    const int8_t* slot_bucket_src;
};

// First dispatch (bf16; launch_pack_fp8_first and launch_pack_bytes_first for
// FP8 and pre-quantised input) on a handle prepared
// with launch_layout_partials (or borrowing a layout's partials, ht), in one
// launch that also finishes the handle's prefixes; for T <= 4096, R a multiple
// of 4 up to 16 and (C + 1) * R <= 768 (pack_first_fits).  `la` carries every handle array
// (group_cnt, chan_part and token_mask being the partials read).
bool pack_first_fits(int T, int R, int E, int C);
hipError_t launch_pack_bf16_first(const LayoutArgs& la, const HandleTokens& ht, const void* x,
                                  int H, int64_t rows, const HandleRows& hr, void* recv_x,
                                  const float* topk_weights, int64_t* recv_topk_idx,
                                  float* recv_topk_weights, const Launch& L);

// Copy of borrowed layout partials into a handle's own arrays (and its
// is_token_in_rank rows from the token masks): what a scan of the layout's
// outputs would have written.
struct AdoptArgs {
    const uint64_t* mask_src;
    const int8_t* slot_bucket_src;
    const int32_t* group_cnt_src;
    const int32_t* chan_part_src;
    const int32_t* experts_src;
    uint64_t* token_mask;
    uint8_t* is_token_in_rank;
    int8_t* slot_bucket;
    int32_t* group_cnt;
    int32_t* chan_part;
    int32_t* num_tokens_per_expert;
    int T, K, R, E, n_group_cnt, n_chan_part;
};
hipError_t launch_adopt(const AdoptArgs& a, const Launch& L);

hipError_t launch_pack_bf16(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                            void* recv_x, const int64_t* topk_idx, const float* topk_weights,
                            int K, int E, int P, BucketDiv bucket, int64_t* recv_topk_idx,
                            float* recv_topk_weights, const Launch& L);

// The first FP8 dispatch on the same kind of handle as launch_pack_bf16_first
// (pack_first_fits), in one launch that also finishes its prefixes; mode and
// scales as launch_pack_fp8.
hipError_t launch_pack_fp8_first(const LayoutArgs& la, const HandleTokens& ht, const void* x,
                                 int H, int64_t rows, const HandleRows& hr, void* recv_x8,
                                 void* recv_scales, int mode, float tensor_scale, const Launch& L);

// mode: MOEDX_FP8_SCALE_* (AMAX 0, POW2 1, UE8M0 2, TENSOR 3); recv_scales fp32,
// uint8 (UE8M0) or unused (TENSOR).
hipError_t launch_pack_fp8(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                           void* recv_x8, void* recv_scales, int mode, float tensor_scale,
                           const Launch& L);

// The first pre-quantised dispatch on the same kind of handle as
// launch_pack_bf16_first, in one launch that also finishes its prefixes.
hipError_t launch_pack_bytes_first(const LayoutArgs& la, const HandleTokens& ht, const void* codes,
                                  const void* scales, int H, int scale_bytes, int64_t rows,
                                  const HandleRows& hr, void* recv_codes, void* recv_scales,
                                  const Launch& L);

// Pre-quantised rows: codes uint8 [T, H] and scale rows of scale_bytes bytes
// (scales may be NULL when scale_bytes == 0).
hipError_t launch_pack_bytes(const void* codes, const void* scales, int T, int H, int scale_bytes,
                             const RowMap& rm, const HandleRows& hr, void* recv_codes,
                             void* recv_scales, const Launch& L);

hipError_t launch_combine(const void* y, int T, int H, int K, const RowMap& rm,
                          const int8_t* slot_bucket, const float* gate_weights,
                          const float* recv_topk_weights, void* out,
                          float* combined_topk_weights, const Launch& L);

hipError_t launch_ll_dispatch(const void* x, const int64_t* topk_idx, int T, int K, int H, int E,
                              int cap, void* recv_x, int32_t* recv_count, int32_t* src_idx,
                              int32_t* slot_of, const Launch& L);

// The deferred receive (rows only) of a dispatch launched with recv_x NULL.
hipError_t launch_ll_recv(const void* x, const int64_t* topk_idx, const int32_t* slot_of, int T,
                          int K, int H, int E, int cap, void* recv_x, const Launch& L);

hipError_t launch_ll_combine(const void* y, const int64_t* topk_idx, const float* topk_weights,
                             const int32_t* slot_of, int T, int K, int H, int E, int cap, void* out,
                             const Launch& L);

}  // namespace moedx
