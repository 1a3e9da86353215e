// The two phases of the dispatch layout as device functions (gfx950, wave64),
// shared by the layout kernels and the first-dispatch pack.
//
// The layout is what get_dispatch_layout returns in the normal-kernel example
// of the EnflameTechnology/DeepEP README: tokens per bucket, tokens per expert
// and the token-by-bucket mask.  For a handle it also yields the fields listed
// under "What the Handle Contains" on the handle-reuse page that do not depend
// on the row data: rank_prefix_matrix, channel_prefix_matrix and
// recv_channel_prefix_matrix, all on the device (no host prefix sum).
//
// Phase 1 (layout_tile): a workgroup takes a tile of 256 tokens, one per lane.
// Bucket membership of a wave's 64 tokens (a "group") gives group counts and
// the counts from a group's start to any channel boundary inside it; expert
// counts go through an LDS histogram.  The partials are published with a
// release fence and an atomic ticket; no workgroup ever waits on another.
// Phase 2 (layout_finish), run by the workgroup that takes the last ticket (or
// by a later launch): the group counts become exclusive per-bucket prefixes,
// and the bucket totals and offsets, expert totals and channel prefixes
// follow.  A receive position is then base[r] + group_prefix[g][r] + a
// popcount inside the group.  Every value is a pure function of the routing;
// no atomic decides an order.
//
// The layout is one chain of dependent steps (the topk loads, the partials'
// stores and fence, the ticket, the finishing workgroup's loads) run by
// workgroups that each have a SIMD to themselves, so its time is latency:
// loads are issued together before their first use, and the finishing step at
// the usual sizes is straight-line code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

constexpr int kLayoutWaves = kTile / 64;

// LDS of a workgroup that runs the layout phases.  gp holds the group
// prefixes (GP slots: the fast finishing step needs ng * R of them) and chan
// stages the channel-boundary partials of the general finishing step when
// they fit (CH slots).
template <int GP, int CH>
struct LayoutShared {
    int32_t hist[kMaxExperts];
    int32_t gp[GP];
    int32_t chan[CH > 0 ? CH : 1];
    int32_t total[kMaxRanks];
    int32_t base[kMaxRanks];
    unsigned int ticket;
    static constexpr int kGp = GP;
    static constexpr int kChan = CH;
};

// A raw buffer over n 32-bit words.  A buffer load checks its offset against
// the buffer's size in hardware and returns 0 past the end without touching
// memory, so a batch of such loads needs no branch and all of it can be in
// flight at once.  (The resource's last word is the
// gfx9-family raw-buffer format.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t word_buffer(const int32_t* p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p), (short)0, n * 4,
                                             0x00020000);
}
// Word i of a word_buffer; kNoWord (or any index past the end) reads 0.
constexpr unsigned int kNoWord = 0x20000000u;  // 2 GiB in: past every buffer here
__device__ __forceinline__ int32_t load_word(__amdgpu_buffer_rsrc_t r, unsigned int i) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)(i * 4u), 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// inside each row of 16 lanes, then the last lane of row 0 (row 2) is added to
// row 1 (row 3) and the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Channel c starts at token b_c = min(c * per, T), c = 0..C (b_C = T).
__device__ __forceinline__ int64_t layout_boundary(int c, int per, int T) {
    const int64_t b = (int64_t)c * per;
    return b < T ? b : T;
}

// What a tile's thread keeps of its token for the per-token outputs: the
// bucket mask and the bucket of every slot, four per word (0xFF: empty slot).
struct TileToken {
    uint64_t mask;
    uint32_t sb[kMaxTopk / 4];
};

// Per-token outputs of token t (t < T): is_token_in_rank, the token mask and
// the slot buckets.
__device__ __forceinline__ void layout_token_outputs(const LayoutArgs& a, int t,
                                                     const TileToken& tk) {
    const int R = a.R, K = a.K;
    const uint64_t mask = tk.mask;
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
        int8_t* sbo = a.slot_bucket + (int64_t)t * K;
        if ((K & 3) == 0) {  // t * K is a multiple of 4: whole words
#pragma unroll
            for (int w = 0; w < kMaxTopk / 4; ++w)
                if (4 * w < K) reinterpret_cast<uint32_t*>(sbo)[w] = tk.sb[w];
        } else {
#pragma unroll
            for (int k = 0; k < kMaxTopk; ++k)
                if (k < K) sbo[k] = (int8_t)(tk.sb[k >> 2] >> (8 * (k & 3)));
        }
    }
}

// The NS slots of one token (NS >= K, row = its topk_idx row): its bucket
// mask, its slot buckets in *tk and (kHist) its experts counted in the LDS
// histogram.  Slots past K re-read slot K - 1 and are ignored; ids outside
// [0, E) are empty slots.
template <int NS, bool kHist, typename Lds>
__device__ __forceinline__ uint64_t tile_slots(const LayoutArgs& a, const int64_t* row,
                                               Lds& s, TileToken* tk) {
    const int K = a.K, E = a.E;
    int64_t ids[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) ids[k] = row[k < K ? k : K - 1];
    uint64_t mask = 0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int64_t e = ids[k];
        const bool valid = k < K && e >= 0 && e < E;
        const int b = a.bucket.of(valid ? (int)e : 0);
        mask |= valid ? (1ull << b) : 0ull;
        tk->sb[k >> 2] ^= valid ? (uint32_t)(0xff ^ b) << (8 * (k & 3)) : 0u;
        if (kHist && valid) atomicAdd(&s.hist[(int)e], 1);
    }
    return mask;
}

// A token's is_token_in_rank row (bytes [row, row + R) of the buffer itr; a
// nonzero byte is a member), for R <= MR: the loads only, so that the slot
// loads can go out before anything waits for these.  32-bit words when R is a
// multiple of 4, else single bytes; loads past the row read past the buffer's
// end (0).
template <int MR>
struct ItrRow {
    uint32_t w[MR];  // words: w[0..MR/4); bytes: w[0..MR)
};

template <int MR>
__device__ __forceinline__ ItrRow<MR> itr_row_load(__amdgpu_buffer_rsrc_t itr, int row, int R) {
    ItrRow<MR> x;
    constexpr int kPast = (int)(kNoWord * 4u);
    if ((R & 3) == 0) {
#pragma unroll
        for (int q = 0; q < MR / 4; ++q)
            x.w[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(itr, 4 * q < R ? row + 4 * q : kPast,
                                                                    0, 0);
    } else {
#pragma unroll
        for (int r = 0; r < MR; ++r)
            x.w[r] = __builtin_amdgcn_raw_buffer_load_b8(itr, r < R ? row + r : kPast, 0, 0);
    }
    return x;
}

template <int MR>
__device__ __forceinline__ uint64_t itr_row_mask(const ItrRow<MR>& x, int R) {
    uint64_t m = 0;
    if ((R & 3) == 0) {
#pragma unroll
        for (int q = 0; q < MR / 4; ++q) {
            const uint32_t v = x.w[q];
            const uint64_t nib = (uint64_t)((v & 0xffu) != 0) | ((uint64_t)((v & 0xff00u) != 0) << 1) |
                                 ((uint64_t)((v & 0xff0000u) != 0) << 2) |
                                 ((uint64_t)((v & 0xff000000u) != 0) << 3);
            m |= nib << (4 * q);
        }
    } else {
#pragma unroll
        for (int r = 0; r < MR; ++r) m |= (uint64_t)(x.w[r] != 0) << r;
    }
    return m;
}

// The partials of group g (the 64 tokens of one wave; this lane's token has
// bucket mask `mask`): bucket counts over the group and, with channels, the
// counts from the group's start to every channel boundary inside it.  Eight
// buckets at a time: each token's bits for buckets j..j+7 are spread to one
// byte each (a count never exceeds 64, so bytes never carry) and one wave
// prefix sum per 32-bit half gives, at lane i, the counts over lanes 0..i of
// four buckets.  Lane 63 holds the group counts; the counts from the group
// start to a channel boundary at offset o are those of lane o - 1.  Lane r
// stores bucket r's values.  Wave-uniform g; every lane takes part.
__device__ __forceinline__ void group_partials(const LayoutArgs& a, int g, uint64_t mask, int lane,
                                               bool with_channels) {
    const int T = a.T, R = a.R;
    const int g_begin = g * kGroup;
    if (g_begin >= T) return;
    // First channel boundary at or after g_begin: ceil(g_begin / per).
    const int c_first =
        with_channels ? (int)a.per_div.div((uint32_t)(g_begin + a.per - 1)) : a.C + 1;
    for (int j = 0; j < R; j += 8) {
        const uint32_t bits = (uint32_t)(mask >> j) & 0xffu;
        const uint32_t lo = ((bits & 0xfu) * 0x00204081u) & 0x01010101u;
        const uint32_t hi = ((bits >> 4) * 0x00204081u) & 0x01010101u;
        const uint32_t slo = (uint32_t)wave_inclusive_sum((int32_t)lo);
        const uint32_t shi = (uint32_t)wave_inclusive_sum((int32_t)hi);
        const int rr = lane - j;  // this lane's bucket within the eight
        const bool mine = rr >= 0 && rr < 8 && lane < R;
        const int sh = 8 * (rr & 3);
        {
            const uint32_t w = rr < 4 ? __builtin_amdgcn_readlane(slo, 63)
                                      : __builtin_amdgcn_readlane(shi, 63);
            if (mine) a.group_cnt[(int64_t)g * R + lane] = (int32_t)((w >> sh) & 0xffu);
        }
        for (int c = c_first; c <= a.C; ++c) {
            const int64_t b = layout_boundary(c, a.per, T);
            if (b >= T || b >= g_begin + kGroup) break;
            const int off = (int)(b - g_begin);
            uint32_t w = 0;
            if (off > 0)
                w = rr < 4 ? __builtin_amdgcn_readlane(slo, off - 1)
                           : __builtin_amdgcn_readlane(shi, off - 1);
            if (mine) a.chan_part[(int64_t)c * R + lane] = (int32_t)((w >> sh) & 0xffu);
        }
    }
}

// Phase 1 for tile `tile` of `ntiles`.  Returns true in the workgroup that took
// the last ticket (workgroup-uniform), which must then run layout_finish and
// see that its own per-token outputs (*tk) are written; the other workgroups
// have written theirs when this returns.  With partials_only every workgroup
// stores its partials and per-token outputs and returns false: the finishing
// step runs in a later launch.  kFromLayout: the bucket masks come from the
// given is_token_in_rank (a.itr_in), topk_idx gives only the slot buckets, no
// expert is counted, and tile 0 copies the given expert totals (a.experts_in)
// into the handle.  kMaxR (kFromLayout): a bound on R that sizes the mask
// row's loads.
template <bool kFromLayout = false, int kMaxR = kMaxRanks, typename Lds>
__device__ __forceinline__ bool layout_tile(const LayoutArgs& a, int tile, int ntiles, Lds& s,
                                            TileToken* tk, bool partials_only = false) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int T = a.T, K = a.K, E = a.E, R = a.R;
    const bool with_channels = a.channel_prefix_matrix != nullptr;

    // The small partials the finishing workgroup reads are stored first and
    // published (fence + ticket) before the large per-token outputs, so the
    // fence only waits for them.
    const int t = tile * kTile + tid;
    uint64_t mask = 0;
    tk->mask = 0;
#pragma unroll
    for (int w = 0; w < kMaxTopk / 4; ++w) tk->sb[w] = 0xffffffffu;
    constexpr int kEq = kMaxExperts / kTile;
    int32_t ecopy[kEq];  // kFromLayout, tile 0: the given expert totals
    if (kFromLayout && tile == 0) {
#pragma unroll
        for (int q = 0; q < kEq; ++q)
            ecopy[q] = tid + q * kTile < E ? a.experts_in[tid + q * kTile] : 0;
    }
    if (T > 0) {
        if (!kFromLayout) {
            for (int e = tid; e < E; e += kTile) s.hist[e] = 0;
            __syncthreads();
        }
        if (t < T) {
            // Every slot load is issued before the first is used (one memory
            // round trip); slots past K re-read slot K - 1 and are ignored.
            const int64_t* row = a.topk_idx + (int64_t)t * K;
            if (kFromLayout) {
                // the mask row's loads, then the slots' (issued before either
                // is waited for), then the mask
                const __amdgpu_buffer_rsrc_t itr = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint8_t*>(a.itr_in), (short)0, T * R, 0x00020000);
                const ItrRow<kMaxR> given = itr_row_load<kMaxR>(itr, t * R, R);
                if (K <= kMaxTopk / 2)
                    (void)tile_slots<kMaxTopk / 2, false>(a, row, s, tk);
                else
                    (void)tile_slots<kMaxTopk, false>(a, row, s, tk);
                mask = itr_row_mask<kMaxR>(given, R);
            } else {
                if (K <= kMaxTopk / 2)
                    mask = tile_slots<kMaxTopk / 2, true>(a, row, s, tk);
                else
                    mask = tile_slots<kMaxTopk, true>(a, row, s, tk);
            }
            tk->mask = mask;
        }
        group_partials(a, tile * kLayoutWaves + wave, mask, lane, with_channels);
        if (!kFromLayout) {
            __syncthreads();
            for (int e = tid; e < E; e += kTile) a.tile_expert[(int64_t)tile * E + e] = s.hist[e];
        }
    }
    if (kFromLayout && tile == 0) {
#pragma unroll
        for (int q = 0; q < kEq; ++q)
            if (tid + q * kTile < E) a.num_tokens_per_expert[tid + q * kTile] = ecopy[q];
    }
    if (partials_only) {  // a later launch finishes (the kernel boundary publishes)
        if (t < T) layout_token_outputs(a, t, *tk);
        return false;
    }
    // Release at device scope: the partials are visible to every XCD's L2
    // before the ticket moves.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) s.ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const bool last = s.ticket == (unsigned int)(ntiles - 1);
    // The per-token outputs (not read by the finishing step).  The last
    // workgroup writes its own during or after its finish, so that its acquire
    // fence does not wait for these stores.
    if (!last && t < T) layout_token_outputs(a, t, *tk);
    return last;
}

// The fast finishing step keeps every load of its partials in registers:
// up to 4 buckets per wave (R <= 16) times 4 chunks of 64 groups (T <= 16384),
// up to 32 tiles per expert thread, three channel boundaries per thread; and
// its group prefixes in LDS (gp).
constexpr int kFastChunks = 4;
constexpr int kFastBuckets = 4;
constexpr int kFastTiles = 32;
constexpr int kFastBounds = 3;

__device__ __forceinline__ int layout_per_expert(int E) { return E >= kTile ? 1 : kTile / E; }

// kChunks (<= kFastChunks) and kTiles (<= kFastTiles) size the registers of
// one instantiation; a kernel that only meets small shapes passes smaller ones.
template <int kChunks = kFastChunks, int kTiles = kFastTiles>
__host__ __device__ inline bool layout_fast_finish_fits(int T, int R, int E, int C, int ntiles,
                                                        bool with_channels, int gp_slots) {
    const int nb = with_channels ? (C + 1) * R : 0;
    const int ng = num_groups(T);
    const int per_e = E >= kTile ? 1 : kTile / E;
    return T > 0 && ng <= kChunks * kGroup && R <= kFastBuckets * kLayoutWaves &&
           ng * R <= gp_slots && ntiles <= kTiles * per_e && nb <= kFastBounds * kTile;
}

// Phase 2 for the sizes layout_fast_finish_fits admits: every load is issued
// before the first is used (one memory round trip), and the scan is branch-free:
// wave w takes buckets w, w + 4, ..., lane g of chunk c holding group 64c + g,
// and one wave prefix sum per bucket and chunk (plus the running total of the
// chunks before) gives every group prefix and the bucket total.
template <int kChunks, int kTiles, typename Lds>
__device__ __forceinline__ void layout_finish_fast(const LayoutArgs& a, int ntiles, Lds& s,
                                                   const TileToken* tk) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, E = a.E, R = a.R;
    const int ng = num_groups(T);
    const int nch = (ng + kGroup - 1) / kGroup;
    const int nb = a.channel_prefix_matrix != nullptr ? (a.C + 1) * R : 0;
    // Expert partials: thread i < E * per_e sums tiles i / E, i / E + per_e, ...
    // of expert i % E (experts past 256 are summed after the fast part).  A
    // handle scanned from given layout outputs has its totals already.
    const bool experts = a.tile_expert != nullptr;
    const int per_e = layout_per_expert(E);
    const bool e_thread = experts && tid < E * per_e;
    const int e0 = tid % E;
    for (int e = tid; e < E; e += kTile) s.hist[e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // Indices first, then every load.
    const __amdgpu_buffer_rsrc_t gc = word_buffer(a.group_cnt, ng * R);
    const __amdgpu_buffer_rsrc_t te = word_buffer(a.tile_expert, experts ? ntiles * E : 0);
    const __amdgpu_buffer_rsrc_t cp = word_buffer(a.chan_part, nb);
    const unsigned int ebase = e_thread ? (unsigned int)((tid / E) * E + e0) : kNoWord;
    int32_t cnt[kFastBuckets][kChunks], ev[kTiles], cv[kFastBounds];
#pragma unroll
    for (int i = 0; i < kFastBuckets; ++i)
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {  // past R or ng: past the buffer's end
            const int r = wave + kLayoutWaves * i, gg = c * kGroup + lane;
            cnt[i][c] = load_word(gc, r < R && gg < ng ? (unsigned int)(gg * R + r) : kNoWord);
        }
#pragma unroll
    for (int u = 0; u < kTiles; ++u)  // tiles past ntiles lie past the buffer's end
        ev[u] = load_word(te, ebase + (unsigned int)(u * per_e * E));
#pragma unroll
    for (int q = 0; q < kFastBounds; ++q) cv[q] = load_word(cp, (unsigned int)(tid + q * kTile));
    // This workgroup's own per-token outputs, issued while the loads are in flight.
    if (tk) {
        const int t = (int)blockIdx.x * kTile + tid;
        if (t < T) layout_token_outputs(a, t, *tk);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Group prefixes and bucket totals.
#pragma unroll
    for (int i = 0; i < kFastBuckets; ++i) {
        const int r = wave + kLayoutWaves * i;
        if (r >= R) break;  // wave-uniform
        int32_t carry = 0;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (c >= nch) break;  // wave-uniform
            const int32_t incl = wave_inclusive_sum(cnt[i][c]);
            const int gg = c * kGroup + lane;
            if (gg < ng) {
                const int32_t excl = carry + incl - cnt[i][c];
                s.gp[gg * R + r] = excl;
                if (a.group_prefix) a.group_prefix[(int64_t)gg * R + r] = excl;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) s.total[r] = carry;
    }
    // Expert totals: the partial sums of each expert meet in LDS.
    int32_t esum = 0;
#pragma unroll
    for (int u = 0; u < kTiles; ++u) esum += ev[u];
    __syncthreads();  // hist cleared by every thread
    if (e_thread) atomicAdd(&s.hist[e0], esum);
    if (experts) {
        for (int e = tid + kTile; e < E; e += kTile) {  // E > 256
            int32_t v = 0;
            for (int j = 0; j < ntiles; ++j) v += a.tile_expert[(int64_t)j * E + e];
            s.hist[e] = v;
        }
    }
    __syncthreads();
    if (experts)
        for (int e = tid; e < E; e += kTile) a.num_tokens_per_expert[e] = s.hist[e];
    else if (a.experts_in)  // totals given with the partials: copied into the handle
        for (int e = tid; e < E; e += kTile) a.num_tokens_per_expert[e] = a.experts_in[e];
    // Bucket offsets: one wave prefix sum over the bucket totals.
    if (wave == 0) {
        const int32_t tot = lane < R ? s.total[lane] : 0;
        const int32_t incl = wave_inclusive_sum(tot);
        if (lane < R) {
            a.num_tokens_per_rank[lane] = tot;
            if (a.rank_prefix_matrix) a.rank_prefix_matrix[lane] = incl;
            if (a.num_recv && lane == R - 1) *a.num_recv = incl;
        }
    }
    // Channel prefixes: excl(b, r) = group prefix of b's group + count from the
    // group start to b (the bucket total for b = T).
#pragma unroll
    for (int q = 0; q < kFastBounds; ++q) {
        const int i = tid + q * kTile;
        if (i < nb) {
            const int c = i / R, r = i - (i / R) * R;
            const int64_t b = layout_boundary(c, a.per, T);
            const int32_t val = b >= T ? s.total[r] : s.gp[(int)(b / kGroup) * R + r] + cv[q];
            if (c < a.C) a.recv_channel_prefix_matrix[r * a.C + c] = val;
            if (c > 0) a.channel_prefix_matrix[r * a.C + c - 1] = val;
        }
    }
    if (tid == 0 && a.ticket) atomicExch(a.ticket, 0u);  // only a launch that took tickets
}

// Phase 2, in the workgroup that took the last ticket of `ntiles` tiles.
// Returns whether it has also written this workgroup's per-token outputs (tk;
// the fast step issues them while its loads are in flight).
template <typename Lds>
__device__ __forceinline__ bool layout_finish(const LayoutArgs& a, int ntiles, Lds& s,
                                              const TileToken* tk) {
    if (layout_fast_finish_fits(a.T, a.R, a.E, a.C, ntiles, a.channel_prefix_matrix != nullptr,
                                Lds::kGp)) {
        layout_finish_fast<kFastChunks, kFastTiles>(a, ntiles, s, tk);
        return tk != nullptr;
    }
    constexpr int kPerThread = 16;  // groups per finishing thread per pass
    constexpr int kBatch = 16;      // loads issued together for the expert totals
    const int tid = threadIdx.x;
    const int T = a.T, E = a.E, R = a.R;
    const bool with_channels = a.channel_prefix_matrix != nullptr;
    // Acquire: drop stale lines before reading the other workgroups' partials.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    const int ng = num_groups(T);
    const int nt = T > 0 ? ntiles : 0;

    // The first pass of every partial sum below loads its values before any
    // is used, so that at the usual sizes (at most 16 tiles, 1024 groups and
    // 256 channel boundaries) all of them take one memory round trip.  These
    // are buffer loads (word_buffer): out-of-range indices read 0, so none
    // waits behind a branch.  Every index is computed before the first load.
    // Expert totals: thread i < E * per_e sums the partials of expert i % E
    // from tiles i / E + u * per_e.
    const bool experts = a.tile_expert != nullptr;  // else the totals are given
    const int per_e = E >= kTile ? 1 : kTile / E;
    const bool e_thread = experts && tid < E * per_e;
    const int e0 = e_thread ? tid % E : 0, part0 = tid / E;
    const unsigned int ebase = e_thread ? (unsigned int)(part0 * E + e0) : kNoWord;
    // Channel-boundary partial counts (written in phase 1), staged in LDS.
    const int nb = with_channels ? (a.C + 1) * R : 0;
    const bool cp_in_lds = nb <= Lds::kChan;
    // Exclusive prefix over groups per bucket.  Bucket r owns L consecutive
    // lanes of one wave (L a power of two, L * R <= 256); each lane takes G
    // consecutive groups per pass and the L lanes combine their sums with a
    // shuffle scan.  Prefixes also go to LDS when they fit, for the channel step.
    int L = 64;
    while (L * R > kTile) L >>= 1;
    int G = (ng + L - 1) / L;
    if (G > kPerThread) G = kPerThread;
    if (G < 1) G = 1;
    const bool gp_in_lds = ng * R <= Lds::kGp;
    const bool scan_thread = tid < L * R;
    const int sr = tid / L, sj = tid % L;
    const unsigned int gbase = scan_thread ? (unsigned int)(sj * G * R + sr) : kNoWord;

    const __amdgpu_buffer_rsrc_t te = word_buffer(a.tile_expert, experts ? nt * E : 0);
    int32_t ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)  // tiles past nt lie past the buffer's end
        ev[u] = load_word(te, ebase + (unsigned int)(u * per_e * E));
    int32_t cv = 0;
    if (cp_in_lds && nb > 0) cv = load_word(word_buffer(a.chan_part, nb), (unsigned int)tid);
    const __amdgpu_buffer_rsrc_t gc = word_buffer(a.group_cnt, ng * R);
    int32_t gv[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)  // groups past ng lie past the buffer's end
        gv[u] = load_word(gc, gbase + (unsigned int)(u * R));
    // Keep every use below the last of these loads: all of them are in flight
    // before the first wait.
    __builtin_amdgcn_sched_barrier(0);

    int32_t esum[kMaxExperts / kTile];  // one partial per expert this thread sums
#pragma unroll
    for (int q = 0; q < kMaxExperts / kTile; ++q) esum[q] = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) esum[0] += ev[u];
    if (e_thread)  // tiles past the first pass
        for (int j = part0 + per_e * kBatch; j < nt; j += per_e * kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int jj = j + u * per_e;
                v[u] = jj < nt ? a.tile_expert[(int64_t)jj * E + e0] : 0;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) esum[0] += v[u];
        }
#pragma unroll
    for (int q = 1; q < kMaxExperts / kTile; ++q) {  // E > 256 only
        const int i = tid + q * kTile;
        if (!experts || i >= E * per_e) continue;
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
    if (cp_in_lds) {
        if (tid < nb) s.chan[tid] = cv;
        for (int i = tid + kTile; i < nb; i += kTile) s.chan[i] = a.chan_part[i];
    }

    int32_t carry = 0;
    if (scan_thread) {
        for (int pass = 0; pass < ng; pass += L * G) {
            const int g0 = pass + sj * G;
            int32_t v[kPerThread];
#pragma unroll
            for (int u = 0; u < kPerThread; ++u)
                v[u] = pass == 0 ? (u < G ? gv[u] : 0)
                       : (u < G && g0 + u < ng) ? a.group_cnt[(int64_t)(g0 + u) * R + sr] : 0;
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
                    if (gp_in_lds) s.gp[gg * R + sr] = run;
                }
                run += v[u];
            }
            carry += __shfl(incl, L - 1, L);
        }
        if (sj == 0) s.total[sr] = carry;
    }
    // Expert partials meet in LDS.
    for (int e = tid; e < E; e += kTile) s.hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxExperts / kTile; ++q) {
        const int i = tid + q * kTile;
        if (experts && i < E * per_e) {
            if (per_e == 1) s.hist[i] = esum[q];
            else atomicAdd(&s.hist[i % E], esum[q]);
        }
    }
    if (tid == 0) {
        int32_t run = 0;
        for (int r = 0; r < R; ++r) {
            s.base[r] = run;
            run += s.total[r];
        }
    }
    __syncthreads();
    if (tid < R) {
        a.num_tokens_per_rank[tid] = s.total[tid];
        if (a.rank_prefix_matrix) a.rank_prefix_matrix[tid] = s.base[tid] + s.total[tid];
        if (a.num_recv && tid == R - 1) *a.num_recv = s.base[tid] + s.total[tid];
    }
    if (experts)
        for (int e = tid; e < E; e += kTile) a.num_tokens_per_expert[e] = s.hist[e];
    // Channel prefixes, one (boundary, bucket) pair per thread:
    // excl(b, r) = group_prefix[b / 64][r] + (count from the group start to b).
    for (int i = tid; i < nb; i += kTile) {
        const int c = i / R, r = i % R;
        const int64_t b = layout_boundary(c, a.per, T);
        int32_t val;
        if (b >= T) {
            val = s.total[r];
        } else {
            const int g = (int)(b / kGroup);
            const int32_t gp = gp_in_lds ? s.gp[g * R + r] : a.group_prefix[(int64_t)g * R + r];
            val = gp + (cp_in_lds ? s.chan[i] : a.chan_part[i]);
        }
        if (c < a.C) a.recv_channel_prefix_matrix[r * a.C + c] = val;
        if (c > 0) a.channel_prefix_matrix[r * a.C + c - 1] = val;
    }
    if (tid == 0 && a.ticket) atomicExch(a.ticket, 0u);  // only a launch that took tickets
    return false;
}

}  // namespace moedx
