// Token pack (dispatch) kernels for gfx950: bf16 rows and FP8 E4M3 rows.
//
// The dispatch of the normal-kernel example in the EnflameTechnology/DeepEP
// README moves every token to each rank its routing names; on one GPU the
// ranks are buckets of one receive buffer, so the move is a copy of x[t] to
// the rows row(t, r) of t's buckets.  A first dispatch also completes the
// handle ("What the Handle Contains" on the handle-reuse page) with send_head
// and recv_src_idx; a cached dispatch only moves rows.
//
// Design (HBM-bound, no MFMA): one wavefront per part of a token's row (at
// most 64 chunks of 16 bytes for bf16, 8 blocks of 1x128 for FP8), so a
// 7168-wide row is spread over 14 (bf16) or 7 (FP8) waves.  The wave finds the
// token's rows itself (rows.h: one ballot per destination bucket), reads its
// part of the row once with 16-byte loads, all of a lane's chunks in flight
// before the first store, then writes it to each destination row with
// streaming write-through 16-byte stores; destination rows are wave-uniform
// scalars.
// Positions are a function of the routing only, so the launch shape never
// changes a result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fp8_codec.h"
#include "launch.h"
#include "layout_core.h"
#include "rows.h"

#ifndef MOEDX_PACK_WAVE_CHUNKS
#define MOEDX_PACK_WAVE_CHUNKS 64  // 16-byte chunks of a bf16 row per wave (at most)
#endif
#ifndef MOEDX_PACK_FP8_WAVE_BLOCKS
#define MOEDX_PACK_FP8_WAVE_BLOCKS 8  // 1x128 blocks of an FP8 row per wave (at most)
#endif
#ifndef MOEDX_PACK_NT_STORE
#define MOEDX_PACK_NT_STORE 1  // streaming, write-through stores of receive rows
#endif

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaveChunks = MOEDX_PACK_WAVE_CHUNKS;
constexpr int kWaveBlocks = MOEDX_PACK_FP8_WAVE_BLOCKS;
// Every kernel below moves its part of a row in one pass of CPL chunks per
// lane; the launchers' CPL choices cover these part sizes.
static_assert(kWaveChunks >= 1 && kWaveChunks <= 128, "bf16 / byte parts: at most 2 chunks per lane");
static_assert(kWaveBlocks >= 1 && kWaveBlocks <= 8, "FP8 parts: at most 2 chunks per lane");


// 16-byte receive-row stores: streaming (nt) and written through to memory at
// system scope (sc0 sc1), which measured about 1 us faster than plain
// non-temporal stores on the 4096 x 7168 bf16 pack and about 2 us on the
// 16384 x 4096 cached dispatch (FP8: no difference).  No builtin sets sc0 /
// sc1 on a store, so this is one vector store in inline assembly; it returns
// nothing, so no wait counter is involved.
__device__ __forceinline__ void store_row(u32x4 v, u32x4* p) {
#if MOEDX_PACK_NT_STORE
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt" : : "v"(p), "v"(v) : "memory");
#else
    *p = v;
#endif
}

__device__ __forceinline__ void write_handle_rows(const HandleRows& hr, const TokenRows& d, int t,
                                                  int R, int lane) {
    if (hr.send_head == nullptr) return;
    if (lane < R) hr.send_head[(int64_t)t * R + lane] = d.pos;
    if (d.row >= 0) hr.recv_src_idx[d.row] = t;
}

// One wave's part of token t's bf16 row: chunks [c_begin, c_end).  The row
// loads are issued by pack_bf16_load (all of a lane's chunks in flight at
// once), before the row lookup; pack_bf16_store writes the part to each of the
// token's rows d, plus the handle rows and recv_topk_* from the first part.
// Chunks [c_begin, c_end) of one row, lane l taking c_begin + 64 i + l into
// v[i] (all of a lane's chunks in flight at once), as buffer loads: chunks
// past c_end read 0 and no load sits behind a branch, so a wait for loads
// issued before these (the row lookup's) need not wait for these.
template <int CPL>
__device__ __forceinline__ void load_row_part(const u32x4* __restrict__ row, int c_begin, int c_end,
                                              int lane, u32x4 (&v)[CPL]) {
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(row + c_begin), (short)0, (c_end - c_begin) * 16, 0x00020000);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (i * 64 + lane) * 16, 0, 0);
}

template <int CPL>
__device__ __forceinline__ void pack_bf16_store(
    const u32x4 (&v)[CPL], const TokenRows& d, int t, int part, int H8, int c_begin, int c_end,
    int lane, int R, const HandleRows& hr, u32x4* __restrict__ recv_x,
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int K, int E,
    int P, BucketDiv bucket, int64_t* __restrict__ recv_topk_idx,
    float* __restrict__ recv_topk_weights) {
    if (part == 0) write_handle_rows(hr, d, t, R, lane);
    {
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int row = __builtin_amdgcn_readlane(d.row, r);
            u32x4* dst = recv_x + (int64_t)row * H8;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = c_begin + i * 64 + lane;
                if (c < c_end) store_row(v[i], dst + c);
            }
        }
    }

    if (part == 0 && recv_topk_idx != nullptr && lane < K) {
        const int64_t e = topk_idx[(int64_t)t * K + lane];
        const float w = topk_weights ? topk_weights[(int64_t)t * K + lane] : 0.0f;
        const int eb = (e >= 0 && e < E) ? bucket.of((int)e) : -1;
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(d.row, r);
            const bool mine = (eb == r);
            recv_topk_idx[row * K + lane] = mine ? e - (int64_t)r * P : -1;
            if (recv_topk_weights) recv_topk_weights[row * K + lane] = mine ? w : 0.0f;
        }
    }
}

// CPL = 16-byte chunks each lane moves per pass over its part of the row.
template <int CPL>
__global__ __launch_bounds__(kRowThreads) void pack_bf16_kernel(
    const u32x4* __restrict__ x, int T, int H8, RowSplit rs, RowMap rm, HandleRows hr,
    u32x4* __restrict__ recv_x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, int K, int E, int P, BucketDiv bucket,
    int64_t* __restrict__ recv_topk_idx, float* __restrict__ recv_topk_weights) {
    const int lane = threadIdx.x & 63;
    int t, part;
    row_part(rs, &t, &part);
    if (t >= T) return;
    const int c_begin = part * rs.per;
    const int c_end = min(c_begin + rs.per, H8);
    // One pass (CPL * 64 >= rs.per).  The lookup's loads go out first, then
    // the row loads (no branch), so the lookup waits for its own loads only
    // and runs while the row is in flight.
    const RowLoads lk = token_rows_load(rm, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(x + (int64_t)t * H8, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from(rm, lk, t, lane);
    pack_bf16_store<CPL>(v, d, t, part, H8, c_begin, c_end, lane, rm.R, hr, recv_x, topk_idx,
                         topk_weights, K, E, P, bucket, recv_topk_idx, recv_topk_weights);
}

// ---- first dispatch on a handle whose prefixes are not yet computed ------------

// Rows of token t from the layout's partials alone (at most 64 groups, R a
// multiple of 4 and at most 16): lane l holds group l's count of every bucket,
// loaded as R / 4 16-byte words of its group_cnt row, so that a wave asks for
// each line of group_cnt once.  Two buckets share a 32-bit word (16-bit fields:
// a bucket holds at most 4096 tokens here) and one wave prefix sum per pair
// gives the bucket totals (lane 63) and the counts of the groups before t's
// group g (lane g - 1).  The bucket offsets are the running sum of the totals.
// Then as token_rows: lane r holds row(t, r).  The loads are issued by
// load_group_counts, the rows computed by token_rows_from_counts.
template <int RB>
struct GroupCounts {
    u32x4 c[RB / 4];  // lane l: buckets 4q..4q+3 of group l
    uint64_t gm;      // lane l: token_mask of token 64 g + l
};

template <int RB>
__device__ __forceinline__ GroupCounts<RB> load_group_counts(const uint64_t* token_mask,
                                                             const int32_t* group_cnt, int T,
                                                             int R, int t, int lane) {
    const int ng = num_groups(T);
    const __amdgpu_buffer_rsrc_t gc = word_buffer(group_cnt, ng * R);
    const unsigned int lbase = lane < ng ? (unsigned int)(lane * R) : kNoWord;
    GroupCounts<RB> gcnt;
#pragma unroll
    for (int q = 0; q < RB / 4; ++q) {
        const unsigned int i = 4 * q < R ? lbase + (unsigned int)(4 * q) : kNoWord;
        gcnt.c[q] = __builtin_amdgcn_raw_buffer_load_b128(gc, (int)(i * 4u), 0, 0);
    }
    const int tj = ((t >> 6) << 6) + lane;
    gcnt.gm = tj < T ? token_mask[tj] : 0ull;
    return gcnt;
}

template <int RB>
__device__ __forceinline__ TokenRows token_rows_from_counts(const GroupCounts<RB>& gcnt, int R,
                                                            int64_t rows, int t, int lane) {
    const int g = t >> 6;
    const int j = t & 63;
    const uint64_t gm = gcnt.gm;
    int base = 0, pfx = 0, run = 0;
#pragma unroll
    for (int p = 0; p < RB; p += 2) {
        if (p >= R) break;  // wave-uniform
        const uint32_t lo = gcnt.c[p >> 2][p & 3], hi = gcnt.c[p >> 2][(p & 3) + 1];
        const uint32_t incl = (uint32_t)wave_inclusive_sum((int)(lo | (hi << 16)));
        const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t pre = g > 0 ? __builtin_amdgcn_readlane(incl, g - 1) : 0u;
        if (lane == p) {
            base = run;
            pfx = (int)(pre & 0xffffu);
        }
        run += (int)(tot & 0xffffu);
        if (lane == p + 1) {
            base = run;
            pfx = (int)(pre >> 16);
        }
        run += (int)(tot >> 16);
    }
    const uint64_t mine = readlane64(gm, j);
    const uint64_t below = (j == 0) ? 0ull : (~0ull >> (64 - j));
    int pos = -1;
    uint64_t m = mine;
    while (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
        const int c = __popcll(__ballot((gm >> r) & 1u) & below);
        if (lane == r) pos = pfx + c;
    }
    const int64_t row64 = pos >= 0 ? (int64_t)base + pos : -1;
    const int row = (row64 >= 0 && row64 < rows) ? (int)row64 : -1;
    return TokenRows{row, pos, mine, __ballot(row >= 0)};
}

// A handle that borrowed a layout's partials gets token t's mask,
// is_token_in_rank row and slot buckets from its first pack (nothing otherwise).
__device__ __forceinline__ void write_borrowed_token(const HandleTokens& ht, const TokenRows& d,
                                                     int t, int R, int K, int lane) {
    if (ht.token_mask == nullptr) return;
    if (lane == 0) ht.token_mask[t] = d.mask;
    if (lane < R) ht.is_token_in_rank[(int64_t)t * R + lane] = (uint8_t)((d.mask >> lane) & 1u);
    if (lane < K) ht.slot_bucket[(int64_t)t * K + lane] = ht.slot_bucket_src[(int64_t)t * K + lane];
}

// The workgroup that finishes the handle runs the layout's straight-line
// finishing step for one chunk of 64 groups and 16 tiles: its LDS holds the
// group prefixes of up to 64 groups of 16 buckets.
using FirstLds = LayoutShared<kGroup * 16, 0>;
constexpr int kFirstChunks = 1;
constexpr int kFirstTiles = 16;

// The first dispatch on a capacity-mode handle prepared with the layout's
// partials only.  Workgroup 0 finishes the handle (every prefix, total and
// channel matrix, as the layout's finishing step); every other workgroup is a
// pack_bf16_kernel workgroup that finds its token's rows from the partials
// (token_rows_from_counts) instead of from the prefixes, so nothing in this
// launch waits for workgroup 0.
template <int CPL, int RB>
__global__ __launch_bounds__(kRowThreads) void pack_bf16_first_kernel(
    LayoutArgs la, HandleTokens ht, int ntiles, const u32x4* __restrict__ x, int H8, RowSplit rs,
    int64_t rows, HandleRows hr, u32x4* __restrict__ recv_x, const float* __restrict__ topk_weights,
    int64_t* __restrict__ recv_topk_idx, float* __restrict__ recv_topk_weights) {
    __shared__ FirstLds s;
    if (blockIdx.x == 0) {
        layout_finish_fast<kFirstChunks, kFirstTiles>(la, ntiles, s, (const TileToken*)nullptr);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((blockIdx.x - 1) * kRowWavesPerBlock +
                                                 (threadIdx.x >> 6));
    const int t = (int)rs.div.div((uint32_t)w);
    const int part = w - t * rs.split;
    if (t >= la.T) return;
    const int c_begin = part * rs.per;
    const int c_end = min(c_begin + rs.per, H8);
    // The counts go out first: their prefix sums run while the row is in flight.
    const GroupCounts<RB> gcnt =
        load_group_counts<RB>(la.token_mask, la.group_cnt, la.T, la.R, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(x + (int64_t)t * H8, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from_counts<RB>(gcnt, la.R, rows, t, lane);
    if (part == 0) write_borrowed_token(ht, d, t, la.R, la.K, lane);
    pack_bf16_store<CPL>(v, d, t, part, H8, c_begin, c_end, lane, la.R, hr, recv_x, la.topk_idx,
                         topk_weights, la.K, la.E, la.P, la.bucket, recv_topk_idx,
                         recv_topk_weights);
}

// ---- FP8 -------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Maximum over the 16 lanes of a DPP row (the lanes of one 1x128 block), by
// lane permutations within the row: swap neighbours, swap pairs, mirror each
// half, mirror the row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    return v;
}

// Scale modes of the FP8 pack (the values of moedx.h's MOEDX_FP8_SCALE_*).
enum Fp8Mode { kAmax = 0, kPow2 = 1, kUe8m0 = 2, kTensor = 3 };

// One 16-byte chunk = 8 bf16 values; 16 consecutive lanes (one DPP row) form
// one 1x128 block.  Codes are bit-identical to encoding the IEEE quotient
// x / s with e4m3_code, the definition the scale and codes follow; the scale
// s of a block depends on kMode (moedx.h).  tensor_s / tensor_rs: the caller's
// scale and its correctly rounded reciprocal (kTensor only).
// One wave's part of token t's FP8 row, chunks [c_begin, c_end) of its bf16
// row in v (whole 1x128 blocks), quantised and stored to each of the token's
// rows d, with the handle rows from the first part.
template <int CPL, int kMode>
__device__ __forceinline__ void pack_fp8_part(const u32x4 (&v)[CPL], const TokenRows& d, int t,
                                              int part, int H8, int c_begin, int c_end, int lane,
                                              int R, const HandleRows& hr,
                                              u32x2* __restrict__ recv_x8,
                                              void* __restrict__ recv_scales, float tensor_s,
                                              float tensor_rs) {
    const int G = H8 >> 4;  // blocks per row
    if (part == 0) write_handle_rows(hr, d, t, R, lane);
    {
        const int base = c_begin;
        u32x2 code[CPL];
        float scale[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            // Block maximum of |x| on the bit patterns: for non-negative
            // floats the integer order is the numeric order, and inf / NaN
            // sort above every finite value.
            uint32_t ab = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ab = max(ab, max((v[i][j] << 16) & 0x7fffffffu, v[i][j] & 0x7fff0000u));
            ab = row16_max(ab);
            uint32_t w0, w1;
            float s;
            if (ab < 0x7f800000u) {
                // Finite block: every q = x / s as a correctly rounded quotient
                // (exact when s is a power of two), then gfx950's fp32 ->
                // E4M3FN pack conversion (round to nearest even).  That
                // instruction gives e4m3_code's result on every
                // |q| <= 448 * (1 + 2^-23) of either sign (checked exhaustively
                // on the device), and |q| never exceeds that bound here (the
                // per-tensor scale clamps), so no saturation or NaN case
                // reaches it.
                float rs;
                if (kMode == kTensor) {
                    s = tensor_s;
                    rs = tensor_rs;
                } else {
                    const float sa = fp8_block_scale(ab);
                    if (kMode == kAmax) {
                        s = sa;
                        rs = 1.0f / s;
                    } else {  // a power of two: its reciprocal flips the exponent
                        s = pow2_ceil(sa);
                        rs = pow2_reciprocal(s);
                    }
                }
                float qs[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t fb =
                        (j & 1) ? (v[i][j >> 1] & 0xffff0000u) : (v[i][j >> 1] << 16);
                    const float a = fabsf(__uint_as_float(fb));
                    float q;
                    if (kMode == kPow2 || kMode == kUe8m0) {
                        q = a * rs;  // exact
                    } else if (kMode == kTensor) {
                        q = tensor_quotient(a, s, rs);
                    } else {
                        q = quotient(a, s, rs);
                    }
                    qs[j] = __uint_as_float(__float_as_uint(q) | (fb & 0x80000000u));
                }
                w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qs[0], qs[1], 0, false);
                w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qs[2], qs[3], (int)w0, true);
                w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qs[4], qs[5], 0, false);
                w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qs[6], qs[7], (int)w1, true);
            } else {
                // A block holding inf or NaN (all 16 lanes take this branch):
                // amax ignores NaN, then IEEE quotients through the general
                // encoder (saturation, NaN -> 0x7F).
                float f[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f[2 * j] = bf16_lo(v[i][j]);
                    f[2 * j + 1] = bf16_hi(v[i][j]);
                }
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
                amax = fmaxf(amax, __shfl_xor(amax, 8));
                amax = fmaxf(amax, __shfl_xor(amax, 4));
                amax = fmaxf(amax, __shfl_xor(amax, 2));
                amax = fmaxf(amax, __shfl_xor(amax, 1));
                if (kMode == kTensor) s = tensor_s;
                else s = fmaxf(amax, 1e-4f) / 448.0f;
                if (kMode == kPow2 || kMode == kUe8m0) s = pow2_ceil(s);
                uint32_t cj[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) cj[j] = e4m3_code(f[j] / s);
                w0 = cj[0] | (cj[1] << 8) | (cj[2] << 16) | (cj[3] << 24);
                w1 = cj[4] | (cj[5] << 8) | (cj[6] << 16) | (cj[7] << 24);
            }
            scale[i] = s;
            code[i] = u32x2{w0, w1};
        }
        // Even lanes take their odd neighbour's 8 code bytes and store 16.
        u32x4 code2[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t nx =
                (uint32_t)__builtin_amdgcn_update_dpp(0, (int)code[i][0], 0xF5, 0xf, 0xf, false);
            const uint32_t ny =
                (uint32_t)__builtin_amdgcn_update_dpp(0, (int)code[i][1], 0xF5, 0xf, 0xf, false);
            code2[i] = u32x4{code[i][0], code[i][1], nx, ny};
        }
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(d.row, r);
            u32x2* dst = recv_x8 + row * H8;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < c_end) {
                    if ((lane & 1) == 0) store_row(code2[i], reinterpret_cast<u32x4*>(dst + c));
                    if ((lane & 15) == 0) {
                        if (kMode == kAmax || kMode == kPow2)
                            static_cast<float*>(recv_scales)[row * G + (c >> 4)] = scale[i];
                        else if (kMode == kUe8m0)  // the exponent field of s (0xFF for inf)
                            static_cast<uint8_t*>(recv_scales)[row * G + (c >> 4)] =
                                (uint8_t)(__float_as_uint(scale[i]) >> 23);
                    }
                }
            }
        }
    }
}

template <int CPL, int kMode>
__global__ __launch_bounds__(kRowThreads) void pack_fp8_kernel(
    const u32x4* __restrict__ x, int T, int H8, RowSplit rs, RowMap rm, HandleRows hr,
    u32x2* __restrict__ recv_x8, void* __restrict__ recv_scales, float tensor_s, float tensor_rs) {
    const int lane = threadIdx.x & 63;
    int t, part;
    row_part(rs, &t, &part);
    if (t >= T) return;
    const u32x4* src = x + (int64_t)t * H8;
    const int G = H8 >> 4;  // blocks per row; parts hold whole blocks (rs counts blocks)
    const int c_begin = part * rs.per * 16;
    const int c_end = min(part * rs.per + rs.per, G) * 16;
    // One pass (CPL * 64 >= 16 * rs.per): the lookup's loads, then the row
    // loads (chunks past c_end read 0).
    const RowLoads lk = token_rows_load(rm, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(src, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from(rm, lk, t, lane);
    pack_fp8_part<CPL, kMode>(v, d, t, part, H8, c_begin, c_end, lane, rm.R, hr, recv_x8,
                              recv_scales, tensor_s, tensor_rs);
}

// The first FP8 dispatch on a capacity-mode handle prepared with the layout's
// partials only (or borrowing them), in one launch: workgroup 0 finishes the
// handle and every other wave finds its token's rows from the partials, as in
// pack_bf16_first_kernel, then quantises and stores as pack_fp8_kernel.
template <int CPL, int kMode, int RB>
__global__ __launch_bounds__(kRowThreads) void pack_fp8_first_kernel(
    LayoutArgs la, HandleTokens ht, int ntiles, const u32x4* __restrict__ x, int H8, RowSplit rs,
    int64_t rows, HandleRows hr, u32x2* __restrict__ recv_x8, void* __restrict__ recv_scales,
    float tensor_s, float tensor_rs) {
    __shared__ FirstLds s;
    if (blockIdx.x == 0) {
        layout_finish_fast<kFirstChunks, kFirstTiles>(la, ntiles, s, (const TileToken*)nullptr);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((blockIdx.x - 1) * kRowWavesPerBlock +
                                                 (threadIdx.x >> 6));
    const int t = (int)rs.div.div((uint32_t)w);
    const int part = w - t * rs.split;
    if (t >= la.T) return;
    const int G = H8 >> 4;
    const int c_begin = part * rs.per * 16;
    const int c_end = min(part * rs.per + rs.per, G) * 16;
    const GroupCounts<RB> gcnt =
        load_group_counts<RB>(la.token_mask, la.group_cnt, la.T, la.R, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(x + (int64_t)t * H8, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from_counts<RB>(gcnt, la.R, rows, t, lane);
    if (part == 0) write_borrowed_token(ht, d, t, la.R, la.K, lane);
    pack_fp8_part<CPL, kMode>(v, d, t, part, H8, c_begin, c_end, lane, la.R, hr, recv_x8,
                              recv_scales, tensor_s, tensor_rs);
}

// Pre-quantised rows: code rows (C16 16-byte chunks) and scale rows (SB bytes)
// of token t go unchanged to every receive row of t.  One wave per (token,
// part of the code row); part 0 also moves the scale row.  pack_bytes_part is
// what a wave does once it holds its part of the code row (v) and the token's
// rows (d).
template <int CPL>
__device__ __forceinline__ void pack_bytes_part(
    const u32x4 (&v)[CPL], const TokenRows& d, int t, int part, int C16, int c_begin, int c_end,
    int lane, int R, const HandleRows& hr, const uint8_t* __restrict__ scales, int SB,
    u32x4* __restrict__ recv, uint8_t* __restrict__ recv_scales, bool words) {
    if (part == 0) write_handle_rows(hr, d, t, R, lane);
    {
        const int base = c_begin;
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(d.row, r);
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < c_end) store_row(v[i], recv + row * C16 + c);
            }
        }
    }
    if (part == 0 && scales != nullptr) {
        if (words) {  // SB % 4 == 0 and both scale arrays 4-byte aligned: 4 bytes per lane
            const int SW = SB >> 2;
            const uint32_t* s32 = reinterpret_cast<const uint32_t*>(scales);
            uint32_t* r32 = reinterpret_cast<uint32_t*>(recv_scales);
            for (int b0 = 0; b0 < SW; b0 += 64) {
                const int b = b0 + lane;
                const uint32_t sv = b < SW ? s32[(int64_t)t * SW + b] : 0u;
                uint64_t m = d.dest;
                while (m) {
                    const int r = __builtin_ctzll(m);
                    m &= m - 1;
                    const int64_t row = __builtin_amdgcn_readlane(d.row, r);
                    if (b < SW) r32[row * SW + b] = sv;
                }
            }
        } else {
            for (int b0 = 0; b0 < SB; b0 += 64) {
                const int b = b0 + lane;
                const uint8_t sv = b < SB ? scales[(int64_t)t * SB + b] : 0;
                uint64_t m = d.dest;
                while (m) {
                    const int r = __builtin_ctzll(m);
                    m &= m - 1;
                    const int64_t row = __builtin_amdgcn_readlane(d.row, r);
                    if (b < SB) recv_scales[row * SB + b] = sv;
                }
            }
        }
    }
}

template <int CPL>
__global__ __launch_bounds__(kRowThreads) void pack_bytes_kernel(
    const u32x4* __restrict__ codes, const uint8_t* __restrict__ scales, int T, int C16, int SB,
    RowSplit rs, RowMap rm, HandleRows hr, u32x4* __restrict__ recv,
    uint8_t* __restrict__ recv_scales, bool words) {
    const int lane = threadIdx.x & 63;
    int t, part;
    row_part(rs, &t, &part);
    if (t >= T) return;
    const u32x4* src = codes + (int64_t)t * C16;
    const int c_begin = part * rs.per;
    const int c_end = min(c_begin + rs.per, C16);
    // One pass (CPL * 64 >= rs.per): the lookup's loads, then the row loads.
    const RowLoads lk = token_rows_load(rm, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(src, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from(rm, lk, t, lane);
    pack_bytes_part<CPL>(v, d, t, part, C16, c_begin, c_end, lane, rm.R, hr, scales, SB, recv,
                         recv_scales, words);
}

// The first pre-quantised dispatch on a capacity-mode handle prepared with the
// layout's partials only (or borrowing them), in one launch: workgroup 0
// finishes the handle and every other wave finds its token's rows from the
// partials, as in pack_bf16_first_kernel, then moves its part as
// pack_bytes_kernel.
template <int CPL, int RB>
__global__ __launch_bounds__(kRowThreads) void pack_bytes_first_kernel(
    LayoutArgs la, HandleTokens ht, int ntiles, const u32x4* __restrict__ codes,
    const uint8_t* __restrict__ scales, int C16, int SB, RowSplit rs, int64_t rows, HandleRows hr,
    u32x4* __restrict__ recv, uint8_t* __restrict__ recv_scales, bool words) {
    __shared__ FirstLds s;
    if (blockIdx.x == 0) {
        layout_finish_fast<kFirstChunks, kFirstTiles>(la, ntiles, s, (const TileToken*)nullptr);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((blockIdx.x - 1) * kRowWavesPerBlock +
                                                 (threadIdx.x >> 6));
    const int t = (int)rs.div.div((uint32_t)w);
    const int part = w - t * rs.split;
    if (t >= la.T) return;
    const int c_begin = part * rs.per;
    const int c_end = min(c_begin + rs.per, C16);
    const GroupCounts<RB> gcnt =
        load_group_counts<RB>(la.token_mask, la.group_cnt, la.T, la.R, t, lane);
    u32x4 v[CPL];
    load_row_part<CPL>(codes + (int64_t)t * C16, c_begin, c_end, lane, v);
    const TokenRows d = token_rows_from_counts<RB>(gcnt, la.R, rows, t, lane);
    if (part == 0) write_borrowed_token(ht, d, t, la.R, la.K, lane);
    pack_bytes_part<CPL>(v, d, t, part, C16, c_begin, c_end, lane, la.R, hr, scales, SB, recv,
                         recv_scales, words);
}

int pick_cpl(int chunks) {
    const int need = (chunks + 63) / 64;
    if (need <= 1) return 1;
    if (need <= 2) return 2;
    if (need <= 4) return 4;
    if (need <= 7) return 7;
    if (need <= 8) return 8;
    if (need <= 14) return 14;
    return 16;
}

// Waves per token row: enough that no wave moves more than kWaveChunks chunks
// (kWaveBlocks whole 1x128 blocks for FP8); each part holds ceil(units /
// split) units, the last one what remains (RowSplit).  Short
// parts keep many small waves in flight (measured best for bf16 rows); the
// FP8 pack, which also computes, does best with 128 chunks per wave.
int pack_split(int units, int units_per_wave) {
    const int s = (units + units_per_wave - 1) / units_per_wave;
    return s < 1 ? 1 : s;
}

int pack_blocks(int T, int split) { return (int)row_blocks(T, split); }

// Workgroups (of 4 waves) per CU that the row-copy kernels below run with,
// measured with every input read from HBM (time per launch over back-to-back
// launches; 8 is what their registers allow, so 8 means no cap):
//   bf16 cached pack: 7 against 8 -- 48.1-48.4 against 50.1-50.3 us on
//   4096 x 7168 (8 buckets), 139.0-140.3 against 144.5-146.7 us on 16384 x 4096
//   (16 buckets), 73.4-74.4 against 72.6-72.9 us on the 8192 x 7168 Zipf
//   routing; 6 or fewer were slower on all three.  A first dispatch through the
//   same kernel (handle rows and recv_topk_* too) was slower capped (layout +
//   pack at 16384 x 4096: 177.5-178.0 against 168.5-169.3 us) and runs
//   uncapped.
//   FP8 pack: 4 against 8 -- 49.7-50.0 against 52.0-52.9 us (8192 x 7168 Zipf),
//   31.9-32.0 against 34.0-34.4 us (4096 x 7168), 82.8 against 90.1-90.4 us
//   (16384 x 4096); 3 were slower (72-73 us at 8192 x 7168); a first FP8
//   dispatch (layout + pack at 8192 x 7168) 59.2-61.9 against 60.0-61.2 us.
//   The first bf16 pack, whose row lookup is a longer chain of loads, and the
//   combine were slower under every cap and run uncapped.
constexpr int kCachedPackWorkgroupsPerCu = 7;
constexpr int kFp8PackWorkgroupsPerCu = 4;

}  // namespace

unsigned int occupancy_lds(int workgroups_per_cu, unsigned int static_lds) {
    constexpr unsigned int kLdsPerCu = 160u * 1024u, kMaxPerWorkgroup = 64u * 1024u;
    if (workgroups_per_cu < 1) return 0;
    const unsigned int per_wg =
        std::min((kLdsPerCu / (unsigned int)workgroups_per_cu) & ~511u, kMaxPerWorkgroup);
    return per_wg > static_lds ? per_wg - static_lds : 0u;
}

hipError_t launch_pack_bf16(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                            void* recv_x, const int64_t* topk_idx, const float* topk_weights,
                            int K, int E, int P, BucketDiv bucket, int64_t* recv_topk_idx,
                            float* recv_topk_weights, const Launch& L) {
    const int H8 = H / 8;
    const int split = pack_split(H8, kWaveChunks);
    const RowSplit rs = make_row_split(H8, split);
    const dim3 grid(pack_blocks(T, split)), block(kRowThreads);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* rx = static_cast<u32x4*>(recv_x);
    const bool cached = hr.send_head == nullptr && recv_topk_idx == nullptr;
    Launch Lc = L;
    Lc.lds_bytes = cached ? occupancy_lds(kCachedPackWorkgroupsPerCu, 0) : 0u;
#define MOEDX_PACK(N)                                                                   \
    return launch_kernel(pack_bf16_kernel<N>, grid, block, Lc, xs, T, H8, rs, rm, hr, rx, \
                         topk_idx, topk_weights, K, E, P, bucket, recv_topk_idx,         \
                         recv_topk_weights)
    switch (pick_cpl(rs.per)) {
        case 1: MOEDX_PACK(1);
        case 2: MOEDX_PACK(2);
        case 4: MOEDX_PACK(4);
        case 7: MOEDX_PACK(7);
        case 8: MOEDX_PACK(8);
        case 14: MOEDX_PACK(14);
        default: MOEDX_PACK(16);
    }
#undef MOEDX_PACK
}

bool pack_first_fits(int T, int R, int E, int C) {
    return layout_fast_finish_fits<kFirstChunks, kFirstTiles>(T, R, E, C, num_tiles(T), true,
                                                              FirstLds::kGp) &&
           R <= 16 && R % 4 == 0;
}

hipError_t launch_pack_bf16_first(const LayoutArgs& la, const HandleTokens& ht, const void* x,
                                  int H, int64_t rows, const HandleRows& hr, void* recv_x,
                                  const float* topk_weights, int64_t* recv_topk_idx,
                                  float* recv_topk_weights, const Launch& L) {
    const int T = la.T;
    const int H8 = H / 8;
    const int split = pack_split(H8, kWaveChunks);
    const RowSplit rs = make_row_split(H8, split);
    const dim3 grid(1 + pack_blocks(T, split)), block(kRowThreads);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* rx = static_cast<u32x4*>(recv_x);
    const int ntiles = num_tiles(T);
#define MOEDX_FIRST(N, B)                                                                       \
    return launch_kernel(pack_bf16_first_kernel<N, B>, grid, block, L, la, ht, ntiles, xs, H8, \
                         rs, rows, hr, rx, topk_weights, recv_topk_idx, recv_topk_weights)
#define MOEDX_FIRST_CPL(B)              \
    switch (pick_cpl(rs.per)) {         \
        case 1: MOEDX_FIRST(1, B);      \
        case 2: MOEDX_FIRST(2, B);      \
        case 4: MOEDX_FIRST(4, B);      \
        case 7: MOEDX_FIRST(7, B);      \
        case 8: MOEDX_FIRST(8, B);      \
        case 14: MOEDX_FIRST(14, B);    \
        default: MOEDX_FIRST(16, B);    \
    }
    if (la.R <= 8) {
        MOEDX_FIRST_CPL(8)
    } else {
        MOEDX_FIRST_CPL(16)
    }
#undef MOEDX_FIRST_CPL
#undef MOEDX_FIRST
}

hipError_t launch_pack_fp8(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                           void* recv_x8, void* recv_scales, int mode, float tensor_scale,
                           const Launch& L) {
    const int H8 = H / 8;
    const int split = pack_split(H8 / 16, kWaveBlocks);
    const RowSplit rs = make_row_split(H8 / 16, split);  // in 1x128 blocks
    const dim3 grid(pack_blocks(T, split)), block(kRowThreads);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* rx = static_cast<u32x2*>(recv_x8);
    const float trs = mode == kTensor ? 1.0f / tensor_scale : 0.0f;
    const bool two = pick_cpl(rs.per * 16) > 1;  // at most 16 * kWaveBlocks chunks
    Launch Lc = L;
    Lc.lds_bytes = occupancy_lds(kFp8PackWorkgroupsPerCu, 0);
#define MOEDX_PACK8(M)                                                                        \
    return two ? launch_kernel(pack_fp8_kernel<2, M>, grid, block, Lc, xs, T, H8, rs, rm, hr, \
                               rx, recv_scales, tensor_scale, trs)                            \
               : launch_kernel(pack_fp8_kernel<1, M>, grid, block, Lc, xs, T, H8, rs, rm, hr, \
                               rx, recv_scales, tensor_scale, trs)
    switch (mode) {
        case kAmax: MOEDX_PACK8(kAmax);
        case kPow2: MOEDX_PACK8(kPow2);
        case kUe8m0: MOEDX_PACK8(kUe8m0);
        default: MOEDX_PACK8(kTensor);
    }
#undef MOEDX_PACK8
}

hipError_t launch_pack_fp8_first(const LayoutArgs& la, const HandleTokens& ht, const void* x,
                                 int H, int64_t rows, const HandleRows& hr, void* recv_x8,
                                 void* recv_scales, int mode, float tensor_scale, const Launch& L) {
    const int T = la.T;
    const int H8 = H / 8;
    const int split = pack_split(H8 / 16, kWaveBlocks);
    const RowSplit rs = make_row_split(H8 / 16, split);  // in 1x128 blocks
    const dim3 grid(1 + pack_blocks(T, split)), block(kRowThreads);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* rx = static_cast<u32x2*>(recv_x8);
    const float trs = mode == kTensor ? 1.0f / tensor_scale : 0.0f;
    const int ntiles = num_tiles(T);
    const bool two = pick_cpl(rs.per * 16) > 1;
    Launch Lc = L;
    Lc.lds_bytes = occupancy_lds(kFp8PackWorkgroupsPerCu, (unsigned int)sizeof(FirstLds));
#define MOEDX_FIRST8(C, M, B)                                                                    \
    return launch_kernel(pack_fp8_first_kernel<C, M, B>, grid, block, Lc, la, ht, ntiles, xs, H8, \
                         rs, rows, hr, rx, recv_scales, tensor_scale, trs)
#define MOEDX_FIRST8_MODE(C, B)              \
    switch (mode) {                          \
        case kAmax: MOEDX_FIRST8(C, kAmax, B);   \
        case kPow2: MOEDX_FIRST8(C, kPow2, B);   \
        case kUe8m0: MOEDX_FIRST8(C, kUe8m0, B); \
        default: MOEDX_FIRST8(C, kTensor, B);    \
    }
    if (la.R <= 8) {
        if (two) { MOEDX_FIRST8_MODE(2, 8) } else { MOEDX_FIRST8_MODE(1, 8) }
    } else {
        if (two) { MOEDX_FIRST8_MODE(2, 16) } else { MOEDX_FIRST8_MODE(1, 16) }
    }
#undef MOEDX_FIRST8_MODE
#undef MOEDX_FIRST8
}

hipError_t launch_pack_bytes_first(const LayoutArgs& la, const HandleTokens& ht, const void* codes,
                                  const void* scales, int H, int scale_bytes, int64_t rows,
                                  const HandleRows& hr, void* recv_codes, void* recv_scales,
                                  const Launch& L) {
    const int T = la.T;
    const int C16 = H / 16;
    const int split = pack_split(C16, kWaveChunks);
    const RowSplit parts = make_row_split(C16, split);
    const dim3 grid(1 + pack_blocks(T, split)), block(kRowThreads);
    const u32x4* cs = static_cast<const u32x4*>(codes);
    u32x4* rc = static_cast<u32x4*>(recv_codes);
    const uint8_t* ss = static_cast<const uint8_t*>(scales);
    uint8_t* rs = static_cast<uint8_t*>(recv_scales);
    const bool words = (scale_bytes & 3) == 0 && (reinterpret_cast<uintptr_t>(ss) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(rs) & 3u) == 0;
    const int ntiles = num_tiles(T);
    const bool two = pick_cpl(parts.per) > 1;
#define MOEDX_FIRSTB(C, B)                                                                        \
    return launch_kernel(pack_bytes_first_kernel<C, B>, grid, block, L, la, ht, ntiles, cs, ss, C16, \
                         scale_bytes, parts, rows, hr, rc, rs, words)
    if (la.R <= 8) {
        if (two) MOEDX_FIRSTB(2, 8);
        MOEDX_FIRSTB(1, 8);
    }
    if (two) MOEDX_FIRSTB(2, 16);
    MOEDX_FIRSTB(1, 16);
#undef MOEDX_FIRSTB
}

hipError_t launch_pack_bytes(const void* codes, const void* scales, int T, int H, int scale_bytes,
                             const RowMap& rm, const HandleRows& hr, void* recv_codes,
                             void* recv_scales, const Launch& L) {
    const int C16 = H / 16;
    const int split = pack_split(C16, kWaveChunks);
    const RowSplit parts = make_row_split(C16, split);
    const dim3 grid(pack_blocks(T, split)), block(kRowThreads);
    const u32x4* cs = static_cast<const u32x4*>(codes);
    u32x4* rc = static_cast<u32x4*>(recv_codes);
    const uint8_t* ss = static_cast<const uint8_t*>(scales);
    uint8_t* rs = static_cast<uint8_t*>(recv_scales);
    const bool words = (scale_bytes & 3) == 0 && (reinterpret_cast<uintptr_t>(ss) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(rs) & 3u) == 0;
    if (pick_cpl(parts.per) > 1)
        return launch_kernel(pack_bytes_kernel<2>, grid, block, L, cs, ss, T, C16, scale_bytes,
                             parts, rm, hr, rc, rs, words);
    return launch_kernel(pack_bytes_kernel<1>, grid, block, L, cs, ss, T, C16, scale_bytes, parts,
                         rm, hr, rc, rs, words);
}

}  // namespace moedx
