// Token pack (dispatch) kernels for gfx950: bf16 rows and FP8 E4M3 rows.
//
// The dispatch of the normal-kernel example in the EnflameTechnology/DeepEP
// README moves every token to each rank its routing names; on one GPU the
// ranks are buckets of one receive buffer, so the move is a copy of x[t] to
// the rows row(t, r) of t's buckets.  A first dispatch also completes the
// handle ("What the Handle Contains" on the handle-reuse page) with send_head
// and recv_src_idx; a cached dispatch only moves rows.
//
// Design (HBM-bound, no MFMA): one wavefront per token (or per 1/SPLIT of a
// token's row).  The wave finds the token's rows itself (rows.h: one ballot per
// destination bucket), reads its part of the row once with 16-byte loads, all
// of a lane's chunks in flight before the first store, then writes it to each
// destination row with 16-byte stores; destination rows are wave-uniform
// scalars.  Positions are a function of the routing only, so the launch shape
// never changes a result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "rows.h"

#ifndef MOEDX_PACK_SPLIT
#define MOEDX_PACK_SPLIT 4  // waves per token row
#endif
#ifndef MOEDX_PACK_NT_LOAD
#define MOEDX_PACK_NT_LOAD 0  // streaming (non-temporal) loads of x
#endif
#ifndef MOEDX_PACK_NT_STORE
#define MOEDX_PACK_NT_STORE 1  // streaming (non-temporal) stores of receive rows
#endif

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;
constexpr int kSplit = MOEDX_PACK_SPLIT;

template <typename V>
__device__ __forceinline__ V load_row(const V* p) {
#if MOEDX_PACK_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename V>
__device__ __forceinline__ void store_row(V v, V* p) {
#if MOEDX_PACK_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// The wave's token and part of the row; t is wave-uniform.
__device__ __forceinline__ void wave_work(int* t, int* part) {
    const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
    *t = w / kSplit;
    *part = w - *t * kSplit;
}

__device__ __forceinline__ void write_handle_rows(const HandleRows& hr, const TokenRows& d, int t,
                                                  int R, int lane) {
    if (hr.send_head == nullptr) return;
    if (lane < R) hr.send_head[(int64_t)t * R + lane] = d.pos;
    if (d.row >= 0) hr.recv_src_idx[d.row] = t;
}

// CPL = 16-byte chunks each lane moves per pass over its part of the row.
template <int CPL>
__global__ __launch_bounds__(256) void pack_bf16_kernel(
    const u32x4* __restrict__ x, int T, int H8, RowMap rm, HandleRows hr,
    u32x4* __restrict__ recv_x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, int K, int E, int P,
    int64_t* __restrict__ recv_topk_idx, float* __restrict__ recv_topk_weights) {
    const int lane = threadIdx.x & 63;
    int t, part;
    wave_work(&t, &part);
    if (t >= T) return;
    const TokenRows d = token_rows(rm, t, lane);
    if (part == 0) write_handle_rows(hr, d, t, rm.R, lane);
    const u32x4* src = x + (int64_t)t * H8;
    const int c_begin = (int)((int64_t)part * H8 / kSplit);
    const int c_end = (int)((int64_t)(part + 1) * H8 / kSplit);

    for (int base = c_begin; base < c_end; base += CPL * 64) {
        u32x4 v[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = base + i * 64 + lane;
            if (c < c_end) v[i] = load_row(src + c);
        }
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int row = __builtin_amdgcn_readlane(d.row, r);
            u32x4* dst = recv_x + (int64_t)row * H8;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < c_end) store_row(v[i], dst + c);
            }
        }
    }

    if (part == 0 && recv_topk_idx != nullptr && lane < K) {
        const int64_t e = topk_idx[(int64_t)t * K + lane];
        const float w = topk_weights ? topk_weights[(int64_t)t * K + lane] : 0.0f;
        const int eb = (e >= 0 && e < E) ? (int)e / P : -1;
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

// ---- FP8 -------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Nearest OCP E4M3FN code, ties to even, saturating at +/-448 (code 0x7E);
// NaN -> 0x7F.  Normal range (|q| >= 2^-6): round the fp32 mantissa to 3 bits
// with the round-half-even bias and re-bias the exponent from 127 to 7;
// subnormal range: the code is round-half-even(|q| * 2^9) directly.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0x7fu;
    uint32_t code;
    if (mag >= 0x3c800000u) {  // 2^-6
        const uint32_t r = (mag + 0x7ffffu + ((mag >> 20) & 1u)) >> 20;
        const int c = (int)r - (120 << 3);
        code = c > 0x7e ? 0x7eu : (uint32_t)c;
    } else {
        code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
    }
    return sign | code;
}

// One 16-byte chunk = 8 bf16 values; 16 consecutive lanes form one 1x128 block.
template <int CPL>
__global__ __launch_bounds__(256) void pack_fp8_kernel(const u32x4* __restrict__ x, int T, int H8,
                                                       RowMap rm, HandleRows hr,
                                                       u32x2* __restrict__ recv_x8,
                                                       float* __restrict__ recv_scales) {
    const int lane = threadIdx.x & 63;
    int t, part;
    wave_work(&t, &part);
    if (t >= T) return;
    const TokenRows d = token_rows(rm, t, lane);
    if (part == 0) write_handle_rows(hr, d, t, rm.R, lane);
    const u32x4* src = x + (int64_t)t * H8;
    const int G = H8 >> 4;  // blocks per row; parts hold whole blocks
    const int c_begin = (int)((int64_t)part * G / kSplit) * 16;
    const int c_end = (int)((int64_t)(part + 1) * G / kSplit) * 16;

    for (int base = c_begin; base < c_end; base += CPL * 64) {
        u32x2 code[CPL];
        float scale[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = base + i * 64 + lane;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < c_end) v = load_row(src + c);
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[2 * j] = bf16_lo(v[j]);
                f[2 * j + 1] = bf16_hi(v[j]);
            }
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
            // max over the 16 lanes of the block (all in the same 16-lane group)
            amax = fmaxf(amax, __shfl_xor(amax, 8));
            amax = fmaxf(amax, __shfl_xor(amax, 4));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            const float s = fmaxf(amax, 1e-4f) / 448.0f;
            scale[i] = s;
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) lo |= e4m3_code(f[j] / s) << (8 * j);
#pragma unroll
            for (int j = 0; j < 4; ++j) hi |= e4m3_code(f[4 + j] / s) << (8 * j);
            code[i] = u32x2{lo, hi};
        }
        uint64_t m = d.dest;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(d.row, r);
            u32x2* dst = recv_x8 + row * H8;
            float* sdst = recv_scales + row * G;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < c_end) {
                    store_row(code[i], dst + c);
                    if ((lane & 15) == 0) sdst[c >> 4] = scale[i];
                }
            }
        }
    }
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

int pack_blocks(int T) {
    return (int)(((int64_t)T * kSplit + kWavesPerBlock - 1) / kWavesPerBlock);
}

}  // namespace

hipError_t launch_pack_bf16(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                            void* recv_x, const int64_t* topk_idx, const float* topk_weights,
                            int K, int E, int P, int64_t* recv_topk_idx,
                            float* recv_topk_weights, const Launch& L) {
    const int H8 = H / 8;
    const dim3 grid(pack_blocks(T)), block(256);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* rx = static_cast<u32x4*>(recv_x);
#define MOEDX_PACK(N)                                                                         \
    return launch_kernel(pack_bf16_kernel<N>, grid, block, L, xs, T, H8, rm, hr, rx, topk_idx, \
                         topk_weights, K, E, P, recv_topk_idx, recv_topk_weights)
    switch (pick_cpl((H8 + kSplit - 1) / kSplit)) {
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

hipError_t launch_pack_fp8(const void* x, int T, int H, const RowMap& rm, const HandleRows& hr,
                           void* recv_x8, float* recv_scales, const Launch& L) {
    const int H8 = H / 8;
    const dim3 grid(pack_blocks(T)), block(256);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* rx = static_cast<u32x2*>(recv_x8);
    const int per_part = ((H8 / 16 + kSplit - 1) / kSplit) * 16;
#define MOEDX_PACK8(N) \
    return launch_kernel(pack_fp8_kernel<N>, grid, block, L, xs, T, H8, rm, hr, rx, recv_scales)
    switch (pick_cpl(per_part)) {
        case 1: MOEDX_PACK8(1);
        case 2: MOEDX_PACK8(2);
        case 4: MOEDX_PACK8(4);
        case 7: MOEDX_PACK8(7);
        case 8: MOEDX_PACK8(8);
        case 14: MOEDX_PACK8(14);
        default: MOEDX_PACK8(16);
    }
#undef MOEDX_PACK8
}

}  // namespace moedx
