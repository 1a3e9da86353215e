// Token pack (dispatch) kernels for gfx950: bf16 rows and FP8 E4M3 rows.
//
// The dispatch of the normal-kernel example in the EnflameTechnology/DeepEP
// README moves every token to each rank its routing names; on one GPU the
// ranks are buckets of one receive buffer, so the move is a copy of x[t] to
// rows row(t,r) = base[r] + send_head[t,r] (handle fields listed under "What
// the Handle Contains" on the handle-reuse page).
//
// Design (HBM-bound, no MFMA): one wavefront per token.  The wave reads the
// token's row once with 16-byte loads (all of a lane's chunks in flight before
// the first store), then writes it to each destination row with 16-byte
// non-temporal stores; destination rows are wave-uniform (scalar registers).
// Rows are located through send_head, so the launch shape never changes a
// result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;

struct Dest {
    int row;        // this lane's bucket row (lane = bucket), or -1
    uint64_t mask;  // buckets the token goes to (wave-uniform)
};

__device__ __forceinline__ Dest token_rows(const RowMap& rm, int t, int lane) {
    int row = -1;
    if (lane < rm.R) {
        const int pos = rm.send_head[(int64_t)t * rm.R + lane];
        if (pos >= 0) row = rm.rank_prefix_matrix[lane] - rm.num_tokens_per_rank[lane] + pos;
    }
    return Dest{row, __ballot(row >= 0)};
}

__device__ __forceinline__ int wave_token() {
    return __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
}

// CPL = 16-byte chunks each lane moves per pass over the row.
template <int CPL>
__global__ __launch_bounds__(256) void pack_bf16_kernel(
    const u32x4* __restrict__ x, int T, int H8, RowMap rm, u32x4* __restrict__ recv_x,
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int K, int E,
    int P, int64_t* __restrict__ recv_topk_idx, float* __restrict__ recv_topk_weights) {
    const int lane = threadIdx.x & 63;
    const int t = wave_token();
    if (t >= T) return;
    const Dest d = token_rows(rm, t, lane);
    const u32x4* src = x + (int64_t)t * H8;

    for (int base = 0; base < H8; base += CPL * 64) {
        u32x4 v[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = base + i * 64 + lane;
            if (c < H8) v[i] = __builtin_nontemporal_load(src + c);
        }
        uint64_t m = d.mask;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int row = __builtin_amdgcn_readlane(d.row, r);
            u32x4* dst = recv_x + (int64_t)row * H8;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < H8) __builtin_nontemporal_store(v[i], dst + c);
            }
        }
    }

    if (recv_topk_idx != nullptr && lane < K) {
        const int64_t e = topk_idx[(int64_t)t * K + lane];
        const float w = topk_weights ? topk_weights[(int64_t)t * K + lane] : 0.0f;
        const int eb = (e >= 0 && e < E) ? (int)e / P : -1;
        uint64_t m = d.mask;
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
                                                       RowMap rm, u32x2* __restrict__ recv_x8,
                                                       float* __restrict__ recv_scales) {
    const int lane = threadIdx.x & 63;
    const int t = wave_token();
    if (t >= T) return;
    const Dest d = token_rows(rm, t, lane);
    const u32x4* src = x + (int64_t)t * H8;
    const int G = H8 >> 4;  // blocks per row

    for (int base = 0; base < H8; base += CPL * 64) {
        u32x2 code[CPL];
        float scale[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = base + i * 64 + lane;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < H8) v = __builtin_nontemporal_load(src + c);
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
        uint64_t m = d.mask;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t row = __builtin_amdgcn_readlane(d.row, r);
            u32x2* dst = recv_x8 + row * H8;
            float* sdst = recv_scales + row * G;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < H8) {
                    __builtin_nontemporal_store(code[i], dst + c);
                    if ((lane & 15) == 0) sdst[c >> 4] = scale[i];
                }
            }
        }
    }
}

int pick_cpl(int H8) {
    const int need = (H8 + 63) / 64;
    if (need <= 1) return 1;
    if (need <= 2) return 2;
    if (need <= 4) return 4;
    if (need <= 8) return 8;
    if (need <= 14) return 14;
    return 16;
}

}  // namespace

hipError_t launch_pack_bf16(const void* x, int T, int H, const RowMap& rm, void* recv_x,
                            const int64_t* topk_idx, const float* topk_weights, int K, int E, int P,
                            int64_t* recv_topk_idx, float* recv_topk_weights, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int H8 = H / 8;
    const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* rx = static_cast<u32x4*>(recv_x);
#define MOEDX_PACK(N)                                                                          \
    pack_bf16_kernel<N><<<blocks, 256, 0, stream>>>(xs, T, H8, rm, rx, topk_idx, topk_weights, \
                                                    K, E, P, recv_topk_idx, recv_topk_weights)
    switch (pick_cpl(H8)) {
        case 1: MOEDX_PACK(1); break;
        case 2: MOEDX_PACK(2); break;
        case 4: MOEDX_PACK(4); break;
        case 8: MOEDX_PACK(8); break;
        case 14: MOEDX_PACK(14); break;
        default: MOEDX_PACK(16); break;
    }
#undef MOEDX_PACK
    return hipGetLastError();
}

hipError_t launch_pack_fp8(const void* x, int T, int H, const RowMap& rm, void* recv_x8,
                           float* recv_scales, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int H8 = H / 8;
    const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* rx = static_cast<u32x2*>(recv_x8);
#define MOEDX_PACK8(N) \
    pack_fp8_kernel<N><<<blocks, 256, 0, stream>>>(xs, T, H8, rm, rx, recv_scales)
    switch (pick_cpl(H8)) {
        case 1: MOEDX_PACK8(1); break;
        case 2: MOEDX_PACK8(2); break;
        case 4: MOEDX_PACK8(4); break;
        case 8: MOEDX_PACK8(8); break;
        case 14: MOEDX_PACK8(14); break;
        default: MOEDX_PACK8(16); break;
    }
#undef MOEDX_PACK8
    return hipGetLastError();
}

}  // namespace moedx
