// Combine kernel for gfx950: the weighted gather-reduce of receive rows back
// to token order.
//
// combine_forward in the normal-kernel example of the EnflameTechnology/DeepEP
// README reduces the rows a token was sent to back into one row, and its
// dispatch_backward reduces the top-k weight payload the same way; the
// handle-reuse page ("Combining with Handle Reuse") runs it from the cached
// handle.  Here each token gathers the rows of its distinct buckets, in the
// order those buckets first occur among its top-k slots, scales each by the
// bucket's summed gate weight and accumulates in fp32 with fused multiply-adds
// from +0.0, then rounds once to bf16 (nearest even).
//
// Design (HBM-bound, no MFMA): one wavefront per token.  Lanes 0..K-1 hold the
// token's slots; first occurrence, the per-bucket weight and the row index are
// computed with lane reads, so every visited row, its weight and its address
// are wave-uniform.  Each pass loads CPL 16-byte chunks per lane of one row
// before the FMAs, and the visit order is fixed, so the result does not depend
// on the launch shape.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moedx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CPL>
__global__ __launch_bounds__(256) void combine_kernel(
    const u32x4* __restrict__ y, int T, int H8, int K, RowMap rm,
    const int8_t* __restrict__ slot_bucket, const float* __restrict__ gate_weights,
    const float* __restrict__ recv_topk_weights, u32x4* __restrict__ out,
    float* __restrict__ combined_topk_weights) {
    const int lane = threadIdx.x & 63;
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
    if (t >= T) return;

    int rk = -1;
    float wk = 0.0f;
    if (lane < K) {
        rk = slot_bucket[(int64_t)t * K + lane];
        if (gate_weights) wk = gate_weights[(int64_t)t * K + lane];
    }
    // A slot is visited if it is the first slot of its bucket; its weight is the
    // sum, in ascending slot order from +0.0, of the gate weights of its bucket.
    bool first = rk >= 0;
    float om = 0.0f;
    for (int kk = 0; kk < K; ++kk) {
        const int r2 = __builtin_amdgcn_readlane(rk, kk);
        const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), kk));
        if (r2 == rk) {
            if (kk < lane) first = false;
            om = om + w2;
        }
    }
    if (!gate_weights) om = 1.0f;
    int row = -1;
    if (first) {
        row = rm.rank_prefix_matrix[rk] - rm.num_tokens_per_rank[rk] +
              rm.send_head[(int64_t)t * rm.R + rk];
    }
    const uint64_t visits = __ballot(first);

    u32x4* dst = out + (int64_t)t * H8;
    for (int base = 0; base < H8; base += CPL * 64) {
        float acc[CPL][8];
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
        uint64_t m = visits;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t r = __builtin_amdgcn_readlane(row, k);
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(om), k));
            const u32x4* src = y + r * H8;
            u32x4 v[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < H8) v[i] = __builtin_nontemporal_load(src + c);
            }
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = base + i * 64 + lane;
                if (c < H8) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][2 * j] = __builtin_fmaf(w, bf16_lo(v[i][j]), acc[i][2 * j]);
                        acc[i][2 * j + 1] = __builtin_fmaf(w, bf16_hi(v[i][j]), acc[i][2 * j + 1]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = base + i * 64 + lane;
            if (c < H8) {
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = bf16_bits(acc[i][2 * j]) | (bf16_bits(acc[i][2 * j + 1]) << 16);
                __builtin_nontemporal_store(o, dst + c);
            }
        }
    }

    if (combined_topk_weights != nullptr && recv_topk_weights != nullptr && lane < K) {
        float s = 0.0f;
        uint64_t m = visits;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int64_t r = __builtin_amdgcn_readlane(row, k);
            s = s + recv_topk_weights[r * K + lane];
        }
        combined_topk_weights[(int64_t)t * K + lane] = s;
    }
}

int pick_cpl(int H8) {
    const int need = (H8 + 63) / 64;
    if (need <= 1) return 1;
    if (need <= 2) return 2;
    if (need <= 4) return 4;
    if (need <= 7) return 7;  // 7168 / 8 / 64 = 14 -> two passes of 7
    if (need <= 8) return 8;
    if (need <= 14) return 7;
    return 8;
}

}  // namespace

hipError_t launch_combine(const void* y, int T, int H, int K, const RowMap& rm,
                          const int8_t* slot_bucket, const float* gate_weights,
                          const float* recv_topk_weights, void* out,
                          float* combined_topk_weights, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int H8 = H / 8;
    const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    const u32x4* ys = static_cast<const u32x4*>(y);
    u32x4* os = static_cast<u32x4*>(out);
#define MOEDX_COMBINE(N)                                                                    \
    combine_kernel<N><<<blocks, 256, 0, stream>>>(ys, T, H8, K, rm, slot_bucket, gate_weights, \
                                                  recv_topk_weights, os, combined_topk_weights)
    switch (pick_cpl(H8)) {
        case 1: MOEDX_COMBINE(1); break;
        case 2: MOEDX_COMBINE(2); break;
        case 4: MOEDX_COMBINE(4); break;
        case 7: MOEDX_COMBINE(7); break;
        default: MOEDX_COMBINE(8); break;
    }
#undef MOEDX_COMBINE
    return hipGetLastError();
}

}  // namespace moedx
