// q4_0 cache writer: quantizes rows of f32, f16 or bf16 elements into q4_0 blocks, e.g. the K
// and V rows of a new chunk appended to a q4_0 cache (the format the attention kernels read:
// mi210-llm-stack "FlashAttention on gfx90a", the q4_0 KV cache of its runs). Per block of 32
// elements: d = max|x| / 8 rounded to the nearest f16 (ties to even); an element's code is
// clamp(round_half_away(x / d) + 8, 0, 15) with x / d the correctly rounded f32 quotient (so
// +max|x| gives 16, clamped to 15); every code is 8 when d = 0. Byte t of the 16 code bytes holds
// element t's code (low nibble) and element t + 16's (high nibble).
//
// One thread per block: 128 (f32) or 64 bytes in as 16-byte loads, 18 bytes out as 2-byte
// stores (block starts are only 2-byte aligned). The path is HBM-bound.
#include "fa_kernels.h"
#include "fa_device.h"

namespace fa {

namespace {

struct QuantParams {
    const void *x;
    uint8_t *blocks;
    int64_t n_seq, blocks_per_seq;
    int64_t x_seq_stride;       // elements between consecutive sequences' first rows
    int64_t blk_seq_stride;     // bytes between consecutive sequences' first output rows
};

__device__ __forceinline__ uint32_t q4_code(float x, float d)
{
    if (d == 0.0f)
        return 8u;
    const int c = (int)__builtin_roundf(x / d) + 8;
    return (uint32_t)min(max(c, 0), 15);
}

template <int SRC>      // 0: f32, 1: f16, 2: bf16
__global__ __launch_bounds__(256) void quantize_q4_0_kernel(QuantParams p)
{
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= p.n_seq * p.blocks_per_seq)
        return;
    const int64_t s = id / p.blocks_per_seq, j = id % p.blocks_per_seq;
    float v[32];
    if constexpr (SRC == 0) {
        const f32x4 *src = (const f32x4 *)((const float *)p.x + s * p.x_seq_stride + 32 * j);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const f32x4 t = src[u];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[4 * u + e] = t[e];
        }
    } else {
        const u32x4 *src = (const u32x4 *)((const uint16_t *)p.x + s * p.x_seq_stride + 32 * j);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 t = src[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (SRC == 1) {
                    const f32x2 f = unpack2<false>(t[e]);
                    v[8 * u + 2 * e] = f[0];
                    v[8 * u + 2 * e + 1] = f[1];
                } else {
                    v[8 * u + 2 * e] = __builtin_bit_cast(float, t[e] << 16);
                    v[8 * u + 2 * e + 1] = __builtin_bit_cast(float, t[e] & 0xFFFF0000u);
                }
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t)
        amax = fmaxf(amax, fabsf(v[t]));
    const _Float16 dh = (_Float16)(amax * 0.125f);      // exact quotient, then RNE to f16
    const float d = (float)dh;
    uint32_t code4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t byte = q4_code(v[t], d) | (q4_code(v[t + 16], d) << 4);
        code4[t / 4] |= byte << (8 * (t % 4));
    }
    uint16_t *dst = (uint16_t *)(p.blocks + s * p.blk_seq_stride + 18 * j);
    dst[0] = __builtin_bit_cast(uint16_t, dh);
#pragma unroll
    for (int m = 0; m < 8; ++m)
        dst[1 + m] = (uint16_t)(code4[m / 2] >> (16 * (m % 2)));
}

}  // namespace

hipError_t launch_quantize_q4_0(const void *x, int src, void *blocks, int64_t n_seq,
                                int64_t blocks_per_seq, int64_t x_seq_stride,
                                int64_t blk_seq_stride, hipStream_t stream)
{
    const int64_t total = n_seq * blocks_per_seq;
    if (total == 0)
        return hipSuccess;
    const QuantParams p{x, (uint8_t *)blocks, n_seq, blocks_per_seq, x_seq_stride,
                        blk_seq_stride};
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (src == 0)
        hipLaunchKernelGGL(quantize_q4_0_kernel<0>, grid, block, 0, stream, p);
    else if (src == 1)
        hipLaunchKernelGGL(quantize_q4_0_kernel<1>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(quantize_q4_0_kernel<2>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
