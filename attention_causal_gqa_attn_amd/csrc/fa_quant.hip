// q4_0 cache writer: quantizes rows of f32, f16 or bf16 elements into q4_0 blocks, e.g. the K
// and V rows of a new chunk appended to a q4_0 cache (the format the attention kernels read:
// mi210-llm-stack "FlashAttention on gfx90a", the q4_0 KV cache of its runs). Per block of 32
// elements: d = max|x| / 8 rounded to the nearest f16 (ties to even); an element's code is
// clamp(round_half_away(x / d) + 8, 0, 15) with x / d the correctly rounded f32 quotient (so
// +max|x| gives 16, clamped to 15); every code is 8 when d = 0. Byte t of the 16 code bytes holds
// element t's code (low nibble) and element t + 16's (high nibble).
//
// One thread per block: 128 (f32) or 64 bytes in as 16-byte loads. A wave's 64 consecutive
// blocks are 1152 contiguous output bytes when they belong to one sequence: they are staged in
// LDS and written as one run of 16-byte, 4-byte or 2-byte stores (whichever the run's start
// address allows; block starts are only 2-byte aligned), every store instruction covering
// consecutive bytes. A wave whose blocks straddle two sequences writes each block's 18 bytes
// itself. The path is HBM-bound.
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

// The same code without a full division per element: with r = RN(1 / d) (one correctly rounded
// division per block), q0 = RN(x r), the residual e = x - q0 d (exact, one fma) and
// q1 = RN(q0 + e r) (one fma) is the correctly rounded quotient RN(x / d) (Markstein's
// theorem on division by a correctly rounded reciprocal, round to nearest). Here x / d stays in
// [-8.004, 8.004] and d is a positive f16 value, so no step over- or underflows; the argument
// needs x and q0 d away from the subnormal range, which the exact fallback below covers
// (|x| < 2^-100: the code is 8 either way unless d is as small, checked by the caller).
// |q1| <= 8.004 also bounds the rounded value by 8, so the code is never below 0 and only
// +max|x| (16) needs the clamp.
// Rounding half away from zero: for f16 and bf16 sources v_cvt_rpi_i32_f32 (floor(s + 0.5))
// of |q1|, the sign put back as (r ^ s) - s with s = 0 or -1. That is exact even if the
// instruction rounds s + 0.5 to f32 first: such a rounding can move the floor only when
// s + 0.5 lies within half an ulp below an integer, which for |q1| <= 8.004 needs
// 0.5 - 2^-25 < |q1| < 0.5, and a quotient of two 16-bit values (x f16 or bf16, d f16 and
// normal) that is not 0.5 differs from it by at least 2^-11 relative (2x and d lie on the grid
// of d's ulp). An f32 x can come that close, so f32 sources round with roundf.
template <int SRC>
__device__ __forceinline__ uint32_t q4_code_r(float x, float d, float r)
{
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, d, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    int c;
    if constexpr (SRC == 0) {
        c = (int)__builtin_roundf(q1) + 8;
    } else {
        int m;
        asm("v_cvt_rpi_i32_f32 %0, |%1|" : "=v"(m) : "v"(q1));
        const int sg = (int)__builtin_bit_cast(uint32_t, q1) >> 31;
        c = (m ^ sg) - sg + 8;
    }
    return (uint32_t)min(c, 15);
}

template <int SRC>      // 0: f32, 1: f16, 2: bf16
__global__ __launch_bounds__(256) void quantize_q4_0_kernel(QuantParams p)
{
    __shared__ __attribute__((aligned(16))) uint16_t stage[4][64 * 9];   // a wave's 64 blocks
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t total = p.n_seq * p.blocks_per_seq;
    const int64_t id0 = ((int64_t)blockIdx.x * blockDim.x) + 64 * wave;  // the wave's first block
    if (id0 >= total)
        return;                                    // whole wave
    const int64_t id = min(id0 + lane, total - 1); // lanes past the end redo the last block
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
    if (d >= 0x1p-14f) {                                // a normal f16 scale: no subnormal steps
        const float r = 1.0f / d;                       // correctly rounded
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t byte =
                q4_code_r<SRC>(v[t], d, r) | (q4_code_r<SRC>(v[t + 16], d, r) << 4);
            code4[t / 4] |= byte << (8 * (t % 4));
        }
    } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t byte = q4_code(v[t], d) | (q4_code(v[t + 16], d) << 4);
            code4[t / 4] |= byte << (8 * (t % 4));
        }
    }
    uint16_t out[9];
    out[0] = __builtin_bit_cast(uint16_t, dh);
#pragma unroll
    for (int m = 0; m < 8; ++m)
        out[1 + m] = (uint16_t)(code4[m / 2] >> (16 * (m % 2)));

    // the wave's blocks [id0, id0 + n): one output run if they lie in one sequence
    const int n = (int)min((int64_t)64, total - id0);
    const int64_t s0 = id0 / p.blocks_per_seq, j0 = id0 % p.blocks_per_seq;
    if (j0 + n > p.blocks_per_seq) {
        if (id0 + lane < total) {
            uint16_t *dst = (uint16_t *)(p.blocks + s * p.blk_seq_stride + 18 * j);
#pragma unroll
            for (int m = 0; m < 9; ++m)
                dst[m] = out[m];
        }
        return;
    }
    uint16_t *st = stage[wave];
#pragma unroll
    for (int m = 0; m < 9; ++m)
        st[9 * lane + m] = out[m];
    // other lanes' staged bytes are read next: the wave's LDS writes complete first, and the
    // clobber keeps the compiler from moving the reads above them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint8_t *run = p.blocks + s0 * p.blk_seq_stride + 18 * j0;
    const int bytes = 18 * n;
    if (((uintptr_t)run & 15) == 0) {
        for (int o = 16 * lane; o + 16 <= bytes; o += 16 * 64)
            *(u32x4 *)(run + o) = *(const u32x4 *)((const uint8_t *)st + o);
        const int tail = bytes & ~15;               // n odd: the last 2-byte pieces
        for (int o = tail + 2 * lane; o < bytes; o += 2 * 64)
            *(uint16_t *)(run + o) = *(const uint16_t *)((const uint8_t *)st + o);
    } else if (((uintptr_t)run & 3) == 0) {
        for (int o = 4 * lane; o + 4 <= bytes; o += 4 * 64)
            *(uint32_t *)(run + o) = *(const uint32_t *)((const uint8_t *)st + o);
        const int tail = bytes & ~3;
        for (int o = tail + 2 * lane; o < bytes; o += 2 * 64)
            *(uint16_t *)(run + o) = *(const uint16_t *)((const uint8_t *)st + o);
    } else {
        for (int o = 2 * lane; o < bytes; o += 2 * 64)
            *(uint16_t *)(run + o) = *(const uint16_t *)((const uint8_t *)st + o);
    }
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
