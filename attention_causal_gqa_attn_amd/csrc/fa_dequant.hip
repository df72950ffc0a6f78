// q4_0 dequantization export: runs the same unpack routine the attention kernels use to fill
// their K tiles, so its output shows bit for bit what values enter the MFMAs.
#include "fa_kernels.h"
#include "fa_device.h"

namespace fa {

namespace {

// One thread per 18-byte block (2-byte aligned: read as 9 halfwords).
__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint16_t *blocks, int64_t n,
                                                          float *out_f32, uint32_t *out_f16)
{
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= n)
        return;
    const uint16_t *src = blocks + 9 * blk;
    uint16_t hw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i)
        hw[i] = src[i];
    const uint32_t dbits = hw[0];
    uint32_t codes[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        codes[g] = (uint32_t)hw[1 + 2 * g] | ((uint32_t)hw[2 + 2 * g] << 16);

    if (out_f16) {
        const uint32_t d2 = dbits * 0x10001u;
        uint32_t lo[4][2], hi[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            q4_unpack_row(codes[g], d2, lo[g], hi[g]);
        uint32_t *dst = out_f16 + 16 * blk;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            dst[2 * g] = lo[g][0];
            dst[2 * g + 1] = lo[g][1];
            dst[8 + 2 * g] = hi[g][0];
            dst[8 + 2 * g + 1] = hi[g][1];
        }
    }
    if (out_f32) {
        const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits);
        float *dst = out_f32 + 32 * blk;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t byte = (codes[g] >> (8 * j)) & 0xFFu;
                dst[4 * g + j] = (float)((int)(byte & 15u) - 8) * d;
                dst[16 + 4 * g + j] = (float)((int)(byte >> 4) - 8) * d;
            }
    }
}

}  // namespace

hipError_t launch_dequant_q4_0(const void *blocks, int64_t n_blocks, float *out_f32,
                               void *out_f16, hipStream_t stream)
{
    if (n_blocks == 0)
        return hipSuccess;
    const int64_t grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(dequant_q4_0_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint16_t *)blocks, n_blocks, out_f32, (uint32_t *)out_f16);
    return hipGetLastError();
}

}  // namespace fa
