// Measurement export: a plain streaming read of a device buffer, the HBM read rate the decode
// kernels are compared with. Each thread keeps four 16-byte loads in flight per iteration over
// a grid-strided range and folds what it read into one word, which is stored only if it equals
// a value the caller passes (so the loads cannot be dropped and nothing else is written).
#include "fa_kernels.h"
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4 *buf, int64_t n16,
                                                           uint32_t *sink, uint32_t magic)
{
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (x == magic)
        *sink = x;
}

}  // namespace

hipError_t launch_read(const void *buf, int64_t n16, uint32_t *sink, uint32_t magic, int grid,
                       hipStream_t stream)
{
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, stream,
                       (const u32x4 *)buf, n16, sink, magic);
    return hipGetLastError();
}

}  // namespace fa
