// combine.hip -- y += x over a flat array (the sum of the forward and reverse
// outputs of a bidirectional call).  Plain streaming: 16-byte vectors when both
// arrays are aligned, a grid-stride loop sized to fill the chip.
#include "combine.h"
#include "common.h"

namespace drs {

namespace {

constexpr int kAddThreads = 256;

__global__ __launch_bounds__(kAddThreads) void add_f32(float *y, const float *x, size_t n, int vec) {
    const size_t stride = (size_t)gridDim.x * kAddThreads;
    size_t i = (size_t)blockIdx.x * kAddThreads + threadIdx.x;
    if (vec) {
        const size_t nv = n / 4;
        f32x4 *y4 = reinterpret_cast<f32x4 *>(y);
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
        for (size_t j = i; j < nv; j += stride) y4[j] = y4[j] + x4[j];
        for (size_t j = nv * 4 + i; j < n; j += stride) y[j] += x[j];
    } else {
        for (size_t j = i; j < n; j += stride) y[j] += x[j];
    }
}

__global__ __launch_bounds__(kAddThreads) void add_bf16(uint16_t *y, const uint16_t *x, size_t n, int vec) {
    const size_t stride = (size_t)gridDim.x * kAddThreads;
    size_t i = (size_t)blockIdx.x * kAddThreads + threadIdx.x;
    size_t done = 0;
    if (vec) {
        const size_t nv = n / 8;
        u32x4 *y4 = reinterpret_cast<u32x4 *>(y);
        const u32x4 *x4 = reinterpret_cast<const u32x4 *>(x);
        for (size_t j = i; j < nv; j += stride) {
            const u32x4 a = y4[j], b = x4[j];
            u32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = pack_bf16x2(bf16_lo(a[r]) + bf16_lo(b[r]), bf16_hi(a[r]) + bf16_hi(b[r]));
            y4[j] = o;
        }
        done = nv * 8;
    }
    for (size_t j = done + i; j < n; j += stride)
        y[j] = f32_to_bf16_bits(bf16_bits_to_f32(y[j]) + bf16_bits_to_f32(x[j]));
}

}  // namespace

hipError_t add_into_launch(void *y, const void *x, size_t n, bool bf16, bool vec, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const size_t per = (size_t)kAddThreads * (bf16 ? 8 : 4);
    size_t blocks = (n + per - 1) / per;
    if (blocks > 8192) blocks = 8192;
    if (bf16)
        hipLaunchKernelGGL(add_bf16, dim3((unsigned)blocks), dim3(kAddThreads), 0, stream,
                           static_cast<uint16_t *>(y), static_cast<const uint16_t *>(x), n, vec ? 1 : 0);
    else
        hipLaunchKernelGGL(add_f32, dim3((unsigned)blocks), dim3(kAddThreads), 0, stream, static_cast<float *>(y),
                           static_cast<const float *>(x), n, vec ? 1 : 0);
    return hipGetLastError();
}

}  // namespace drs
