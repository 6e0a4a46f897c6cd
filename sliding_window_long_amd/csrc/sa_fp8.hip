// sa_fp8.hip -- FP8 inputs: exact decoding of OCP E4M3 values into bf16.
//
// [Naive-N0.5-Flash page: the model runs FP8 mixed-precision inference.]
// E4M3 (bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN) holds
// normal values 2^-6 .. 448 and subnormals m * 2^-9; every one of them is a
// bf16 value (8 exponent bits, 7 mantissa bits), so the decoded tensors
// carry exactly the inputs' values into the bf16 path.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// 16 fp8 values per thread -> 16 bf16 values.
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint4* __restrict__ x,
                                                          uint4* __restrict__ y, size_t n16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n16) return;
    const uint4 u = x[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[2 * t] = e4m3_to_bf16(w[t] & 0xffu) | (e4m3_to_bf16((w[t] >> 8) & 0xffu) << 16);
        o[2 * t + 1] = e4m3_to_bf16((w[t] >> 16) & 0xffu) | (e4m3_to_bf16(w[t] >> 24) << 16);
    }
    y[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
    y[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_fp8_to_bf16(const void* x, uint16_t* y, size_t n, hipStream_t s) {
    const size_t n16 = n / 16;   // every tensor holds a multiple of 16 elements
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       (const uint4*)x, (uint4*)y, n16);
    return hipGetLastError();
}

}  // namespace sa
