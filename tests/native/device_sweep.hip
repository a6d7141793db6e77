// device_sweep.hip -- test-only: the library's device encoders over every
// finite fp32 bit pattern, reduced to the order-independent checksums that
// exhaustive.c computes from the oracle's encoders: sum of (code + 1) *
// mix(pattern) mod 2^64, mix the splitmix64 finaliser (Vigna).  The
// encoders are the kernels' own (device.hpp): E2M1 codes for the FP4
// planes [P1 §3.1; P2 四、"P4 main KV"], bf16 round-to-nearest-even for the
// window rows.  Not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void sweep_kernel(uint64_t first, uint64_t count, uint64_t *partial)
{
    __shared__ uint64_t red[2][kThreads];
    uint64_t se = 0, sb = 0;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = first + (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < first + count; i += stride) {
        const uint32_t u = (uint32_t)i;
        if ((u & 0x7F800000u) == 0x7F800000u) continue;          // inf and NaN
        const float x = __uint_as_float(u);
        const uint64_t m = mix64(u);
        se += (uint64_t)(cskv::e2m1_code(x) + 1u) * m;
        sb += (uint64_t)(cskv::bf16_bits_rne(x) + 1u) * m;
    }
    red[0][threadIdx.x] = se;
    red[1][threadIdx.x] = sb;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            red[0][threadIdx.x] += red[0][threadIdx.x + h];
            red[1][threadIdx.x] += red[1][threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x < 2) partial[2 * blockIdx.x + threadIdx.x] = red[threadIdx.x][0];
}

}  // namespace

// Checksums of patterns [first, first + count) into out[0] (E2M1) and out[1]
// (bf16); 0 on success, else the HIP error.
extern "C" int cskv_test_encoder_sweep(uint64_t first, uint64_t count, uint64_t *out)
{
    constexpr int kBlocks = 2048;
    uint64_t *d = nullptr;
    hipError_t e = hipMalloc(&d, sizeof(uint64_t) * 2 * kBlocks);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(sweep_kernel, dim3(kBlocks), dim3(kThreads), 0, 0, first, count, d);
    uint64_t h[2 * kBlocks];
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
    (void)hipFree(d);
    if (e != hipSuccess) return (int)e;
    out[0] = out[1] = 0;
    for (int i = 0; i < kBlocks; ++i) {
        out[0] += h[2 * i];
        out[1] += h[2 * i + 1];
    }
    return 0;
}
