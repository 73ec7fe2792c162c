// copy_calib.hip -- a plain copy of a known number of bytes, to calibrate
// the HBM traffic counters (FETCH_SIZE, WRITE_SIZE) against: one launch
// reads exactly `bytes` and writes exactly `bytes`.
//
// build: hipcc -O3 --offload-arch=gfx950 -o copy_calib copy_calib.hip
// usage: copy_calib [MiB=256] [launches=3]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                                   \
    do {                                                                                        \
        hipError_t err_ = (x);                                                                  \
        if (err_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(err_)); \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int main(int argc, char** argv)
{
    const size_t mib = argc > 1 ? (size_t)atoi(argv[1]) : 256;
    const int launches = argc > 2 ? atoi(argv[2]) : 3;
    const size_t bytes = mib << 20, n16 = bytes / 16;
    uint4 *src, *dst;
    CK(hipMalloc(&src, bytes));
    CK(hipMalloc(&dst, bytes));
    CK(hipMemset(src, 3, bytes));
    CK(hipDeviceSynchronize());
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    for (int i = 0; i < launches; i++) {
        CK(hipEventRecord(a, 0));
        hipLaunchKernelGGL(k_copy, dim3(1024), dim3(256), 0, 0, src, dst, n16);
        CK(hipEventRecord(b, 0));
        CK(hipEventSynchronize(b));
        float ms;
        CK(hipEventElapsedTime(&ms, a, b));
        std::printf("copy %zu MiB: %.3f ms, %.1f GB/s (read+write)\n", mib, ms, 2.0 * bytes / ms / 1e6);
    }
    return 0;
}
