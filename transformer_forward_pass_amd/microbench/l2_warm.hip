// l2_warm.hip -- does data read by one kernel help the next kernel that
// reads it again?
//
// Kernel B (workgroup b reads 16 KB tile b) is timed with HIP events stamped
// at its own start and end, after a 1 GB stream has evicted everything, and:
//   1. nothing else (cold);
//   2. kernel A reading the same tiles from the same workgroups, which are
//      dispatched to the same XCD (round-robin over 8: blockIdx mod 8), or
//      from workgroups 8 apart (also the same XCD);
//   3. kernel A reading them from the neighbouring XCD.
// It sizes what a kernel with one dependent read of a few KB per workgroup
// costs, and whether prefetching the next kernel's weights into an XCD's L2
// could shorten it.
//
// build: hipcc -O3 --offload-arch=gfx950 -o l2_warm l2_warm.hip
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdio>
#include <cstdlib>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); exit(1); } } while (0)

constexpr int TILE16 = 1024;   // 16 KB tile = 1024 uint4; 256 threads x 4 loads

__global__ __launch_bounds__(256) void k_tile(const uint4* __restrict__ x, int n_tiles, int shift, uint4* out)
{
    const int t = (blockIdx.x + shift) % n_tiles;
    const uint4* p = x + (size_t)t * TILE16 + threadIdx.x;
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = p[k * 256];
    uint4 a = v[0];
#pragma unroll
    for (int k = 1; k < 4; k++) { a.x ^= v[k].x; a.y ^= v[k].y; a.z ^= v[k].z; a.w ^= v[k].w; }
    if (a.x == 0x12345678u && a.y == 0x9abcdef0u) out[0] = a;
}

__global__ __launch_bounds__(512) void k_stream(const uint4* __restrict__ src, size_t n16, uint4* out)
{
    uint4 a = make_uint4(0, 0, 0, 0);
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
        uint4 v = src[i];
        a.x ^= v.x; a.y ^= v.y; a.z ^= v.z; a.w ^= v.w;
    }
    if (a.x == 0x12345678u && a.y == 0x9abcdef0u) out[0] = a;
}

int main()
{
    const size_t MAXT = 256, X = MAXT * TILE16 * 16, BIG = 1ull << 30;
    uint4 *x, *big, *out;
    CK(hipMalloc(&x, X)); CK(hipMalloc(&big, BIG)); CK(hipMalloc(&out, 64));
    CK(hipMemset(x, 1, X)); CK(hipMemset(big, 2, BIG));
    hipStream_t s; CK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    auto timed = [&](int n, int shift) {
        hipExtLaunchKernelGGL(k_tile, dim3(n), dim3(256), 0, s, e0, e1, 0, (const uint4*)x, n, shift, out);
        CK(hipEventSynchronize(e1)); float ms; CK(hipEventElapsedTime(&ms, e0, e1)); return ms * 1000.f;
    };
    auto cold = [&]() { hipLaunchKernelGGL(k_stream, dim3(2048), dim3(512), 0, s, (const uint4*)big, BIG / 16, out); };
    auto pre = [&](int n, int shift) { hipLaunchKernelGGL(k_tile, dim3(n), dim3(256), 0, s, (const uint4*)x, n, shift, out); };
    for (int n : {64, 128, 256}) {
        double c = 0, w0 = 0, w8 = 0, w1 = 0, ww = 0;
        const int R = 20;
        for (int r = 0; r < R; r++) {
            cold(); c += timed(n, 0);
            cold(); pre(n, 0); w0 += timed(n, 0);     // same workgroups, same XCD
            cold(); pre(n, 8); w8 += timed(n, 0);     // other workgroups, same XCD
            cold(); pre(n, 1); w1 += timed(n, 0);     // other XCD
            cold(); pre(n, 0); pre(n, 1); ww += timed(n, 0);   // both
        }
        printf("tiles %3d (%4d KB): cold %.2f us | warm same XCD %.2f us (shift 8: %.2f) | warm other XCD %.2f us | both %.2f us\n",
               n, n * 16, c / R, w0 / R, w8 / R, w1 / R, ww / R);
    }
    return 0;
}
