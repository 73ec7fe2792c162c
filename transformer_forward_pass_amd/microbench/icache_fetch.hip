// icache_fetch.hip -- what instruction fetch adds to a short kernel.
//
// Kernels that run straight-line s_nop bodies of 16 KB and 64 KB (the
// assembler emits 16 bytes per statement here), one workgroup or 256, timed
// with HIP events stamped at each kernel's start and end:
//   - warm: the same kernel has just run;
//   - after another kernel with its own body of the same size;
//   - an empty kernel, the floor of a launch on this GPU.
//
// build: hipcc -O3 --offload-arch=gfx950 -o icache_fetch icache_fetch.hip
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdio>
#include <cstdlib>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); exit(1); } } while (0)
#define N1 asm volatile("s_nop 0");
#define N8 N1 N1 N1 N1 N1 N1 N1 N1
#define N64 N8 N8 N8 N8 N8 N8 N8 N8
#define N512 N64 N64 N64 N64 N64 N64 N64 N64
#define N4K N512 N512 N512 N512 N512 N512 N512 N512
__global__ void k_codeA(int* out) { N4K if (threadIdx.x == 0 && blockIdx.x == 0) out[0] = 1; }
__global__ void k_codeB(int* out) { N4K N1 if (threadIdx.x == 0 && blockIdx.x == 0) out[1] = 2; }
#define N1K N512 N512
__global__ void k_codeC(int* out) { N1K if (threadIdx.x == 0 && blockIdx.x == 0) out[3] = 1; }
__global__ void k_codeD(int* out) { N1K N1 if (threadIdx.x == 0 && blockIdx.x == 0) out[4] = 2; }
__global__ void k_tiny(int* out) { if (threadIdx.x == 0 && blockIdx.x == 0) out[2] = 3; }

int main()
{
    int* out;
    CK(hipMalloc(&out, 64));
    hipStream_t s; CK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    auto timed = [&](void (*k)(int*), int blocks) {
        hipExtLaunchKernelGGL(k, dim3(blocks), dim3(64), 0, s, e0, e1, 0, out);
        CK(hipEventSynchronize(e1)); float ms; CK(hipEventElapsedTime(&ms, e0, e1)); return ms * 1000.f;
    };
    for (int blocks : {1, 256}) {
        double tiny = 0, warm = 0, cold = 0, warm16 = 0, cold16 = 0;
        const int R = 50;
        for (int r = 0; r < R; r++) {
            tiny += timed(k_tiny, blocks);
            hipLaunchKernelGGL(k_codeA, dim3(blocks), dim3(64), 0, s, out);
            warm += timed(k_codeA, blocks);
            hipLaunchKernelGGL(k_codeB, dim3(blocks), dim3(64), 0, s, out);
            cold += timed(k_codeA, blocks);
            hipLaunchKernelGGL(k_codeC, dim3(blocks), dim3(64), 0, s, out);
            warm16 += timed(k_codeC, blocks);
            hipLaunchKernelGGL(k_codeD, dim3(blocks), dim3(64), 0, s, out);
            cold16 += timed(k_codeC, blocks);
        }
        printf("blocks %3d: tiny kernel %.2f us | 64 KB body: warm %.2f us, after another 64 KB kernel %.2f us | 16 KB body: warm %.2f, after another %.2f us\n",
               blocks, tiny / R, warm / R, cold / R, warm16 / R, cold16 / R);
    }
    return 0;
}
