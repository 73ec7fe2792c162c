// fp64_mfma.hip -- sustained rate of gfx950's two fp64 matrix instructions:
// v_mfma_f64_16x16x4_f64 (one 16x16 tile, 1024 multiply-adds per wave
// instruction) and v_mfma_f64_4x4x4_4b_f64 (four independent 4x4 tiles, 256).
// Every wave runs independent accumulator chains so that no instruction
// waits on the previous one's result; 2048 workgroups of four waves fill
// every SIMD several times over.  Three passes each, HIP-event timed.
//
// build: hipcc -O3 --offload-arch=gfx950 -o fp64_mfma fp64_mfma.hip
// usage: fp64_mfma
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

typedef double d4_t __attribute__((ext_vector_type(4)));
constexpr int kIter = 2000;
constexpr int kBlocks = 2048;   // of 256 threads

__global__ __launch_bounds__(256) void k_16x16(const double* in, double* out)
{
    const int l = threadIdx.x & 63;
    const double a = in[l], b = in[64 + l];
    d4_t c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < kIter; i++) {
        c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c3, 0, 0, 0);
    }
    const d4_t s = c0 + c1 + c2 + c3;
    out[blockIdx.x * 256 + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void k_4x4(const double* in, double* out)
{
    const int l = threadIdx.x & 63;
    const double a = in[l], b = in[64 + l];
    double c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < kIter; i++) {
#pragma unroll
        for (int j = 0; j < 8; j++) c[j] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, b, c[j], 0, 0, 0);
    }
    double s = 0.0;
    for (int j = 0; j < 8; j++) s += c[j];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

int main()
{
    double *in, *out;
    CK(hipMalloc(&in, 128 * sizeof(double)));
    CK(hipMalloc(&out, (size_t)kBlocks * 256 * sizeof(double)));
    CK(hipMemset(in, 0, 128 * sizeof(double)));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    const double waves = kBlocks * 4.0;
    for (int rep = 0; rep < 3; rep++) {
        float ms16 = 0.f, ms4 = 0.f;
        CK(hipEventRecord(e0));
        k_16x16<<<kBlocks, 256>>>(in, out);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        CK(hipEventElapsedTime(&ms16, e0, e1));
        CK(hipEventRecord(e0));
        k_4x4<<<kBlocks, 256>>>(in, out);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        CK(hipEventElapsedTime(&ms4, e0, e1));
        const double f16 = waves * kIter * 4 * 1024 * 2.0, f4 = waves * kIter * 8 * 256 * 2.0;
        std::printf("v_mfma_f64_16x16x4_f64: %.3f ms, %.1f TFLOP/s   v_mfma_f64_4x4x4_4b_f64: %.3f ms, %.1f TFLOP/s\n",
                    ms16, f16 / ms16 / 1e9, ms4, f4 / ms4 / 1e9);
    }
    CK(hipGetLastError());
    CK(hipFree(in));
    CK(hipFree(out));
    return 0;
}
