// bf16_convert.hip -- checks that gfx950's hardware fp32 -> bf16 conversion
// (v_cvt_pk_bf16_f32, which f2bf in csrc/device_math.h uses) rounds every
// fp32 bit pattern exactly as the integer round-to-nearest-even rule
// bf16 = (u + 0x7fff + ((u >> 16) & 1)) >> 16, NaN -> (u >> 16) | 0x40,
// that the CPU oracle applies.  All 2^32 inputs, one pass.
//
// build: hipcc -O3 --offload-arch=gfx950 -o bf16_convert bf16_convert.hip
// usage: bf16_convert
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>

#include "../csrc/device_math.h"

#define CK(x)                                                                                   \
    do {                                                                                        \
        hipError_t err_ = (x);                                                                  \
        if (err_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(err_)); \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

// the integer rule, written out independently of the library's function
__device__ __forceinline__ uint16_t rne_bits(uint32_t u)
{
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

constexpr uint32_t kThreads = 256, kPerThread = 256;
constexpr uint32_t kBlocks = (uint32_t)((1ull << 32) / ((uint64_t)kThreads * kPerThread));   // 65536
constexpr int kKeep = 16;

// cnt[0] non-NaN mismatches, cnt[1] NaN mismatches, cnt[2] recorded; bad[] the first inputs
__global__ void check(unsigned long long* cnt, uint32_t* bad)
{
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPerThread;
    unsigned long long n_num = 0, n_nan = 0;
    for (uint32_t i = 0; i < kPerThread; i++) {
        const uint32_t u = (uint32_t)(base + i);
        if (mak::f2bf(__uint_as_float(u)) != rne_bits(u)) {
            if ((u & 0x7fffffffu) > 0x7f800000u) {
                n_nan++;
            } else {
                n_num++;
                const unsigned long long slot = atomicAdd(&cnt[2], 1ull);
                if (slot < kKeep) bad[slot] = u;
            }
        }
    }
    if (n_num) atomicAdd(&cnt[0], n_num);
    if (n_nan) atomicAdd(&cnt[1], n_nan);
}

int main()
{
    unsigned long long* cnt;
    uint32_t* bad;
    CK(hipMalloc(&cnt, 3 * sizeof(unsigned long long)));
    CK(hipMalloc(&bad, kKeep * sizeof(uint32_t)));
    CK(hipMemset(cnt, 0, 3 * sizeof(unsigned long long)));
    CK(hipMemset(bad, 0, kKeep * sizeof(uint32_t)));
    hipLaunchKernelGGL(check, dim3(kBlocks), dim3(kThreads), 0, 0, cnt, bad);
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    unsigned long long h[3];
    uint32_t hb[kKeep];
    CK(hipMemcpy(h, cnt, sizeof(h), hipMemcpyDeviceToHost));
    CK(hipMemcpy(hb, bad, sizeof(hb), hipMemcpyDeviceToHost));
    std::printf("fp32 -> bf16, all %llu inputs: non-NaN mismatches %llu, NaN mismatches %llu\n", 1ull << 32, h[0], h[1]);
    for (unsigned long long i = 0; i < h[2] && i < (unsigned long long)kKeep; i++) std::printf("  mismatch: input 0x%08x\n", hb[i]);
    CK(hipFree(cnt));
    CK(hipFree(bad));
    return (h[0] || h[1]) ? 1 : 0;
}
