// mem_stream.hip -- what the memory system gives a decode-step GEMV.
//
// 1. dependent-load latency (one lane chasing a random cycle) for a footprint
//    that fits the L2 (2 MiB), the Infinity Cache (64 MiB) and neither (1 GiB);
// 2. streaming read bandwidth of a 1 GiB buffer: 16-byte loads per lane, D
//    loads in flight, for several grid sizes;
// 3. one-shot reads the size of a small decode phase (the whole read issued
//    at once by B blocks of 4 waves, Q loads per lane), timed from launch to
//    completion.
// 4. a few workgroups of 16 waves streaming alone (1, 3 or 8 CUs busy).
// Every loop is bounded by its arguments; all indices stay inside the buffers
// (checked on the host before each launch).
//
// build: hipcc -O3 --offload-arch=gfx950 -o mem_stream mem_stream.hip
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

#define CK(x)                                                                                   \
    do {                                                                                        \
        hipError_t err_ = (x);                                                                  \
        if (err_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(err_)); \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

__global__ void k_chase(const unsigned* next, unsigned start, int hops, unsigned* out)
{
    unsigned i = start;
    for (int h = 0; h < hops; h++) i = next[i];
    *out = i;
}

// each lane: D loads of 16 B in flight, walking its slice of the buffer
template <int D>
__global__ __launch_bounds__(256) void k_stream(const uint4* __restrict__ buf, size_t n16, uint4* sink)
{
    const size_t lanes = (size_t)gridDim.x * blockDim.x;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    // element e of round r for this lane: (r * D + k) * lanes + gid
    const size_t rounds = n16 / (lanes * D);
    for (size_t r = 0; r < rounds; r++) {
        uint4 v[D];
#pragma unroll
        for (int k = 0; k < D; k++) v[k] = buf[(r * D + k) * lanes + gid];
#pragma unroll
        for (int k = 0; k < D; k++) {
            acc.x ^= v[k].x;
            acc.y ^= v[k].y;
            acc.z ^= v[k].z;
            acc.w ^= v[k].w;
        }
    }
    if (acc.x == 0x12345678u && acc.y == 0x9abcdef0u) sink[gid & 1023] = acc;
}

// one shot: every lane issues Q loads of 16 B (wave-contiguous 1 KiB each)
template <int Q>
__global__ __launch_bounds__(256) void k_oneshot(const uint4* __restrict__ buf, size_t base, uint4* sink)
{
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint4* w = buf + base + (size_t)wave * Q * 64 + lane;
    uint4 v[Q];
#pragma unroll
    for (int k = 0; k < Q; k++) v[k] = w[k * 64];
    uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < Q; k++) {
        acc.x ^= v[k].x;
        acc.w ^= v[k].w;
    }
    if (acc.x == 0x12345678u && acc.w == 0x9abcdef0u) sink[threadIdx.x] = acc;
}

// a few workgroups of 16 waves streaming alone (what one CU can pull while
// the rest of the chip is idle): `rounds` rounds of Q wave-contiguous 1 KiB
// loads per wave
template <int Q>
__global__ __launch_bounds__(1024) void k_cu_stream(const uint4* __restrict__ buf, size_t base, int rounds, uint4* sink)
{
    const int nw = gridDim.x * 16;
    const int wave = blockIdx.x * 16 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int r = 0; r < rounds; r++) {
        const uint4* w = buf + base + ((size_t)r * nw + wave) * Q * 64 + lane;
        uint4 v[Q];
#pragma unroll
        for (int k = 0; k < Q; k++) v[k] = w[k * 64];
#pragma unroll
        for (int k = 0; k < Q; k++) {
            acc.x ^= v[k].x;
            acc.w ^= v[k].w;
        }
    }
    if (acc.x == 0x12345678u && acc.w == 0x9abcdef0u) sink[threadIdx.x] = acc;
}

static float time_ms(hipEvent_t a, hipEvent_t b)
{
    float ms;
    CK(hipEventElapsedTime(&ms, a, b));
    return ms;
}

template <int Q>
static void oneshot(const uint4* buf, uint4* sink, int blocks, size_t n16, hipStream_t st, hipEvent_t a, hipEvent_t b)
{
    // every launch reads a different region, cycling through the whole
    // buffer (larger than the Infinity Cache), so the data comes from HBM
    const size_t region = (size_t)blocks * 4 * Q * 64;
    if (region > n16) return;
    const int reps = 200;
    const size_t n_reg = n16 / region;
    const size_t hop = std::max<size_t>(1, n_reg / reps);
    for (int i = 0; i < 10; i++) hipLaunchKernelGGL(k_oneshot<Q>, dim3(blocks), dim3(256), 0, st, buf, (size_t)0, sink);
    CK(hipEventRecord(a, st));
    for (int i = 0; i < reps; i++) {
        const size_t base = ((size_t)i * hop % n_reg) * region;   // base + region <= n16
        hipLaunchKernelGGL(k_oneshot<Q>, dim3(blocks), dim3(256), 0, st, buf, base, sink);
    }
    CK(hipEventRecord(b, st));
    CK(hipEventSynchronize(b));
    const double us = 1e3 * time_ms(a, b) / reps;
    const double kb = blocks * 4.0 * Q * 1024 / 1024.0;
    std::printf("oneshot  blocks %4d  Q %2d  (%7.0f KiB): %6.2f us per kernel, %7.1f GB/s\n", blocks, Q, kb, us,
                kb * 1024 / us / 1e3);
}

template <int Q>
static void cu_stream(const uint4* buf, uint4* sink, int blocks, int rounds, size_t n16, hipStream_t st, hipEvent_t a,
                      hipEvent_t b)
{
    const size_t region = (size_t)rounds * blocks * 16 * Q * 64;   // 16-byte units per launch
    if (region > n16) return;
    const int reps = 200;
    const size_t n_reg = n16 / region;
    const size_t hop = std::max<size_t>(1, n_reg / reps);
    for (int i = 0; i < 10; i++)
        hipLaunchKernelGGL(k_cu_stream<Q>, dim3(blocks), dim3(1024), 0, st, buf, (size_t)0, rounds, sink);
    CK(hipEventRecord(a, st));
    for (int i = 0; i < reps; i++) {
        const size_t base = ((size_t)i * hop % n_reg) * region;   // base + region <= n16
        hipLaunchKernelGGL(k_cu_stream<Q>, dim3(blocks), dim3(1024), 0, st, buf, base, rounds, sink);
    }
    CK(hipEventRecord(b, st));
    CK(hipEventSynchronize(b));
    const double us = 1e3 * time_ms(a, b) / reps;
    const double kb = region * 16.0 / 1024.0;
    std::printf("cu-stream blocks %2d of 16 waves  Q %2d  rounds %2d (%6.0f KiB): %6.2f us per kernel\n", blocks, Q,
                rounds, kb, us);
}

template <int D>
static void stream(const uint4* buf, uint4* sink, size_t n16, int blocks, hipStream_t st, hipEvent_t a, hipEvent_t b)
{
    const size_t lanes = (size_t)blocks * 256;
    const size_t rounds = n16 / (lanes * D);
    const size_t used = rounds * lanes * D;
    if (used > n16 || rounds == 0) return;
    hipLaunchKernelGGL(k_stream<D>, dim3(blocks), dim3(256), 0, st, buf, n16, sink);
    CK(hipEventRecord(a, st));
    for (int i = 0; i < 5; i++) hipLaunchKernelGGL(k_stream<D>, dim3(blocks), dim3(256), 0, st, buf, n16, sink);
    CK(hipEventRecord(b, st));
    CK(hipEventSynchronize(b));
    const double s = 1e-3 * time_ms(a, b) / 5;
    std::printf("stream   blocks %5d  D %2d: %7.1f GB/s\n", blocks, D, used * 16.0 / s / 1e9);
}

int main()
{
    hipStream_t st;
    CK(hipStreamCreate(&st));
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    unsigned* d_out;
    CK(hipMalloc(&d_out, 64));

    // 1. latency
    for (size_t bytes : {(size_t)2 << 20, (size_t)64 << 20, (size_t)1 << 30}) {
        const size_t n = bytes / 4;
        // random cycle visiting one word per 256-byte line (so every hop is a new line)
        const size_t stride = 64;
        const size_t m = n / stride;
        std::vector<unsigned> perm(m);
        std::iota(perm.begin(), perm.end(), 0u);
        std::mt19937 rng(1);
        std::shuffle(perm.begin(), perm.end(), rng);
        std::vector<unsigned> next(n, 0);
        for (size_t i = 0; i < m; i++) next[(size_t)perm[i] * stride] = (unsigned)(perm[(i + 1) % m] * stride);
        unsigned* d_next;
        CK(hipMalloc(&d_next, n * 4));
        CK(hipMemcpy(d_next, next.data(), n * 4, hipMemcpyHostToDevice));
        const int hops = 20000;
        hipLaunchKernelGGL(k_chase, dim3(1), dim3(1), 0, st, d_next, perm[0] * (unsigned)stride, 2000, d_out);
        CK(hipEventRecord(a, st));
        hipLaunchKernelGGL(k_chase, dim3(1), dim3(1), 0, st, d_next, perm[0] * (unsigned)stride, hops, d_out);
        CK(hipEventRecord(b, st));
        CK(hipEventSynchronize(b));
        std::printf("latency  footprint %6zu MiB: %7.1f ns per dependent load\n", bytes >> 20,
                    1e6 * time_ms(a, b) / hops);
        CK(hipFree(d_next));
    }

    // 2. streaming bandwidth
    const size_t n16 = ((size_t)1 << 30) / 16;
    uint4* buf;
    uint4* sink;
    CK(hipMalloc(&buf, n16 * 16));
    CK(hipMalloc(&sink, 1024 * 16));
    CK(hipMemset(buf, 1, n16 * 16));
    for (int blocks : {256, 512, 1024, 2048, 4096}) {
        stream<4>(buf, sink, n16, blocks, st, a, b);
        stream<8>(buf, sink, n16, blocks, st, a, b);
        stream<16>(buf, sink, n16, blocks, st, a, b);
    }

    // 3. one-shot reads of decode-phase sizes
    for (int blocks : {18, 30, 48, 144, 256, 512, 1024}) {
        oneshot<1>(buf, sink, blocks, n16, st, a, b);
        oneshot<3>(buf, sink, blocks, n16, st, a, b);
        oneshot<9>(buf, sink, blocks, n16, st, a, b);
        oneshot<16>(buf, sink, blocks, n16, st, a, b);
    }
    // 4. a few CUs streaming alone
    for (int blocks : {1, 3, 8}) {
        cu_stream<1>(buf, sink, blocks, 1, n16, st, a, b);
        cu_stream<16>(buf, sink, blocks, 1, n16, st, a, b);
        cu_stream<16>(buf, sink, blocks, 2, n16, st, a, b);
        cu_stream<16>(buf, sink, blocks, 6, n16, st, a, b);
        cu_stream<8>(buf, sink, blocks, 12, n16, st, a, b);
    }
    return 0;
}
