// sync_cost.hip -- what one dependent phase boundary costs on this GPU.
//
// The decode step is a chain of ~5 dependent phases per layer; the
// "model-as-a-kernel" page crosses them with a software grid barrier inside
// one persistent kernel (Method section), and the CuTeDSL page puts a grid
// barrier at roughly the cost of splitting a kernel in two (Grid
// synchronization section).  This program measures both options here:
//   1. a chain of small kernels launched back to back on one stream;
//   2. the same chain captured once into a hipGraph and replayed;
//   3. a persistent kernel (cooperative launch, so all blocks are resident)
//      crossing a grid barrier N times, for several grids, in three forms:
//      a central arrival counter + generation word; the same with polling
//      backoff and the two words on separate 4 KiB pages; and "flat" flags
//      (every block publishes its generation in its own slot, block 0 gathers
//      all slots in parallel and releases everybody through one word).
// Every wait is bounded: a barrier that spins too long sets an error flag
// and the kernel returns.
//
// build: hipcc -O3 --offload-arch=gfx950 -o sync_cost sync_cost.hip
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CK(x)                                                                            \
    do {                                                                                 \
        hipError_t e = (x);                                                              \
        if (e != hipSuccess) {                                                           \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e)); \
            std::exit(1);                                                                \
        }                                                                                \
    } while (0)

__global__ void k_small(float* buf, int i)
{
    // one store per block, like a phase's output write
    if (threadIdx.x == 0) buf[blockIdx.x] = (float)i;
}

struct Bar {
    unsigned count;
    unsigned pad0[63];
    unsigned gen;
    unsigned pad1[63];
    int err;
};

__device__ __forceinline__ void grid_barrier(Bar* b, unsigned nblocks, unsigned& gen)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned arrived = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == nblocks - 1) {
            __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&b->gen, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned spins = 0;
            while (__hip_atomic_load(&b->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                if (++spins > (1u << 22)) {
                    b->err = 1;
                    break;
                }
            }
        }
        __threadfence();
    }
    gen++;
    __syncthreads();
}

// central counter with backoff; count and gen live 4 KiB apart
struct Bar2 {
    unsigned count;
    unsigned pad0[1023];
    unsigned gen;
    unsigned pad1[1023];
    int err;
};

__device__ __forceinline__ void grid_barrier_backoff(Bar2* b, unsigned nblocks, unsigned& gen)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned arrived = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == nblocks - 1) {
            __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&b->gen, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned spins = 0;
            while (__hip_atomic_load(&b->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > (1u << 22)) {
                    b->err = 1;
                    break;
                }
            }
        }
        __threadfence();
    }
    gen++;
    __syncthreads();
}

// flat flags: slot[b] (one 4-byte word per block, contiguous), release word
struct Bar3 {
    unsigned slot[1024];
    unsigned pad[1024];
    unsigned gen;
    unsigned pad1[1023];
    int err;
};

__device__ __forceinline__ void grid_barrier_flat(Bar3* b, unsigned nblocks, unsigned& gen)
{
    __syncthreads();
    const unsigned next = gen + 1;
    if (threadIdx.x == 0) {
        __threadfence();
        __hip_atomic_store(&b->slot[blockIdx.x], next, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blockIdx.x == 0) {
        // every thread watches nblocks/blockDim slots
        for (unsigned s = threadIdx.x; s < nblocks; s += blockDim.x) {
            unsigned spins = 0;
            while (__hip_atomic_load(&b->slot[s], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != next) {
                if (++spins > (1u << 22)) {
                    b->err = 1;
                    break;
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(&b->gen, next, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == 0) {
        unsigned spins = 0;
        while (__hip_atomic_load(&b->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != next) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > (1u << 22)) {
                b->err = 1;
                break;
            }
        }
    }
    if (threadIdx.x == 0) __threadfence();
    gen = next;
    __syncthreads();
}

__global__ void k_persistent(Bar* b, float* buf, int n_barriers)
{
    unsigned gen = 0;
    for (int i = 0; i < n_barriers; i++) {
        if (threadIdx.x == 0) buf[blockIdx.x] = (float)i;
        grid_barrier(b, gridDim.x, gen);
        if (__hip_atomic_load(&b->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    }
}

__global__ void k_persistent_backoff(Bar2* b, float* buf, int n_barriers)
{
    unsigned gen = 0;
    for (int i = 0; i < n_barriers; i++) {
        if (threadIdx.x == 0) buf[blockIdx.x] = (float)i;
        grid_barrier_backoff(b, gridDim.x, gen);
        if (__hip_atomic_load(&b->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    }
}

__global__ void k_persistent_flat(Bar3* b, float* buf, int n_barriers)
{
    unsigned gen = 0;
    for (int i = 0; i < n_barriers; i++) {
        if (threadIdx.x == 0) buf[blockIdx.x] = (float)i;
        grid_barrier_flat(b, gridDim.x, gen);
        if (__hip_atomic_load(&b->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    }
}

template <class B>
static void time_persistent(const char* name, const void* kern, int grid, int occ, int n_cu, int N,
                            hipStream_t st, float* buf, hipEvent_t a, hipEvent_t ev1)
{
    if (grid > occ * n_cu) return;
    B* bar;
    CK(hipMalloc(&bar, sizeof(B)));
    for (int rep = 0; rep < 2; rep++) {
        CK(hipMemset(bar, 0, sizeof(B)));
        int nb = N;
        void* args[] = {&bar, &buf, &nb};
        CK(hipEventRecord(a, st));
        CK(hipLaunchCooperativeKernel(kern, dim3(grid), dim3(256), args, 0, st));
        CK(hipEventRecord(ev1, st));
        CK(hipEventSynchronize(ev1));
        float ms;
        CK(hipEventElapsedTime(&ms, a, ev1));
        B hb;
        CK(hipMemcpy(&hb, bar, sizeof(B), hipMemcpyDeviceToHost));
        if (rep) std::printf("%-22s grid %4d: %.3f us per barrier (err=%d)\n", name, grid, 1e3 * ms / N, hb.err);
    }
    CK(hipFree(bar));
}

int main()
{
    hipDeviceProp_t prop;
    CK(hipGetDeviceProperties(&prop, 0));
    std::printf("device %s, %d CUs, clock %d kHz\n", prop.gcnArchName, prop.multiProcessorCount, prop.clockRate);
    hipStream_t st;
    CK(hipStreamCreate(&st));
    float* buf;
    CK(hipMalloc(&buf, 1 << 20));
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    const int N = 2000;
    for (int grid : {64, 256, 1024}) {
        // 1. stream chain
        for (int w = 0; w < 100; w++) hipLaunchKernelGGL(k_small, dim3(grid), dim3(256), 0, st, buf, w);
        CK(hipStreamSynchronize(st));
        CK(hipEventRecord(a, st));
        for (int i = 0; i < N; i++) hipLaunchKernelGGL(k_small, dim3(grid), dim3(256), 0, st, buf, i);
        CK(hipEventRecord(b, st));
        CK(hipEventSynchronize(b));
        float ms;
        CK(hipEventElapsedTime(&ms, a, b));
        std::printf("stream chain   grid %4d: %.3f us per kernel\n", grid, 1e3 * ms / N);

        // 2. graph replay of the same chain
        hipGraph_t g;
        hipGraphExec_t ge;
        CK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
        for (int i = 0; i < N; i++) hipLaunchKernelGGL(k_small, dim3(grid), dim3(256), 0, st, buf, i);
        CK(hipStreamEndCapture(st, &g));
        CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
        CK(hipGraphLaunch(ge, st));
        CK(hipStreamSynchronize(st));
        CK(hipEventRecord(a, st));
        CK(hipGraphLaunch(ge, st));
        CK(hipEventRecord(b, st));
        CK(hipEventSynchronize(b));
        CK(hipEventElapsedTime(&ms, a, b));
        std::printf("graph replay   grid %4d: %.3f us per kernel\n", grid, 1e3 * ms / N);
        CK(hipGraphExecDestroy(ge));
        CK(hipGraphDestroy(g));
    }
    // 3. persistent kernel + grid barrier
    int occ = 0;
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_persistent, 256, 0));
    std::printf("persistent occupancy: %d blocks of 256 per CU\n", occ);
    for (int grid : {64, 128, 256, 512}) {
        time_persistent<Bar>("barrier central", reinterpret_cast<const void*>(k_persistent), grid, occ,
                             prop.multiProcessorCount, N, st, buf, a, b);
        time_persistent<Bar2>("barrier backoff", reinterpret_cast<const void*>(k_persistent_backoff), grid,
                              occ, prop.multiProcessorCount, N, st, buf, a, b);
        time_persistent<Bar3>("barrier flat", reinterpret_cast<const void*>(k_persistent_flat), grid, occ,
                              prop.multiProcessorCount, N, st, buf, a, b);
    }
    return 0;
}
