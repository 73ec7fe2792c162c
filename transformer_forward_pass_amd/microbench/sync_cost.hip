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
//      all slots in parallel and releases everybody through one word);
//   4. the same persistent kernel with barriers that poll with relaxed loads
//      and take a single acquire fence after the wait: a central counter,
//      and two-level barriers whose first level groups the blocks of one
//      XCD (by blockIdx % 8, and by the hardware XCC id), so only one
//      arrival per group reaches the central counter; and a central barrier
//      with no fence, whose hand-off data is written with agent-scope stores
//      that complete before the relaxed arrival.
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

// ---------------------------------------------------------------------------
// Barriers that poll with relaxed loads and take one acquire fence after the
// wait (an acquire load per poll invalidates the L2 on every spin).
// ---------------------------------------------------------------------------
struct BarR {
    unsigned count;
    unsigned pad0[1023];
    unsigned gen;
    unsigned pad1[1023];
    unsigned xcount[8][64];   // per-group arrival counters, one 256-byte line each
    unsigned xgen[8][64];     // per-group release words
    unsigned xsize[8];        // blocks per group (set by the host)
    unsigned pad2[56];
    int err;
};

constexpr unsigned kSpin = 1u << 22;

__device__ __forceinline__ unsigned ld_relaxed(unsigned* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// central counter: release arrival, relaxed polls, one acquire fence
__device__ __forceinline__ void grid_barrier_relaxed(BarR* b, unsigned nblocks, unsigned& gen)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned arrived = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == nblocks - 1) {
            __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&b->gen, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned spins = 0;
            while (ld_relaxed(&b->gen) == gen) {
                if (++spins > kSpin) {
                    b->err = 1;
                    break;
                }
            }
            __atomic_thread_fence(__ATOMIC_ACQUIRE);
        }
    }
    gen++;
    __syncthreads();
}

// two levels: blocks of one group (group = xcc id or blockIdx % 8) arrive on
// the group's counter; the group's last arrival takes the group to the
// central counter, waits for the central release and releases its group.
// Relaxed polls, one acquire fence after the wait.
__device__ __forceinline__ void grid_barrier_two_level(BarR* b, unsigned grp, unsigned n_groups, unsigned& gen)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned next = gen + 1;
        const unsigned a = __hip_atomic_fetch_add(&b->xcount[grp][0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        unsigned spins = 0;
        if (a == b->xsize[grp] - 1) {
            __hip_atomic_store(&b->xcount[grp][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned c = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (c == n_groups - 1) {
                __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&b->gen, next, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                while (ld_relaxed(&b->gen) != next) {
                    if (++spins > kSpin) {
                        b->err = 1;
                        break;
                    }
                }
                __atomic_thread_fence(__ATOMIC_ACQUIRE);
            }
            __hip_atomic_store(&b->xgen[grp][0], next, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            while (ld_relaxed(&b->xgen[grp][0]) != next) {
                if (++spins > kSpin) {
                    b->err = 1;
                    break;
                }
            }
            __atomic_thread_fence(__ATOMIC_ACQUIRE);
        }
    }
    gen++;
    __syncthreads();
}

// no release or acquire fence at all: the data a phase hands on is written
// with agent-scope stores (not left dirty in one XCD's L2), the arrival waits
// for those stores to complete and then adds to the counter relaxed; the
// waiters poll relaxed and read the data with agent-scope loads.
__device__ __forceinline__ void grid_barrier_nofence(BarR* b, unsigned nblocks, unsigned& gen)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_s_waitcnt(0);   // this block's stores have completed
        const unsigned arrived = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == nblocks - 1) {
            __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);
            __hip_atomic_store(&b->gen, gen + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned spins = 0;
            while (ld_relaxed(&b->gen) == gen) {
                if (++spins > kSpin) {
                    b->err = 1;
                    break;
                }
            }
        }
    }
    gen++;
    __syncthreads();
}

__device__ __forceinline__ unsigned xcc_id()
{
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 7u;
}

// every barrier also checks that the neighbouring block's write before it
// is visible after it (mismatches counted in b->err's upper bits)
__device__ __forceinline__ void check_neighbour(BarR* b, const unsigned* chk, unsigned i)
{
    if (threadIdx.x == 0) {
        const unsigned nb = (blockIdx.x + 1) % gridDim.x;
        if (__hip_atomic_load(&chk[nb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < i)
            atomicAdd(reinterpret_cast<unsigned*>(&b->err), 2u);
    }
}

// mode 0: central relaxed; 1: two-level by blockIdx % 8; 2: two-level by xcc
// id; 3: central, relaxed arrival after the block's agent-scope stores complete
__global__ void k_persistent_relaxed(BarR* b, unsigned* chk, int n_barriers, int mode, unsigned* xcc_out)
{
    unsigned gen = 0;
    const unsigned grp = (mode == 2) ? xcc_id() : (blockIdx.x & 7u);
    if (threadIdx.x == 0 && xcc_out) xcc_out[blockIdx.x] = xcc_id();
    unsigned n_groups = 0;
    for (int g = 0; g < 8; g++) n_groups += b->xsize[g] > 0;
    for (int i = 1; i <= n_barriers; i++) {
        if (threadIdx.x == 0) __hip_atomic_store(&chk[blockIdx.x], (unsigned)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (mode == 0) grid_barrier_relaxed(b, gridDim.x, gen);
        else if (mode == 3) grid_barrier_nofence(b, gridDim.x, gen);
        else grid_barrier_two_level(b, grp, n_groups, gen);
        check_neighbour(b, chk, (unsigned)i);
        if (__hip_atomic_load(&b->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1) return;
    }
}

__global__ void k_xcc_map(unsigned* out)
{
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
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

// Relaxed-poll barriers: mode 0 central, 1 two-level by blockIdx % 8, 2
// two-level by the hardware xcc id (group sizes from a mapping launch of the
// same grid; a block placed differently in the timed launch makes its group
// miss its count, which ends in the bounded-spin error, not a hang).
static void time_relaxed(int mode, int grid, int occ, int n_cu, int N, hipStream_t st, hipEvent_t a, hipEvent_t ev1)
{
    if (grid > occ * n_cu) return;
    static const char* names[] = {"barrier relaxed", "barrier 2-level %8", "barrier 2-level xcc",
                                  "barrier no-fence"};
    BarR* bar;
    unsigned *chk, *xmap;
    CK(hipMalloc(&bar, sizeof(BarR)));
    CK(hipMalloc(&chk, grid * sizeof(unsigned)));
    CK(hipMalloc(&xmap, grid * sizeof(unsigned)));
    std::vector<unsigned> hx(grid);
    CK(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_xcc_map), dim3(grid), dim3(256),
                                  (void*[]){&xmap}, 0, st));
    CK(hipMemcpy(hx.data(), xmap, grid * sizeof(unsigned), hipMemcpyDeviceToHost));
    unsigned sizes[8] = {};
    for (int i = 0; i < grid; i++) sizes[mode == 2 ? (hx[i] & 7u) : (unsigned)(i & 7)]++;
    int same = 0;
    for (int i = 0; i < grid; i++) same += (hx[i] & 7u) == (unsigned)(hx[i % 8] & 7u);
    for (int rep = 0; rep < 2; rep++) {
        BarR hb{};
        for (int g = 0; g < 8; g++) hb.xsize[g] = sizes[g];
        CK(hipMemcpy(bar, &hb, sizeof(BarR), hipMemcpyHostToDevice));
        CK(hipMemset(chk, 0, grid * sizeof(unsigned)));
        int nb = N, md = mode;
        unsigned* xo = rep ? xmap : nullptr;
        void* args[] = {&bar, &chk, &nb, &md, &xo};
        CK(hipEventRecord(a, st));
        CK(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_persistent_relaxed), dim3(grid), dim3(256), args,
                                      0, st));
        CK(hipEventRecord(ev1, st));
        CK(hipEventSynchronize(ev1));
        float ms;
        CK(hipEventElapsedTime(&ms, a, ev1));
        CK(hipMemcpy(&hb, bar, sizeof(BarR), hipMemcpyDeviceToHost));
        std::vector<unsigned> hx2(grid);
        CK(hipMemcpy(hx2.data(), xmap, grid * sizeof(unsigned), hipMemcpyDeviceToHost));
        int moved = 0;
        for (int i = 0; i < grid; i++) moved += hx2[i] != hx[i];
        if (rep)
            std::printf("%-22s grid %4d: %.3f us per barrier (timeout=%d, stale reads=%u, blocks whose xcc matches "
                        "blockIdx%%8's=%d/%d, moved between launches=%d)\n",
                        names[mode], grid, 1e3 * ms / N, hb.err & 1, (unsigned)hb.err >> 1, same, grid, moved);
    }
    CK(hipFree(bar));
    CK(hipFree(chk));
    CK(hipFree(xmap));
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
    for (int grid : {64, 128, 256, 512})
        for (int mode = 0; mode < 4; mode++) time_relaxed(mode, grid, occ, prop.multiProcessorCount, N, st, a, b);
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
