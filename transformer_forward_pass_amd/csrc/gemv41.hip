// gemv41.hip -- the batch-1 decode GEMV over 4-bit (MXFP4) weights with the
// tile shape fixed at compile time (gfx950).
//
// Same arithmetic and layout as k_gemv4 (gemv4.hip): one 16-byte load per
// lane holds one 32-weight block, each block folded exactly in fp64 and
// scaled by its E8M0 power of two.  The launch shape follows the bf16
// batch-1 kernel: one tile (J block iterations of R rows) per wave; every
// wave's input loads go out before any weight load of the workgroup; the
// weight and scale loads are unconditional (a wave past the last tile loads
// the last one and drops it), so the compiler's wait counts stay exact and
// each block iteration waits only for its own loads -- the fold of the first
// blocks overlaps the arrival of the last, and the RMSNorm staging waits for
// the input alone.
#include <hip/hip_runtime.h>

#include "gemv_kernels.h"

namespace mak {

__device__ __forceinline__ double e8m0_f64(uint32_t s) { return __hiloint2double((int)((s + 896u) << 20), 0); }

__device__ __forceinline__ void fp4x8_f32(uint32_t u, float (&f)[8])
{
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 0);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 1);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 2);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 3);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

template <int R, int J, int EPI>
__global__ __launch_bounds__(MAK_BLOCK) void k_gemv41(GemvPhase p)
{
    static_assert(EPI != EPI_LOGITS, "the LM head stays bf16");
    constexpr int QT = J * R;                      // block loads per lane
    constexpr int NW = MAK_BLOCK / 64;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ double red[NW];
    float* hs = reinterpret_cast<float*>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrl = p.geo.lr_log2;
    const int grp = lane >> lrl;
    const int s = lane & ((1 << lrl) - 1);
    const int G = 64 >> lrl;
    const int n_tiles = p.geo.n_tiles;
    const int N = p.geo.n_rows;
    const int tile = blockIdx.x * NW + wave;
    const int t0 = min(tile, n_tiles - 1);

    // 1. the input, issued by every wave before any weight load
    Staged<1> stg;
    issue_input<1>(p, stg, MAK_BLOCK);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // 2. residual rows (lane s == 0 owns rows row0 .. row0 + R - 1), then the
    //    tile's scale bytes and code chunks, in block order
    // (raw bits, loaded by every lane from a clamped row and converted only in
    // the epilogue: a load whose value is used under a branch would make the
    // compiler wait for it, and for the input, before any weight load)
    uint16_t xres[R];
    if (EPI == EPI_RESIDUAL) {
        const int row0 = t0 * G * R + grp * R;
#pragma unroll
        for (int r = 0; r < R; r++) xres[r] = p.out[(size_t)p.col0 * p.out_ld + min(row0 + r, N - 1)];
    }
    const int64_t slot0 = (int64_t)t0 * QT * 64 + lane;
    const unsigned char* S = reinterpret_cast<const unsigned char*>(p.w) + p.geo.scale_off + slot0;
    const uint4* W = reinterpret_cast<const uint4*>(p.w) + slot0;
    uint32_t sc[QT];
    uint4 buf[QT];
#pragma unroll
    for (int i = 0; i < QT; i++) {
        sc[i] = ld_stream_u8(S + i * 64);
        asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < QT; i++) {
        buf[i] = ld_stream16(&W[i * 64]);
        asm volatile("" ::: "memory");
    }

    // 3. stage the input (RMSNorm); LDS-only barrier: the weights keep arriving
    finish_input<1, true>(p, stg, hs, red, MAK_BLOCK);
    lds_barrier();
    if (tile >= n_tiles) return;

    // 4. fold block iteration c as soon as its loads have landed
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = 0.0;
#pragma unroll
    for (int c = 0; c < J; c++) {
        const int blk = (c << lrl) + s;
        double part[R];
        uint4 w[R];
        uint32_t sv[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            part[r] = 0.0;
            w[r] = buf[c * R + r];
            sv[r] = sc[c * R + r];
            // (empty asms: this block's uses stay after its loads, and its
            // input reads and conversions after the previous block's fold)
            asm volatile("" : "+v"(w[r].x), "+v"(w[r].y), "+v"(w[r].z), "+v"(w[r].w), "+v"(sv[r]), "+v"(acc[r])
                         :: "memory");
        }
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float4* x4 = reinterpret_cast<const float4*>(hs + blk * 36 + 8 * g);
            const float4 lo = x4[0], hi = x4[1];
            const double xd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int r = 0; r < R; r++) {
                float wf[8];
                fp4x8_f32(g == 0 ? w[r].x : g == 1 ? w[r].y : g == 2 ? w[r].z : w[r].w, wf);
#pragma unroll
                for (int e = 0; e < 8; e++) part[r] = fma((double)wf[e], xd[e], part[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) acc[r] = fma(part[r], e8m0_f64(sv[r]), acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = group_sum_rt(acc[r], lrl);

    // 5. epilogue (lanes s == 0)
    if (s != 0) return;
    const int row0 = tile * G * R + grp * R;
    const size_t col = (size_t)p.col0;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int r = 0; r + 1 < R; r += 2) {
            if (row0 + r < N) {
                const float gv = rbf((float)acc[r]);
                const float u = rbf((float)acc[r + 1]);
                const double gd = (double)gv;
                const float z = rbf((float)(gd / (1.0 + exp(-gd))));
                p.out[col * p.out_ld + ((row0 + r) >> 1)] = f2bf(z * u);
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int row = row0 + r;
            if (row >= N) continue;
            if (EPI == EPI_STORE) p.out[col * p.out_ld + row] = f2bf((float)acc[r]);
            else p.out[col * p.out_ld + row] = f2bf(bf2f(xres[r]) + rbf((float)acc[r]));
        }
    }
}

}  // namespace mak

using namespace mak;

// (R, J) shapes with a compiled k_gemv41 (SwiGLU: even R only)
#define MAK_GEMV41_SHAPES(X) \
    X(1, 1) X(1, 2) X(1, 3) X(1, 4) X(1, 8) X(1, 9) X(1, 11) X(1, 16) X(2, 1) X(2, 2) X(2, 3) X(2, 4) X(2, 8) X(2, 9)

// k_gemv41<r, j, epi>, or nullptr when that shape is not compiled
const void* mak_gemv41_fn(int r, int j, int epi)
{
#define X(R_, J_)                                                                                  \
    if (r == R_ && j == J_) {                                                                      \
        if (epi == EPI_STORE) return reinterpret_cast<const void*>(&k_gemv41<R_, J_, EPI_STORE>);  \
        if (epi == EPI_RESIDUAL) return reinterpret_cast<const void*>(&k_gemv41<R_, J_, EPI_RESIDUAL>); \
        if (epi == EPI_SWIGLU && R_ % 2 == 0) return reinterpret_cast<const void*>(&k_gemv41<R_, J_, EPI_SWIGLU>); \
        return nullptr;                                                                            \
    }
    MAK_GEMV41_SHAPES(X)
#undef X
    return nullptr;
}

// Raise the dynamic-LDS ceiling of every k_gemv41 instantiation
hipError_t mak_gemv41_set_lds_limit(int bytes)
{
    for (int r : {1, 2})
        for (int j : {1, 2, 3, 4, 8, 9, 11, 16})
            for (int epi : {(int)EPI_STORE, (int)EPI_RESIDUAL, (int)EPI_SWIGLU})
                if (const void* f = mak_gemv41_fn(r, j, epi)) {
                    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
                    if (e != hipSuccess) return e;
                }
    return hipSuccess;
}
