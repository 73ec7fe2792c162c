// gemv4.hip -- the decode GEMV over 4-bit weights (OCP MXFP4) on gfx950.
//
// The "model-as-a-kernel" page lists 4-bit weights among its supported
// variants (API section, "Supported" paragraph): the weight stream, which
// bounds decode, shrinks about fourfold.  Its nf4 format is not given on the
// page; the format here is MXFP4 of the OCP Microscaling (MX) specification
// v1.0, which gfx950 converts in hardware: blocks of 32 weights of one row
// share an E8M0 scale 2^e, each weight an E2M1 code (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6).  A 16-byte load holds exactly one block, so each lane
// loads one block's codes plus its scale byte (packed layout: mak_internal.h).
//
// Arithmetic: every weight code * 2^e is exactly a bf16 value, and the dot
// product stays exact before its single rounding: each block's 32 products
// code * x are summed in fp64 (code from v_cvt_scalef32_pk_f32_fp4 at scale
// 1, exact), the block sum is multiplied by 2^e (exact in fp64), and the
// block sums are added in fp64.  The result is therefore the same as the bf16
// GEMV's on the dequantized weights.  Inputs are staged in LDS as fp32 in
// 32-input blocks at a stride of 36 floats (RMSNorm applied in the prologue
// as in the bf16 GEMV), the epilogues are the bf16 GEMV's (store, residual,
// SwiGLU); the LM head and the embedding stay bf16.
#include <hip/hip_runtime.h>

#include "gemv_kernels.h"

namespace mak {

// 2^(s - 127) as fp64 for an E8M0 scale byte s in [0, 254]
__device__ __forceinline__ double e8m0_to_f64(uint32_t s)
{
    return __hiloint2double((int)((s + 896u) << 20), 0);
}

// the 8 E2M1 codes of one dword as fp32: byte b holds elements 2b (low
// nibble) and 2b + 1 (high nibble)
__device__ __forceinline__ void fp4x8_to_f32(uint32_t u, float (&f)[8])
{
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 0);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 1);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 2);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 3);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// One workgroup of 4 waves; each wave walks tiles t = wave id, + waves in
// grid, ... and streams each tile's Q = J*R block loads in batches of QB,
// ping-ponging two buffers (the next batch is issued before the landed one
// is folded).  Lane (group, s) owns rows row0 .. row0+R-1 of its group and
// block s, s+lr, ... of each; rows are reduced over the lr lanes at the end
// of the tile.
template <int R, int NC, int EPI>
__global__ __launch_bounds__(MAK_BLOCK) void k_gemv4(GemvPhase p)
{
    static_assert(EPI != EPI_LOGITS, "the LM head stays bf16");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int NW = MAK_BLOCK / 64;
    constexpr int QB = 8;                      // block loads per batch (a multiple of R)
    static_assert(QB % R == 0, "batch must hold whole row groups");
    __shared__ double red[NW];
    float* hs = reinterpret_cast<float*>(smem);

    const int K = p.geo.k;
    const int CS = pad32_stride(K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int J = (K >> 5) >> lrl;
    const int Q = J * R;                       // block loads per lane per tile
    const int NB = (Q + QB - 1) / QB;          // batches per tile
    const char* W = reinterpret_cast<const char*>(p.w);
    const unsigned char* S = reinterpret_cast<const unsigned char*>(p.w) + p.geo.scale_off;
    const int n_waves = gridDim.x * NW;
    const int N = p.geo.n_rows;

    auto issue = [&](uint4 (&buf)[QB], uint32_t (&sc)[QB], int t, int b) {
        const int64_t slot0 = ((int64_t)t * Q + (int64_t)b * QB) * 64;
        const char* wt = W + slot0 * 16;
        const unsigned char* st = S + slot0;
        const int n = min(QB, Q - b * QB);
#pragma unroll
        for (int i = 0; i < QB; i++)
            if (i < n) {
                buf[i] = ld_stream16(wt + (lane * 16 + i * 1024));
                sc[i] = ld_stream_u8(st + lane + i * 64);
            }
    };
    // wait for a batch (codes and scales) and keep later loads below
    auto ready = [&](const uint4 (&buf)[QB], const uint32_t (&sc)[QB], int n) {
#pragma unroll
        for (int i = 0; i < QB; i++)
            if (i < n)
                asm volatile("" ::"v"(buf[i].x), "v"(buf[i].y), "v"(buf[i].z), "v"(buf[i].w), "v"(sc[i])
                             : "memory");
    };

    int tile = blockIdx.x * NW + wave;

    Staged<NC> stg;
    issue_input<NC>(p, stg, MAK_BLOCK);
    float xres[R][NC];
    auto load_res = [&](int t) {
        if (EPI == EPI_RESIDUAL && s == 0) {
            const int row0 = t * G * R + grp * R;
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int c = 0; c < NC; c++)
                    xres[r][c] = (row0 + r < N && c < p.ncols)
                                     ? bf2f(p.out[(size_t)(p.col0 + c) * p.out_ld + row0 + r])
                                     : 0.f;
        }
    };
    uint4 bufA[QB], bufB[QB];
    uint32_t scA[QB], scB[QB];
    finish_input<NC, true>(p, stg, hs, red, MAK_BLOCK);
    if (tile < p.geo.n_tiles) {
        load_res(tile);
        issue(bufA, scA, tile, 0);
    }
    __syncthreads();

    double acc[R][NC];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[r][c] = 0.0;

    // fold one landed batch: for each block index in it, the R rows' block
    // sums against the same 32 inputs, then scaled into the accumulators
    auto compute = [&](const uint4 (&buf)[QB], const uint32_t (&sc)[QB], int b) {
        const int n = min(QB, Q - b * QB);
#pragma unroll
        for (int jj = 0; jj < QB / R; jj++) {
            const int i0 = jj * R;
            if (i0 < n) {
                const int blk = (((b * QB + i0) / R) << lrl) + s;   // block index within the row
                double part[R][NC];
#pragma unroll
                for (int r = 0; r < R; r++)
#pragma unroll
                    for (int c = 0; c < NC; c++) part[r][c] = 0.0;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    float wf[R][8];
#pragma unroll
                    for (int r = 0; r < R; r++) {
                        const uint4 v = buf[i0 + r];
                        fp4x8_to_f32(g == 0 ? v.x : g == 1 ? v.y : g == 2 ? v.z : v.w, wf[r]);
                    }
#pragma unroll
                    for (int c = 0; c < NC; c++) {
                        const float4* x4 = reinterpret_cast<const float4*>(hs + (size_t)c * CS + blk * 36 + 8 * g);
                        const float4 lo = x4[0], hi = x4[1];
                        const float xv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const double xd = xv[e];
#pragma unroll
                            for (int r = 0; r < R; r++) part[r][c] = fma((double)wf[r][e], xd, part[r][c]);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const double sd = e8m0_to_f64(sc[i0 + r]);
#pragma unroll
                    for (int c = 0; c < NC; c++) acc[r][c] = fma(part[r][c], sd, acc[r][c]);
                }
            }
        }
    };

    // reduce each row over its lr lanes, then the epilogue
    auto finish_tile = [&](int t) {
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[r][c] = group_sum_rt(acc[r][c], lrl);
        if (s == 0) {
            const int row0 = t * G * R + grp * R;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int r = 0; r + 1 < R; r += 2) {
                    const int i = (row0 + r) >> 1;
                    if (row0 + r < N) {
#pragma unroll
                        for (int c = 0; c < NC; c++) {
                            if (c < p.ncols) {
                                const float gv = rbf((float)acc[r][c]);
                                const float u = rbf((float)acc[r + 1][c]);
                                const double gd = (double)gv;
                                const float z = rbf((float)(gd / (1.0 + exp(-gd))));
                                p.out[(size_t)(p.col0 + c) * p.out_ld + i] = f2bf(z * u);
                            }
                        }
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const int row = row0 + r;
                    if (row >= N) continue;
#pragma unroll
                    for (int c = 0; c < NC; c++) {
                        if (c >= p.ncols) continue;
                        const size_t col = (size_t)(p.col0 + c);
                        if (EPI == EPI_STORE) {
                            p.out[col * p.out_ld + row] = f2bf((float)acc[r][c]);
                        } else {   // EPI_RESIDUAL
                            const float y = rbf((float)acc[r][c]);
                            p.out[col * p.out_ld + row] = f2bf(xres[r][c] + y);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[r][c] = 0.0;
    };

    int b = 0;
    while (tile < p.geo.n_tiles) {
        // bufA holds (tile, b)
        int nt = tile, nbt = b + 1;
        if (nbt == NB) {
            nt = tile + n_waves;
            nbt = 0;
        }
        ready(bufA, scA, min(QB, Q - b * QB));
        if (nt < p.geo.n_tiles) issue(bufB, scB, nt, nbt);
        compute(bufA, scA, b);
        if (b == NB - 1) {
            finish_tile(tile);
            if (nt < p.geo.n_tiles) load_res(nt);
        }
        tile = nt;
        b = nbt;
        if (tile >= p.geo.n_tiles) break;
        // bufB holds (tile, b)
        nt = tile;
        nbt = b + 1;
        if (nbt == NB) {
            nt = tile + n_waves;
            nbt = 0;
        }
        ready(bufB, scB, min(QB, Q - b * QB));
        if (nt < p.geo.n_tiles) issue(bufA, scA, nt, nbt);
        compute(bufB, scB, b);
        if (b == NB - 1) {
            finish_tile(tile);
            if (nt < p.geo.n_tiles) load_res(nt);
        }
        tile = nt;
        b = nbt;
    }
}

}  // namespace mak

using namespace mak;

template <int R, int NC>
static const void* gemv4_fn_rnc(int epi)
{
    switch (epi) {
    case EPI_STORE: return reinterpret_cast<const void*>(&k_gemv4<R, NC, EPI_STORE>);
    case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemv4<R, NC, EPI_RESIDUAL>);
    case EPI_SWIGLU:
        if constexpr (R % 2 == 0) return reinterpret_cast<const void*>(&k_gemv4<R, NC, EPI_SWIGLU>);
        return nullptr;
    }
    return nullptr;
}

template <int R>
static const void* gemv4_fn_r(int nc, int epi)
{
    switch (nc) {
    case 1: return gemv4_fn_rnc<R, 1>(epi);
    case 2: return gemv4_fn_rnc<R, 2>(epi);
    case 4: return gemv4_fn_rnc<R, 4>(epi);
    case 8: return gemv4_fn_rnc<R, 8>(epi);
    }
    return nullptr;
}

// k_gemv4<r, nc, epi>, or nullptr when not compiled (nc in {1, 2, 4, 8};
// r in {1, 2}; SwiGLU needs r = 2; no LM-head form)
const void* mak_gemv4_fn(int r, int nc, int epi)
{
    switch (r) {
    case 1: return gemv4_fn_r<1>(nc, epi);
    case 2: return gemv4_fn_r<2>(nc, epi);
    }
    return nullptr;
}

// dynamic LDS of k_gemv4 for K inputs and nc staged columns
size_t mak_gemv4_lds(int k, int nc) { return (size_t)nc * pad32_stride(k) * sizeof(float); }

// Raise the dynamic-LDS ceiling of every k_gemv4 instantiation
hipError_t mak_gemv4_set_lds_limit(int bytes)
{
    for (int r : {1, 2})
        for (int nc : {1, 2, 4, 8})
            for (int epi : {(int)EPI_STORE, (int)EPI_RESIDUAL, (int)EPI_SWIGLU})
                if (const void* f = mak_gemv4_fn(r, nc, epi)) {
                    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
                    if (e != hipSuccess) return e;
                }
    return hipSuccess;
}
