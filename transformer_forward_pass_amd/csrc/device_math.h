// device_math.h -- number formats and fixed-tree reductions for the gfx950
// kernels.
//
// Rounding schedule: every dot product is accumulated in fp64 (products of
// two bf16 values are exact in fp64) and rounded once to fp32, then to bf16
// where a tensor is stored in bf16; exp/sqrt are evaluated in fp64 on fp32
// operands.  Each operation thus rounds as eager bf16 execution does
// ("model-as-a-kernel", Method section) up to fp64 rounding: the bf16 decisions are
// the same as an ascending-order exact evaluation except in vanishingly rare
// ties.  (fp32 accumulation was measured to flip enough bf16 roundings to
// move whole-model logits by ~1e-2 relative on the 135M shape.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mak {

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Weight streams: every weight byte is read once per step, so its loads carry
// the non-temporal hint (gfx950 `nt`, the caches' streaming policy) and leave
// the cache lines that later phases re-read -- KV rows, activations, the
// control block -- in place.  (Plain loads measured 7-9 % slower end to end
// at the Llama-3.2-1B shape.)
typedef unsigned stream_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p)
{
    const stream_u4 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream_u8(const unsigned char* p) { return __builtin_nontemporal_load(p); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN (sign
// and leading payload kept).  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32): over every fp32 bit pattern it gives exactly the
// integer rounding (u + 0x7fff + bit 16) >> 16, NaN -> (u >> 16) | 0x40.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two values in one conversion: lo in bits 0-15, hi in bits 16-31
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi)
{
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// value of f rounded to bf16
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// ---------------------------------------------------------------------------
// Cross-lane moves.  DPP lane moves are VALU instructions (a few cycles)
// where __shfl_xor goes through the LDS crossbar (ds_bpermute, ~100 cycles),
// so reductions use DPP inside a 16-lane row and the row-swap moves between
// rows.  64-bit values move as two 32-bit halves.
// ---------------------------------------------------------------------------
enum : int {
    DPP_XOR1 = 0xB1,        // quad_perm [1,0,3,2]
    DPP_XOR2 = 0x4E,        // quad_perm [2,3,0,1]
    DPP_HALF_MIRROR = 0x141,// lane i <-> 7-i within each 8 lanes
    DPP_MIRROR = 0x140,     // lane i <-> 15-i within each row of 16
    DPP_ROR4 = 0x124,       // rotate right by 4 within a row
    DPP_ROR8 = 0x128,       // rotate right by 8 within a row
};

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Across rows: gfx950's row-swap moves (v_permlane16_swap, v_permlane32_swap;
// VALU, no LDS crossbar).  With both operands equal, every lane receives the
// value of the lower and of the upper lane of its pair (lane, lane ^ 16) or
// (lane, lane ^ 32), in that order, so both lanes compute the same
// lower-plus-upper sum (equal to v + partner: addition commutes).
template <int DIST>
__device__ __forceinline__ void xor_pair_d(double v, double& lower, double& upper)
{
    static_assert(DIST == 16 || DIST == 32, "row-swap distances");
    const unsigned lo = (unsigned)__double2loint(v), hi = (unsigned)__double2hiint(v);
    if (DIST == 16) {
        const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        lower = __hiloint2double((int)h[0], (int)l[0]);
        upper = __hiloint2double((int)h[1], (int)l[1]);
    } else {
        const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        lower = __hiloint2double((int)h[0], (int)l[0]);
        upper = __hiloint2double((int)h[1], (int)l[1]);
    }
}

// v + (v at lane ^ DIST)
template <int DIST>
__device__ __forceinline__ double add_xor(double v)
{
    double a, b;
    xor_pair_d<DIST>(v, a, b);
    return a + b;
}

// v at lane ^ DIST
template <int DIST>
__device__ __forceinline__ double get_xor(double v)
{
    double a, b;
    xor_pair_d<DIST>(v, a, b);
    return (threadIdx.x & DIST) ? a : b;
}

// max(v, v at lane ^ DIST)
template <int DIST>
__device__ __forceinline__ float max_xor(float v)
{
    static_assert(DIST == 16 || DIST == 32, "row-swap distances");
    const unsigned u = __float_as_uint(v);
    const auto p = (DIST == 16) ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Sum over aligned groups of 2^LOG lanes (LOG <= 6); every lane of a group
// gets the group's sum (the same tree in every group).
template <int LOG>
__device__ __forceinline__ double group_sum(double v)
{
    if (LOG >= 1) v += dpp_d<DPP_XOR1>(v);
    if (LOG >= 2) v += dpp_d<DPP_XOR2>(v);
    if (LOG >= 3) v += dpp_d<DPP_HALF_MIRROR>(v);
    if (LOG >= 4) v += dpp_d<DPP_MIRROR>(v);
    if (LOG >= 5) v = add_xor<16>(v);
    if (LOG >= 6) v = add_xor<32>(v);
    return v;
}

// Runtime group size (1 << log), log <= 6.
__device__ __forceinline__ double group_sum_rt(double v, int log)
{
    if (log >= 1) v += dpp_d<DPP_XOR1>(v);
    if (log >= 2) v += dpp_d<DPP_XOR2>(v);
    if (log >= 3) v += dpp_d<DPP_HALF_MIRROR>(v);
    if (log >= 4) v += dpp_d<DPP_MIRROR>(v);
    if (log >= 5) v = add_xor<16>(v);
    if (log >= 6) v = add_xor<32>(v);
    return v;
}

// group_sum_rt over N values at once, level by level, so the cross-lane
// moves of different values overlap instead of waiting on each other.
template <int N>
__device__ __forceinline__ void group_sum_all(double (&v)[N], int log)
{
    if (log >= 1) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] += dpp_d<DPP_XOR1>(v[i]);
    }
    if (log >= 2) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] += dpp_d<DPP_XOR2>(v[i]);
    }
    if (log >= 3) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] += dpp_d<DPP_HALF_MIRROR>(v[i]);
    }
    if (log >= 4) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] += dpp_d<DPP_MIRROR>(v[i]);
    }
    if (log >= 5) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = add_xor<16>(v[i]);
    }
    if (log >= 6) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = add_xor<32>(v[i]);
    }
}

template <int LOG>
__device__ __forceinline__ float group_max(float v)
{
    if (LOG >= 1) v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    if (LOG >= 2) v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    if (LOG >= 3) v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    if (LOG >= 4) v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
    if (LOG >= 5) v = max_xor<16>(v);
    if (LOG >= 6) v = max_xor<32>(v);
    return v;
}

// Sum over lanes with equal (lane mod 2^LOG): the "stride" reduction that
// folds lane groups of 2^LOG lanes onto each other.  Lanes of one residue
// may differ in the last bit (association order); read one fixed lane.
template <int LOG>
__device__ __forceinline__ double stride_sum(double v)
{
    static_assert(LOG >= 1 && LOG <= 5, "stride 2..32");
    if (LOG <= 1) v += dpp_d<0x122>(v);   // row_ror:2
    if (LOG <= 2) v += dpp_d<DPP_ROR4>(v);
    if (LOG <= 3) v += dpp_d<DPP_ROR8>(v);
    if (LOG <= 4) v = add_xor<16>(v);
    v = add_xor<32>(v);
    return v;
}

// fp64 sum over the 64 lanes of a wave; every lane gets the result.
__device__ __forceinline__ double wave_sum(double v) { return group_sum<6>(v); }

__device__ __forceinline__ float wave_max(float v) { return group_max<6>(v); }

// Block-wide fp64 sum (MAK_BLOCK threads); `red` holds >= 4 doubles of LDS.
// Waves are combined in wave order, so the tree is fixed.
__device__ __forceinline__ double block_sum(double v, double* red)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = ((red[0] + red[1]) + red[2]) + red[3];
    return s;
}

// Block-wide fp64 sum over NW waves, combined in wave order.
template <int NW>
__device__ __forceinline__ double block_sum_n(double v, double* red)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) s += red[i];
    return s;
}

// Block-wide fp64 sum over nw waves (runtime), combined in wave order.
__device__ __forceinline__ double block_sum_rt(double v, double* red, int nw)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = red[0];
    for (int i = 1; i < nw; i++) s += red[i];
    return s;
}

// Workgroup barrier that orders LDS only: global loads still in flight stay
// in flight (a plain __syncthreads also fences global memory, so the
// compiler first drains every outstanding vector load).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// block_sum_rt with LDS-only barriers (a GEMV's input statistics, while its
// first weight batch is still arriving)
__device__ __forceinline__ double block_sum_lds(double v, double* red, int nw)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    lds_barrier();
    double s = red[0];
    for (int i = 1; i < nw; i++) s += red[i];
    return s;
}

__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// RMSNorm scale r = fp32(1 / sqrt(fp32(fp32(ss / n) + eps))) from the fp64
// sum of squares ss ("Building a GPU compiler from scratch ... (Emmy)",
// Tensor IR section: mean of squares, plus epsilon, inverse square root).
__device__ __forceinline__ float rms_scale(double ss, int n, float eps)
{
    float ms = (float)(ss / (double)n);
    float v = ms + eps;
    return (float)(1.0 / sqrt((double)v));
}

// normalised element: bf16(w * bf16(x * r))
__device__ __forceinline__ uint16_t rms_apply(float x, float r, float w)
{
    return f2bf(w * rbf(x * r));
}

// two normalised elements (the bf16 pair u, weights ww) packed as a bf16 pair
__device__ __forceinline__ uint32_t rms_apply2(uint32_t u, float r, uint32_t ww)
{
    const uint32_t t = f2bf2(bf_lo(u) * r, bf_hi(u) * r);
    return f2bf2(bf_lo(ww) * bf_lo(t), bf_hi(ww) * bf_hi(t));
}

}  // namespace mak
