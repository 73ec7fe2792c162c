// device_math.h -- number formats and fixed-tree reductions for the gfx950
// kernels.
//
// Rounding schedule: every dot product is accumulated in fp64 (products of
// two bf16 values are exact in fp64) and rounded once to fp32, then to bf16
// where a tensor is stored in bf16; exp/sqrt are evaluated in fp64 on fp32
// operands.  This reproduces eager bf16 execution op for op ("model-as-a-
// kernel", Method section) up to fp64 rounding, i.e. the bf16 decisions are
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

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// value of f rounded to bf16
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// fp64 sum over the 64 lanes of a wave; every lane gets the result.
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

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

}  // namespace mak
