// gemm16.hip -- the multi-column GEMMs of batched decode and prefill chunks on
// gfx950's fp64 matrix cores: y[c] = W x[c] for up to 16 columns.  k_gemm16
// (v_mfma_f64_16x16x4_f64) serves 9..16 columns; k_gemm8
// (v_mfma_f64_4x4x4_4b_f64, four independent 4x4 tiles per instruction)
// serves 2..8 columns with no padded half tile, and 9..16 columns of raw
// inputs on half-height tiles.  Both share the input staging.
//
// Every dot product of the decode path is exact in fp64 before its single
// rounding (bf16 x bf16 products are exact in fp64), so a column computed
// here rounds exactly as it does alone in the batch-1 kernels: the fp64
// multiply-adds move from the vector ALUs to v_mfma_f64_16x16x4f64, which
// issues alongside the VALU conversions instead of after them.  For 16
// columns a weight feeds 16 multiply-adds, about as many flops per byte as
// the fp64 matrix rate allows at the HBM rate ("model-as-a-kernel", Measured
// section: batching reuses each streamed weight for every sequence).
//
// Work split.  A workgroup of 8 waves owns RT output tiles of 16 rows x 16
// columns; its waves split K (blocks of 32 inputs) into 8 contiguous ranges
// and their partial tiles are summed through LDS in wave order.  Inside a
// 32-input block, lane l (k-group g = l / 16, tile row index i = l % 16)
// holds the 16-byte chunk 4*blk + g of weight row rho(i) and of input column
// i; MFMA step t (t = 0..7) multiplies element t of both, so step t covers
// inputs 32*blk + 8*g + t of the four k-groups.  The result register r of
// lane l is tile row index l/16 + 4r, column l % 16 (measured on the
// device); rho(i) = 4*(i % 4) + i / 4 turns that into the four consecutive
// rows 4*(l/16) .. +3 of one column, so stores are contiguous and gate/up
// row pairs (SwiGLU) sit in one lane.
//
// Inputs: RMSNorm inputs (K <= 4096) are normalised once per workgroup into
// LDS as [chunk][column] (17 slots per chunk: conflict-free reads); raw
// inputs are read by each wave from global memory (L2) for its own K range.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_math.h"
#include "gemv_kernels.h"
#include "mak_internal.h"

namespace mak {

typedef double d4_t __attribute__((ext_vector_type(4)));

// waves per workgroup: 16 for one row tile with RMSNorm inputs staged in LDS
// (K split 16 ways: four waves per SIMD keep the matrix cores busy while the
// staged inputs fill a CU's LDS, and each wave normalises one column), 8
// otherwise (two or four tiles need the registers of two waves per SIMD;
// with raw inputs, 16 waves measured slower: TinyLlama O 9.3 -> 10.6 us,
// down 18.7 -> 21.0 us at 16 columns)
__host__ __device__ constexpr int gemm16_waves(int rt, bool staged) { return (rt == 1 && staged) ? 16 : 8; }
constexpr int kG16Slots = 17;   // LDS slots (16 bytes) per input chunk: 16 columns + 1 pad

__host__ __device__ inline size_t gemm16_input_lds(int k) { return (size_t)(k >> 3) * kG16Slots * 16; }
__host__ __device__ inline size_t gemm16_part_lds(int rt, bool staged)
{
    return (size_t)gemm16_waves(rt, staged) * rt * 4 * 64 * 8;
}

// 8 bf16 values of a 16-byte chunk as fp64
__device__ __forceinline__ void chunk_f64(const uint4 v, double (&d)[8])
{
    d[0] = bf_lo(v.x);
    d[1] = bf_hi(v.x);
    d[2] = bf_lo(v.y);
    d[3] = bf_hi(v.y);
    d[4] = bf_lo(v.z);
    d[5] = bf_hi(v.z);
    d[6] = bf_lo(v.w);
    d[7] = bf_hi(v.w);
}

// RMSNorm inputs of up to 16 columns into LDS as [chunk][column]
// (kG16Slots slots per chunk, the last holding the norm weight's chunk):
// wave w normalises columns w, w + NWAVES, ..., one at a time; lane chunks
// lane + 64*i.  Inactive columns are stored as zeros.  Global loads already
// in flight (a weight batch) stay in flight: the barriers fence LDS only.
template <int NWAVES>
__device__ __forceinline__ void gemm_stage_inputs(const GemvPhase& p, uint4* hsT, int lane, int wave)
{
    const int K = p.geo.k, C = K >> 3;
    constexpr int SI = 8;                               // chunks per lane (K <= 4096)
    const int n_i = (C + 63) >> 6;
    const bool gather = p.in_kind == IN_GATHER_NORM;
    const uint4* nw = reinterpret_cast<const uint4*>(p.norm_w);
    // the norm weight is loaded once per workgroup (thread i: chunk i)
    // into the pad slot of each staged chunk; every wave then reads it
    // from LDS instead of loading all K of it for each of its columns
    const bool w_ld = (int)threadIdx.x < C;
    const uint4 wv = w_ld ? nw[threadIdx.x] : make_uint4(0, 0, 0, 0);
    uint4 sv[16 / NWAVES][SI];
    double ss[16 / NWAVES];
#pragma unroll
    for (int h = 0; h < 16 / NWAVES; h++) {
        const int cw = wave + NWAVES * h;
        const int col = p.col0 + min(cw, p.ncols - 1);
        const uint4* base = gather ? reinterpret_cast<const uint4*>(p.embed)
                                   : reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
        const int token = gather ? p.ctl->cols[col].token : 0;
#pragma unroll
        for (int i = 0; i < SI; i++) {
            if (i < n_i) {
                const int q = min(lane + 64 * i, C - 1);
                sv[h][i] = base[gather ? packed_chunk(p.embed_geo, token, q) : (int64_t)q];
            }
        }
    }
    if (w_ld) hsT[threadIdx.x * kG16Slots + 16] = wv;
#pragma unroll
    for (int h = 0; h < 16 / NWAVES; h++) {
        double a2 = 0.0;
#pragma unroll
        for (int i = 0; i < SI; i++) {
            if (i < n_i && lane + 64 * i < C) {
                const uint32_t u[4] = {sv[h][i].x, sv[h][i].y, sv[h][i].z, sv[h][i].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double x0 = bf_lo(u[e]), x1 = bf_hi(u[e]);
                    a2 = fma(x0, x0, a2);
                    a2 = fma(x1, x1, a2);
                }
            }
        }
        ss[h] = wave_sum(a2);
    }
    lds_barrier();   // the norm weight in LDS (the weight batch stays in flight)
#pragma unroll
    for (int h = 0; h < 16 / NWAVES; h++) {
        const int cw = wave + NWAVES * h;
        const bool active = cw < p.ncols;
        const float rs = rms_scale(ss[h], K, p.eps);
        const bool store_x = active && p.in_kind == IN_GATHER_NORM && blockIdx.x == 0;
        uint4* xs = reinterpret_cast<uint4*>(p.x_store + (size_t)(p.col0 + cw) * p.x_ld);
#pragma unroll
        for (int i = 0; i < SI; i++) {
            const int q = lane + 64 * i;
            if (i < n_i && q < C) {
                if (store_x) xs[q] = sv[h][i];
                const uint4 sw = hsT[q * kG16Slots + 16];
                const uint32_t u[4] = {sv[h][i].x, sv[h][i].y, sv[h][i].z, sv[h][i].w};
                const uint32_t ww[4] = {sw.x, sw.y, sw.z, sw.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    o[e] = rms_apply2(u[e], rs, ww[e]);
                }
                hsT[q * kG16Slots + cw] =
                    active ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
            }
        }
    }
    lds_barrier();   // (LDS only: the weight batch stays in flight)
}

template <int RT, int EPI, bool STAGED>
__global__ __launch_bounds__(gemm16_waves(RT, STAGED) * 64, RT == 1 ? 4 : 2) void k_gemm16(GemvPhase p)
{
    constexpr int kG16Waves = gemm16_waves(RT, STAGED);
    constexpr int QB = 2;                   // 32-input blocks per batch (RT = 1: 4 waves per SIMD)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float bval[kG16Waves][16];
    __shared__ int bidx[kG16Waves][16];
    __shared__ int is_last;

    const int K = p.geo.k, C = K >> 3;
    const int KB = (C + 3) >> 2;                       // 32-input blocks
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = lane >> 4;                          // k-group
    const int ti = lane & 15;                          // tile row index (A) / column (B)
    const int rho = 4 * (ti & 3) + (ti >> 2);          // tile row loaded for index ti
    constexpr bool staged = STAGED;                    // RMSNorm inputs staged in LDS (else raw inputs)
    uint4* hsT = reinterpret_cast<uint4*>(smem);

    // this wave's K range (contiguous blocks)
    const int kb0 = (int)((int64_t)wave * KB / kG16Waves);
    const int kb1 = (int)((int64_t)(wave + 1) * KB / kG16Waves);
    const int nkb = kb1 - kb0;
    const int NB = (nkb + QB - 1) / QB;                // batches per tile group

    // packed-layout geometry
    const int lrl = p.geo.lr_log2, lr = 1 << lrl;
    const int G = 64 >> lrl, R = p.geo.r;
    const int rl = (R == 4) ? 2 : (R == 2) ? 1 : 0;
    const int gl = 6 - lrl;                             // log2(G)
    const int J = C >> lrl;
    const int n_pad = p.geo.n_tiles * G * R;            // rows present in the packed matrix
    const int N = p.geo.n_rows;
    const uint4* W = reinterpret_cast<const uint4*>(p.w);
    const int n_groups = (N + 16 * RT - 1) / (16 * RT);
    const int rounds = (n_groups + (int)gridDim.x - 1) / (int)gridDim.x;
    // partial tiles: after the staged inputs, or over them when every
    // workgroup runs a single round (the inputs are then dead once the
    // MFMAs are done)
    const bool alias = rounds == 1;
    double* part = reinterpret_cast<double*>(smem + (staged && !alias ? gemm16_input_lds(K) : 0));

    // row part of the packed address of each of this lane's rows
    int64_t rbase[RT];
    auto set_rows = [&](int grp_idx) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            int row = (grp_idx * RT + rt) * 16 + rho;
            if (row >= n_pad) row = 0;                   // (padding beyond the matrix: result unused)
            const int tile = row >> (gl + rl);
            const int rr = row & ((G * R) - 1);
            const int grp = rr >> rl, ri = rr & (R - 1);
            rbase[rt] = ((int64_t)tile * J * R + ri) * 64 + grp * lr;
        }
    };
    auto a_addr = [&](int rt, int c) __attribute__((always_inline)) {
        const int j = c >> lrl, s = c & (lr - 1);
        return rbase[rt] + (int64_t)j * R * 64 + s;
    };
    // input column of this lane for raw inputs
    const int col_b = min(ti, p.ncols - 1);
    const bool col_ok = ti < p.ncols;
    const uint4* xin = reinterpret_cast<const uint4*>(p.in + (size_t)(p.col0 + col_b) * p.in_ld);

    // one batch: per block q, RT weight chunks then (raw inputs) the input
    // chunk, at [q * (RT + 1) + rt] and [q * (RT + 1) + RT]
    constexpr int QL = QB * (RT + 1);
    uint4 bufA[QL], bufB[QL];
    auto issue = [&](uint4 (&buf)[QL], int bt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QB; q++) {
            const int kb = kb0 + min(bt * QB + q, max(nkb - 1, 0));
            const int c = min(4 * kb + kg, C - 1);
#pragma unroll
            for (int rt = 0; rt < RT; rt++) buf[q * (RT + 1) + rt] = ld_stream16(&W[a_addr(rt, c)]);
            if constexpr (STAGED) buf[q * (RT + 1) + RT] = make_uint4(0, 0, 0, 0);
            else buf[q * (RT + 1) + RT] = xin[c];
        }
    };

    // 1. the first weight batch, then the input staging (RMSNorm inputs):
    //    wave w normalises columns w, w + waves, ..., one at a time; lane
    //    chunks lane + 64*i.  The weights stay in flight throughout.
    int grp_idx = blockIdx.x;
    set_rows(grp_idx);
    if (NB > 0) issue(bufA, 0);
    if constexpr (STAGED) gemm_stage_inputs<kG16Waves>(p, hsT, lane, wave);

    float best_v = -INFINITY;
    int best_i = 0x7fffffff;

    // 2. one batch: QB blocks x RT tiles x 8 MFMA steps.  All operands of a
    //    block are converted first; steps rotate over 4/RT
    //    accumulators per tile, so consecutive MFMAs do not wait on each other
    constexpr int CH = 4 / RT;                          // accumulator chains per tile (RT tiles interleave too)
    d4_t acc[RT][CH];
    auto compute = [&](const uint4 (&buf)[QL], int bt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QB; q++) {
            if (bt * QB + q >= nkb) break;               // wave-uniform
            const int kb = kb0 + bt * QB + q;
            const int c = 4 * kb + kg;
            uint4 bv;
            if constexpr (STAGED) bv = hsT[min(c, C - 1) * kG16Slots + ti];
            else bv = buf[q * (RT + 1) + RT];
            const bool live = c < C && (STAGED || col_ok);
            bv = make_uint4(live ? bv.x : 0u, live ? bv.y : 0u, live ? bv.z : 0u, live ? bv.w : 0u);
            double bd[8], ad[RT][8];
            chunk_f64(bv, bd);
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                const uint4 av = buf[q * (RT + 1) + rt];
                const bool in_k = c < C;
                chunk_f64(make_uint4(in_k ? av.x : 0u, in_k ? av.y : 0u, in_k ? av.z : 0u, in_k ? av.w : 0u), ad[rt]);
            }
#pragma unroll
            for (int t = 0; t < 8; t++)
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
                    acc[rt][t % CH] = __builtin_amdgcn_mfma_f64_16x16x4f64(ad[rt][t], bd[t], acc[rt][t % CH], 0, 0, 0);
        }
    };

    for (int round = 0; round < rounds; round++) {
        const bool have = grp_idx < n_groups;
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int ch = 0; ch < CH; ch++) acc[rt][ch] = (d4_t){0.0, 0.0, 0.0, 0.0};
        // batches ping-pong between two buffers: once one has landed the
        // next is issued, then the landed one is folded
        for (int bt = 0; bt < NB; bt += 2) {
            batch_ready<QL>(bufA, QL);
            if (bt + 1 < NB) issue(bufB, bt + 1);
            compute(bufA, bt);
            if (bt + 1 >= NB) break;
            batch_ready<QL>(bufB, QL);
            if (bt + 2 < NB) issue(bufA, bt + 2);
            compute(bufB, bt + 1);
        }
        // the next round's rows and first batch go out before the reduction
        const int next_grp = grp_idx + (int)gridDim.x;
        if (round + 1 < rounds) {
            set_rows(min(next_grp, n_groups - 1));
            if (NB > 0) issue(bufA, 0);
        }
        // 3. partial tiles of the 8 waves summed in wave order by wave rt
        if (staged && alias) lds_barrier();              // every wave is done reading the inputs
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                double v = acc[rt][0][r];
#pragma unroll
                for (int ch = 1; ch < CH; ch++) v += acc[rt][ch][r];
                part[((size_t)(wave * RT + rt) * 4 + r) * 64 + lane] = v;
            }
        lds_barrier();
        if (wave < RT && have) {
            const int rt = wave;
            double y[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                double s = 0.0;
#pragma unroll 4
                for (int w2 = 0; w2 < kG16Waves; w2++) s += part[((size_t)(w2 * RT + rt) * 4 + r) * 64 + lane];
                y[r] = s;
            }
            const int row0 = (grp_idx * RT + rt) * 16 + 4 * kg;   // rows row0 .. row0 + 3, column ti
            const int c = ti;
            if (c < p.ncols) {
                const size_t col = (size_t)(p.col0 + c);
                if (EPI == EPI_SWIGLU) {
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        if (row0 + r + 1 < N) {
                            const float gv = rbf((float)y[r]);
                            const float uv = rbf((float)y[r + 1]);
                            const double gd = (double)gv;
                            const float z = rbf((float)(gd / (1.0 + exp(-gd))));
                            p.out[col * p.out_ld + ((row0 + r) >> 1)] = f2bf(z * uv);
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int row = row0 + r;
                        if (row >= N) continue;
                        if (EPI == EPI_STORE) {
                            p.out[col * p.out_ld + row] = f2bf((float)y[r]);
                        } else if (EPI == EPI_RESIDUAL) {
                            const float xr = bf2f(p.out[col * p.out_ld + row]);
                            p.out[col * p.out_ld + row] = f2bf(xr + rbf((float)y[r]));
                        } else {   // EPI_LOGITS
                            const float v = (float)y[r];
                            p.logits[(size_t)c * p.logits_ld + row] = v;
                            if (v > best_v || (v == best_v && row < best_i)) {
                                best_v = v;
                                best_i = row;
                            }
                        }
                    }
                }
            }
        }
        lds_barrier();   // `part` is rewritten by the next round
        grp_idx = next_grp;
    }

    if (EPI == EPI_LOGITS) {
        // per-lane bests belong to column lane % 16: spread them into the
        // per-column form of the greedy argmax tail
        float bv[16];
        int bi[16];
#pragma unroll
        for (int c = 0; c < 16; c++) {
            bv[c] = (c == ti) ? best_v : -INFINITY;
            bi[c] = (c == ti) ? best_i : 0x7fffffff;
        }
        argmax_tail<16>(p, bv, bi, bval, bidx, is_last, lane, wave, kG16Waves);
    }
}


// ---------------------------------------------------------------------------
// k_gemm8: 2..8 columns on v_mfma_f64_4x4x4_4b_f64 (four independent 4x4x4
// products per instruction), so no half of the matrix tile is padding.
// Lane l (k-group kg = l / 16, block bq = (l / 4) % 4, e = l % 4) supplies
// element t of the 16-byte chunk 4*blk + kg of tile row l % 16 as A (row e
// of block bq) and of input column e (+4) as B; its result register is row
// kg of block bq, column e (measured on the device), i.e. tile row
// 4*bq + kg.  Two instructions per step share A: columns 0..3 and 4..7.
// Work split, staging, K split over waves, the reduction in wave order and
// the epilogues are those of k_gemm16.  Gate/up row pairs (2m, 2m + 1) sit
// in lanes l and l ^ 16.
// ---------------------------------------------------------------------------
__host__ __device__ inline size_t gemm8_part_lds(int rt, bool staged, int ng)
{
    return (size_t)gemm16_waves(rt, staged) * rt * ng * 64 * 8;
}

// HALF: tiles of 8 rows, twice the row groups of a short matrix.  Blocks
// b and b + 2 take the same rows 4*(b % 2) .. +3 over two consecutive
// 32-input blocks, and lanes l and l ^ 8 add their halves before the
// cross-wave sum.
// NG: groups of 4 columns (2: up to 8 columns; 4: up to 16, raw inputs on
// half-height tiles), each one instruction per step sharing A.
template <int RT, int EPI, bool STAGED, bool HALF = false, int NG = 2>
__global__ __launch_bounds__(gemm16_waves(RT, STAGED) * 64, (RT == 1 && STAGED) ? 4 : 2) void k_gemm8(GemvPhase p)
{
    constexpr int kW = gemm16_waves(RT, STAGED);
    constexpr int QB = 2;                   // 32-input blocks per batch
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float bval[kW][4 * NG];
    __shared__ int bidx[kW][4 * NG];
    __shared__ int is_last;

    const int K = p.geo.k, C = K >> 3;
    const int KB = (C + 3) >> 2;                       // 32-input blocks
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = lane >> 4;                          // k-group (A, B) / result row in block
    const int bq = (lane >> 2) & 3, e = lane & 3;      // block, column (B, result)
    constexpr int TR = HALF ? 8 : 16;                  // rows per tile
    const int ti = HALF ? 4 * (bq & 1) + e : lane & 15;   // tile row loaded (A)
    const int kh = HALF ? bq >> 1 : 0;                 // HALF: which block of a pair
    uint4* hsT = reinterpret_cast<uint4*>(smem);

    const int kb0 = (int)((int64_t)wave * KB / kW);
    const int kb1 = (int)((int64_t)(wave + 1) * KB / kW);
    const int nkb = kb1 - kb0;
    const int NU = HALF ? (nkb + 1) >> 1 : nkb;        // steps: blocks, or pairs of blocks
    const int NB = (NU + QB - 1) / QB;

    const int lrl = p.geo.lr_log2, lr = 1 << lrl;
    const int G = 64 >> lrl, R = p.geo.r;
    const int rl = (R == 4) ? 2 : (R == 2) ? 1 : 0;
    const int gl = 6 - lrl;
    const int J = C >> lrl;
    const int n_pad = p.geo.n_tiles * G * R;
    const int N = p.geo.n_rows;
    const uint4* W = reinterpret_cast<const uint4*>(p.w);
    const int n_groups = (N + TR * RT - 1) / (TR * RT);
    const int rounds = (n_groups + (int)gridDim.x - 1) / (int)gridDim.x;
    const bool alias = rounds == 1;
    double* part = reinterpret_cast<double*>(smem + (STAGED && !alias ? gemm16_input_lds(K) : 0));

    int64_t rbase[RT];
    auto set_rows = [&](int grp_idx) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            int row = (grp_idx * RT + rt) * TR + ti;
            if (row >= n_pad) row = 0;                   // (padding beyond the matrix: result unused)
            const int tile = row >> (gl + rl);
            const int rr = row & ((G * R) - 1);
            const int grp = rr >> rl, ri = rr & (R - 1);
            rbase[rt] = ((int64_t)tile * J * R + ri) * 64 + grp * lr;
        }
    };
    auto a_addr = [&](int rt, int c) __attribute__((always_inline)) {
        const int j = c >> lrl, s = c & (lr - 1);
        return rbase[rt] + (int64_t)j * R * 64 + s;
    };
    // raw inputs: this lane's columns e, e + 4, ...
    bool col_ok[NG];
    const uint4* xin[NG];
#pragma unroll
    for (int h = 0; h < NG; h++) {
        col_ok[h] = e + 4 * h < p.ncols;
        xin[h] = reinterpret_cast<const uint4*>(p.in + (size_t)(p.col0 + min(e + 4 * h, p.ncols - 1)) * p.in_ld);
    }

    // one batch: per block q, RT weight chunks, then (raw inputs) the NG
    // input chunks, at [q * (RT + NG) + rt] and [q * (RT + NG) + RT + h]
    constexpr int QL = QB * (RT + NG);
    uint4 bufA[QL], bufB[QL];
    auto issue = [&](uint4 (&buf)[QL], int bt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QB; q++) {
            const int u = HALF ? 2 * (bt * QB + q) + kh : bt * QB + q;
            const int kb = kb0 + min(u, max(nkb - 1, 0));
            const int c = min(4 * kb + kg, C - 1);
#pragma unroll
            for (int rt = 0; rt < RT; rt++) buf[q * (RT + NG) + rt] = ld_stream16(&W[a_addr(rt, c)]);
#pragma unroll
            for (int h = 0; h < NG; h++)
                buf[q * (RT + NG) + RT + h] = STAGED ? make_uint4(0, 0, 0, 0) : xin[h][c];
        }
    };

    int grp_idx = blockIdx.x;
    set_rows(grp_idx);
    if (NB > 0) issue(bufA, 0);
    if constexpr (STAGED) gemm_stage_inputs<kW>(p, hsT, lane, wave);

    float best_v[NG];
    int best_i[NG];
#pragma unroll
    for (int h = 0; h < NG; h++) {
        best_v[h] = -INFINITY;
        best_i[h] = 0x7fffffff;
    }

    // one batch: QB blocks x RT tiles x 8 steps x 2 column halves; the
    // steps rotate over CH accumulators per (tile, half)
    constexpr int CH = 8 / (RT * NG) > 1 ? 8 / (RT * NG) : 1;
    double acc[RT][NG][CH];
    auto compute = [&](const uint4 (&buf)[QL], int bt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QB; q++) {
            if (bt * QB + q >= NU) break;                // wave-uniform
            const int u = HALF ? 2 * (bt * QB + q) + kh : bt * QB + q;
            const int kb = kb0 + u;
            const int c = 4 * kb + kg;
            const bool in_k = c < C && u < nkb;
            double bd[NG][8], ad[RT][8];
#pragma unroll
            for (int h = 0; h < NG; h++) {
                uint4 bv = STAGED ? hsT[min(c, C - 1) * kG16Slots + e + 4 * h] : buf[q * (RT + NG) + RT + h];
                const bool live = in_k && (STAGED || col_ok[h]);
                bv = make_uint4(live ? bv.x : 0u, live ? bv.y : 0u, live ? bv.z : 0u, live ? bv.w : 0u);
                chunk_f64(bv, bd[h]);
            }
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                const uint4 av = buf[q * (RT + NG) + rt];
                chunk_f64(make_uint4(in_k ? av.x : 0u, in_k ? av.y : 0u, in_k ? av.z : 0u, in_k ? av.w : 0u), ad[rt]);
            }
#pragma unroll
            for (int t = 0; t < 8; t++)
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int h = 0; h < NG; h++)
                        acc[rt][h][t % CH] = __builtin_amdgcn_mfma_f64_4x4x4f64(ad[rt][t], bd[h][t], acc[rt][h][t % CH], 0, 0, 0);
        }
    };

    for (int round = 0; round < rounds; round++) {
        const bool have = grp_idx < n_groups;
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int h = 0; h < NG; h++)
#pragma unroll
                for (int ch = 0; ch < CH; ch++) acc[rt][h][ch] = 0.0;
        for (int bt = 0; bt < NB; bt += 2) {
            batch_ready<QL>(bufA, QL);
            if (bt + 1 < NB) issue(bufB, bt + 1);
            compute(bufA, bt);
            if (bt + 1 >= NB) break;
            batch_ready<QL>(bufB, QL);
            if (bt + 2 < NB) issue(bufA, bt + 2);
            compute(bufB, bt + 1);
        }
        const int next_grp = grp_idx + (int)gridDim.x;
        if (round + 1 < rounds) {
            set_rows(min(next_grp, n_groups - 1));
            if (NB > 0) issue(bufA, 0);
        }
        // partial tiles of the waves summed in wave order by wave rt
        if (STAGED && alias) lds_barrier();              // every wave is done reading the inputs
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int h = 0; h < NG; h++) {
                double v = acc[rt][h][0];
#pragma unroll
                for (int ch = 1; ch < CH; ch++) v += acc[rt][h][ch];
                if (HALF) v += __shfl_xor(v, 8, 64);     // the other block of the pair
                part[((size_t)(wave * RT + rt) * NG + h) * 64 + lane] = v;
            }
        lds_barrier();
        if (wave < RT && have && (!HALF || kh == 0 || EPI == EPI_SWIGLU)) {
            const int rt = wave;
            double y[NG];
#pragma unroll
            for (int h = 0; h < NG; h++) {
                double s = 0.0;
#pragma unroll 4
                for (int w2 = 0; w2 < kW; w2++) s += part[((size_t)(w2 * RT + rt) * NG + h) * 64 + lane];
                y[h] = s;
            }
            const int row = (grp_idx * RT + rt) * TR + (HALF ? 4 * (bq & 1) : 4 * bq) + kg;
            if (EPI == EPI_SWIGLU) {
                // rows 2m (gate, even kg) and 2m + 1 (up, lane ^ 16)
#pragma unroll
                for (int h = 0; h < NG; h++) {
                    const double yu = __shfl_xor(y[h], 16, 64);
                    const int c = e + 4 * h;
                    if (!(kg & 1) && kh == 0 && c < p.ncols && row + 1 < N) {
                        const float gv = rbf((float)y[h]);
                        const float uv = rbf((float)yu);
                        const double gd = (double)gv;
                        const float z = rbf((float)(gd / (1.0 + exp(-gd))));
                        p.out[(size_t)(p.col0 + c) * p.out_ld + (row >> 1)] = f2bf(z * uv);
                    }
                }
            } else if (row < N) {
#pragma unroll
                for (int h = 0; h < NG; h++) {
                    const int c = e + 4 * h;
                    if (c >= p.ncols) continue;
                    const size_t col = (size_t)(p.col0 + c);
                    if (EPI == EPI_STORE) {
                        p.out[col * p.out_ld + row] = f2bf((float)y[h]);
                    } else if (EPI == EPI_RESIDUAL) {
                        const float xr = bf2f(p.out[col * p.out_ld + row]);
                        p.out[col * p.out_ld + row] = f2bf(xr + rbf((float)y[h]));
                    } else {   // EPI_LOGITS
                        const float v = (float)y[h];
                        p.logits[(size_t)c * p.logits_ld + row] = v;
                        if (v > best_v[h] || (v == best_v[h] && row < best_i[h])) {
                            best_v[h] = v;
                            best_i[h] = row;
                        }
                    }
                }
            }
        }
        lds_barrier();   // `part` is rewritten by the next round
        grp_idx = next_grp;
    }

    if (EPI == EPI_LOGITS) {
        // per-lane bests belong to columns e, e + 4, ...
        float bv[4 * NG];
        int bi[4 * NG];
#pragma unroll
        for (int c = 0; c < 4 * NG; c++) {
            bv[c] = -INFINITY;
            bi[c] = 0x7fffffff;
#pragma unroll
            for (int h = 0; h < NG; h++)
                if (c == e + 4 * h) {
                    bv[c] = best_v[h];
                    bi[c] = best_i[h];
                }
        }
        argmax_tail<4 * NG>(p, bv, bi, bval, bidx, is_last, lane, wave, kW);
    }
}

}  // namespace mak

using namespace mak;

// The instantiated kernels: RMSNorm inputs (QKV, gate/up, LM head) and raw
// inputs (O, down); every epilogue is instantiated for both.
const void* mak_gemm16_fn(int rt, int epi, bool staged)
{
#define X(RT, S)                                                                                         \
    if (rt == RT && staged == S) {                                                                       \
        switch (epi) {                                                                                   \
        case EPI_STORE: return reinterpret_cast<const void*>(&k_gemm16<RT, EPI_STORE, S>);               \
        case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemm16<RT, EPI_RESIDUAL, S>);         \
        case EPI_SWIGLU: return reinterpret_cast<const void*>(&k_gemm16<RT, EPI_SWIGLU, S>);             \
        case EPI_LOGITS: return reinterpret_cast<const void*>(&k_gemm16<RT, EPI_LOGITS, S>);             \
        }                                                                                                \
    }
    X(1, true)
    X(2, true)
    X(4, true)
    X(1, false)
    X(2, false)
    X(4, false)
#undef X
    return nullptr;
}

// dynamic LDS of a k_gemm16 launch (single_round: the partial tiles reuse the
// staged inputs' space)
size_t mak_gemm16_lds(int rt, int k, bool staged, bool single_round)
{
    if (!staged) return gemm16_part_lds(rt, false);
    return single_round ? std::max(gemm16_input_lds(k), gemm16_part_lds(rt, true))
                        : gemm16_input_lds(k) + gemm16_part_lds(rt, true);
}

// workgroup size of k_gemm16 with rt row tiles (staged: RMSNorm inputs)
int mak_gemm16_threads(int rt, bool staged) { return gemm16_waves(rt, staged) * 64; }

const void* mak_gemm8_fn(int rt, int epi, bool staged, bool half, int ng)
{
    if (ng == 4) {   // 9..16 columns: one tile of 8 rows, raw inputs
        if (rt != 1 || staged || !half) return nullptr;
        switch (epi) {
        case EPI_STORE: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_STORE, false, true, 4>);
        case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_RESIDUAL, false, true, 4>);
        case EPI_SWIGLU: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_SWIGLU, false, true, 4>);
        case EPI_LOGITS: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_LOGITS, false, true, 4>);
        }
        return nullptr;
    }
    if (half) {   // one tile of 8 rows, raw inputs
        if (rt != 1 || staged) return nullptr;
        switch (epi) {
        case EPI_STORE: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_STORE, false, true>);
        case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_RESIDUAL, false, true>);
        case EPI_SWIGLU: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_SWIGLU, false, true>);
        case EPI_LOGITS: return reinterpret_cast<const void*>(&k_gemm8<1, EPI_LOGITS, false, true>);
        }
        return nullptr;
    }
#define X(RT, S)                                                                                         \
    if (rt == RT && staged == S) {                                                                       \
        switch (epi) {                                                                                   \
        case EPI_STORE: return reinterpret_cast<const void*>(&k_gemm8<RT, EPI_STORE, S>);                \
        case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemm8<RT, EPI_RESIDUAL, S>);          \
        case EPI_SWIGLU: return reinterpret_cast<const void*>(&k_gemm8<RT, EPI_SWIGLU, S>);              \
        case EPI_LOGITS: return reinterpret_cast<const void*>(&k_gemm8<RT, EPI_LOGITS, S>);              \
        }                                                                                                \
    }
    X(1, true)
    X(2, true)
    X(4, true)
    X(1, false)
    X(2, false)
#undef X
    return nullptr;   // (raw inputs take at most two row tiles: mak_gemm8_plan)
}

// dynamic LDS of a k_gemm8 launch (single_round: the partial tiles reuse the
// staged inputs' space)
size_t mak_gemm8_lds(int rt, int k, bool staged, bool single_round, int ng)
{
    if (!staged) return gemm8_part_lds(rt, false, ng);
    return single_round ? std::max(gemm16_input_lds(k), gemm8_part_lds(rt, true, ng))
                        : gemm16_input_lds(k) + gemm8_part_lds(rt, true, ng);
}
