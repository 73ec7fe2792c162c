// gemv_kernels.h -- the packed-weight GEMV of the decode phases (gfx950).
//
// Weights stream once from HBM in a packed order (mak_internal.h) so that
// each wave instruction loads 1 KiB contiguous (16 B per lane).  The input
// vectors sit in LDS as bf16 (RMSNorm applied in the prologue where the phase
// starts with one); products and sums are fp64; each output row is reduced
// across the lanes that share it with a fixed tree; the epilogue stores bf16,
// adds the residual, applies SwiGLU to gate/up row pairs, or writes fp32
// logits and takes the greedy argmax.  No floating-point atomics: the only
// atomic is the integer ticket that elects the last workgroup of the LM head.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "mak_internal.h"

namespace mak {

// ---------------------------------------------------------------------------
// packed-layout addressing (16-byte units)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t packed_chunk(const PackGeom& g, int64_t row, int chunk)
{
    const int lr = 1 << g.lr_log2;
    const int G = 64 >> g.lr_log2;
    const int J = (g.k >> 3) >> g.lr_log2;
    const int64_t rows_per_tile = (int64_t)G * g.r;
    const int64_t tile = row / rows_per_tile;
    const int rr = (int)(row - tile * rows_per_tile);
    const int grp = rr / g.r, ri = rr - grp * g.r;
    const int j = chunk >> g.lr_log2, s = chunk & (lr - 1);
    return ((tile * J + j) * g.r + ri) * 64 + grp * lr + s;
}

// ---------------------------------------------------------------------------
// GEMV input staging: hs[c*K + k] for c < NC (columns >= ncols zero).
// issue_input() only starts the loads (into registers); finish_input()
// consumes them.  The weight stream is started in between, and since vector
// loads retire in order, waiting for the input never waits for the weights.
// ---------------------------------------------------------------------------
template <int NC>
struct Staged {
    static constexpr int QPT = (NC == 1) ? 4 : 2;   // 16-byte chunks per thread held in registers
    uint4 v[NC][QPT];                                // x or raw input
    uint4 w[2];                                      // norm weight (K <= 4096)
};

template <int NC>
__device__ __forceinline__ void issue_input(const GemvPhase& p, Staged<NC>& st, const int NT)
{
    constexpr int QPT = Staged<NC>::QPT;
    const int C = p.geo.k >> 3;
    const int tid = threadIdx.x;
    const uint4* src[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int col = p.col0 + c;
        src[c] = nullptr;
        if (c < p.ncols) {
            if (p.in_kind == IN_GATHER_NORM) src[c] = reinterpret_cast<const uint4*>(p.embed);
            else src[c] = reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
        }
    }
#pragma unroll
    for (int i = 0; i < QPT; i++) {
        const int q = tid + i * NT;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            if (q < C && src[c]) {
                if (p.in_kind == IN_GATHER_NORM)
                    st.v[c][i] = src[c][packed_chunk(p.embed_geo, p.ctl->cols[p.col0 + c].token, q)];
                else
                    st.v[c][i] = src[c][q];
            }
        }
        if (i < 2 && p.in_kind != IN_RAW && q < C) st.w[i] = reinterpret_cast<const uint4*>(p.norm_w)[q];
    }
}

// 8 bf16 inputs (one 16-byte chunk) as fp32 (exact) into LDS
__device__ __forceinline__ void store_chunk_f32(float* dst, uint4 v)
{
    float4* d = reinterpret_cast<float4*>(dst);
    d[0] = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
    d[1] = make_float4(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
}

// hs[c*K + k] as fp32 (bf16 values, exact): the fold then converts each
// input element to fp64 with one instruction.  PAD32 lays each column out in
// blocks of 32 inputs at a stride of 36 floats (the 4-bit GEMV reads one
// block per lane; the padding spreads neighbouring lanes' blocks over
// distinct LDS banks): input k of column c at hs[c*CS + (k/32)*36 + k%32]
// with CS = (K/32)*36.
__host__ __device__ constexpr int pad32_stride(int k) { return (k >> 5) * 36; }

template <bool PAD32>
__device__ __forceinline__ int stage_off(int q)   // float offset of 8-input chunk q
{
    return PAD32 ? (q >> 2) * 36 + (q & 3) * 8 : 8 * q;
}

template <int NC, bool PAD32 = false>
__device__ __forceinline__ void finish_input(const GemvPhase& p, Staged<NC>& st, float* hs, double* red,
                                             const int NT)
{
    constexpr int QPT = Staged<NC>::QPT;
    const int K = p.geo.k, C = K >> 3;
    const int tid = threadIdx.x;
    const size_t cs = PAD32 ? (size_t)pad32_stride(K) : (size_t)K;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        float* hc = hs + (size_t)c * cs;
        const int col = p.col0 + c;
        if (c >= p.ncols) {
            for (int q = tid; q < C; q += NT) store_chunk_f32(hc + stage_off<PAD32>(q), make_uint4(0, 0, 0, 0));
            continue;
        }
        if (p.in_kind == IN_RAW) {
#pragma unroll
            for (int i = 0; i < QPT; i++) {
                const int q = tid + i * NT;
                if (q < C) store_chunk_f32(hc + stage_off<PAD32>(q), st.v[c][i]);
            }
            // chunks beyond what the registers held (K > QPT*2048)
            const uint4* src = reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
            for (int q = tid + QPT * NT; q < C; q += NT) store_chunk_f32(hc + stage_off<PAD32>(q), src[q]);
            continue;
        }
        // RMSNorm of x: at most 2 chunks per thread (launches size the
        // workgroup so that 16 * NT >= K)
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int q = tid + i * NT;
            if (q < C) {
                if (p.in_kind == IN_GATHER_NORM && blockIdx.x == 0)
                    reinterpret_cast<uint4*>(p.x_store + (size_t)col * p.x_ld)[q] = st.v[c][i];
                const uint32_t u[4] = {st.v[c][i].x, st.v[c][i].y, st.v[c][i].z, st.v[c][i].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double a = bf_lo(u[e]), b = bf_hi(u[e]);
                    ss = fma(a, a, ss);
                    ss = fma(b, b, ss);
                }
            }
        }
        ss = block_sum_lds(ss, red, NT >> 6);
        const float r = rms_scale(ss, K, p.eps);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int q = tid + i * NT;
            if (q < C) {
                const uint32_t u[4] = {st.v[c][i].x, st.v[c][i].y, st.v[c][i].z, st.v[c][i].w};
                const uint32_t ww[4] = {st.w[i].x, st.w[i].y, st.w[i].z, st.w[i].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    o[e] = rms_apply2(u[e], r, ww[e]);
                }
                store_chunk_f32(hc + stage_off<PAD32>(q), make_uint4(o[0], o[1], o[2], o[3]));
            }
        }
        lds_barrier();  // `red` is reused by the next column
    }
}

// ---------------------------------------------------------------------------
// GEMV phase
// ---------------------------------------------------------------------------
// Greedy argmax of an LM-head launch: per-block partial (max, then lowest
// index), then the last block to finish (integer ticket) reduces every
// block's partial and feeds the chosen tokens back as the next step's columns.
template <int NC>
__device__ __forceinline__ void argmax_tail(const GemvPhase& p, const float* best_v, const int* best_i, float (*bval)[NC],
                            int (*bidx)[NC], int& is_last, int lane, int wave, const int NW)
{
    const int NT = NW * 64;
    // ---- greedy argmax: per-block partial, then the last block reduces ----
#pragma unroll
    for (int c = 0; c < NC; c++) {
        float v = best_v[c];
        int i = best_i[c];
        for (int o = 32; o > 0; o >>= 1) {
            const float v2 = __shfl_xor(v, o, 64);
            const int i2 = __shfl_xor(i, o, 64);
            if (v2 > v || (v2 == v && i2 < i)) {
                v = v2;
                i = i2;
            }
        }
        if (lane == 0) {
            bval[wave][c] = v;
            bidx[wave][c] = i;
        }
    }
    __syncthreads();
    if (threadIdx.x < NC) {
        const int c = threadIdx.x;
        float v = bval[0][c];
        int i = bidx[0][c];
        for (int w = 1; w < NW; w++) {
            if (bval[w][c] > v || (bval[w][c] == v && bidx[w][c] < i)) {
                v = bval[w][c];
                i = bidx[w][c];
            }
        }
        p.part_val[blockIdx.x * MAK_MAX_COLS + c] = v;
        p.part_idx[blockIdx.x * MAK_MAX_COLS + c] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned prev = atomicAdd(&p.ctl->ticket, 1u);
        is_last = (prev == (unsigned)(p.n_blocks - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    // the last block: reduce every block's partial (order-free: max, then
    // lowest index), one wave per column, then feed the chosen tokens back as
    // the next step's columns
    __shared__ int next_tok[MAK_MAX_COLS];
    for (int c = wave; c < p.ncols; c += NW) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        // sixteen partials per lane in flight at once (1024 blocks in one batch)
        for (int b0 = lane; b0 < p.n_blocks; b0 += 16 * 64) {
            float vv[16];
            int ii[16];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int b = b0 + 64 * u;
                vv[u] = (b < p.n_blocks) ? p.part_val[b * MAK_MAX_COLS + c] : -INFINITY;
                ii[u] = (b < p.n_blocks) ? p.part_idx[b * MAK_MAX_COLS + c] : 0x7fffffff;
            }
#pragma unroll
            for (int u = 0; u < 16; u++)
                if (vv[u] > v || (vv[u] == v && ii[u] < i)) {
                    v = vv[u];
                    i = ii[u];
                }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const float v2 = __shfl_xor(v, o, 64);
            const int i2 = __shfl_xor(i, o, 64);
            if (v2 > v || (v2 == v && i2 < i)) {
                v = v2;
                i = i2;
            }
        }
        if (lane == 0) next_tok[c] = (i == 0x7fffffff) ? 0 : i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // new column c takes over from column col0 + c >= c, so updating in
        // ascending order never overwrites a column still to be read
        Ctl* ctl = p.ctl;
        const int step = ctl->step;
        for (int c = 0; c < p.ncols; c++) {
            const ColState old = ctl->cols[p.col0 + c];
            if (p.out_tokens) p.out_tokens[step * p.ncols + c] = next_tok[c];
            ColState ns;
            ns.token = next_tok[c];
            ns.pos = old.pos + 1;
            ns.slot = old.slot;
            ns.first_pos = old.pos + 1;
            ns.first_col = c;
            ns.pad_[0] = ns.pad_[1] = ns.pad_[2] = 0;
            ctl->cols[c] = ns;
        }
        ctl->ncols = p.ncols;
        ctl->step = step + 1;
        ctl->ticket = 0;
        __threadfence();
    }
}

// Wait until every register of a batch holds its data, and keep later
// memory operations below this point.  (On gfx950 the compiler waits for all
// outstanding vector loads before using any of them, so the next batch may
// only be issued after this point if computing the current batch is not to
// wait for it.)
template <int QB>
__device__ __forceinline__ void batch_ready(const uint4 (&b)[QB], int n)
{
#pragma unroll
    for (int i = 0; i < QB; i++)
        if (i < n) asm volatile("" ::"v"(b[i].x), "v"(b[i].y), "v"(b[i].z), "v"(b[i].w) : "memory");
}

template <int R, int NC, int EPI>
__global__ __launch_bounds__(MAK_GBLOCK) void k_gemv(GemvPhase p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int NW = MAK_GBLOCK / 64;
    __shared__ double red[NW];
    __shared__ float bval[NW][NC];
    __shared__ int bidx[NW][NC];
    __shared__ int is_last;
    float* hs = reinterpret_cast<float*>(smem);

    const int K = p.geo.k;
    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps tile/batch bookkeeping in scalar registers, so the
    // batch loops are scalar branches rather than lane-masked ones
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int J = (K >> 3) >> lrl;
    const int Q = J * R;                       // 16-byte loads per lane per tile
    const uint4* W = reinterpret_cast<const uint4*>(p.w);
    const int n_waves = gridDim.x * (MAK_GBLOCK / 64);
    const int N = p.geo.n_rows;
    constexpr int QB = (NC <= 2) ? 16 : 8;     // loads per batch (a multiple of R)
    static_assert(QB % R == 0, "batch must hold whole row groups");
    const int NB = (Q + QB - 1) / QB;          // batches per tile

    // batch b of tile t: loads q = b*QB + i, i < min(QB, Q - b*QB)
    // (the batch base is wave-uniform, so it lives in scalar registers and
    // only the lane offset is per-lane)
    const uint32_t lane_off = (uint32_t)lane * 16u;
    auto issue = [&](uint4 (&buf)[QB], int t, int b) {
        const char* wt = reinterpret_cast<const char*>(W + ((int64_t)t * Q + (int64_t)b * QB) * 64);
        const int n = min(QB, Q - b * QB);
#pragma unroll
        for (int i = 0; i < QB; i++)
            if (i < n) buf[i] = ld_stream16(wt + (lane_off + (uint32_t)i * 1024u));
    };

    int tile = blockIdx.x * (MAK_GBLOCK / 64) + wave;

    // 1. this step's input, the residual rows of the first tile (lane s == 0
    //    owns rows row0 .. row0+R-1), then the first weight batch
    Staged<NC> stg;
    issue_input<NC>(p, stg, MAK_GBLOCK);
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
    if (tile < p.geo.n_tiles) {
        load_res(tile);
        issue(bufA, tile, 0);
    }

    // 2. stage the input (RMSNorm); this waits for the first batch as well
    finish_input<NC>(p, stg, hs, red, MAK_GBLOCK);
    __syncthreads();

    float best_v[NC];
    int best_i[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        best_v[c] = -INFINITY;
        best_i[c] = 0x7fffffff;
    }
    double acc[R][NC];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[r][c] = 0.0;

    // 3. fold one completed batch into the accumulators
    auto compute = [&](const uint4 (&buf)[QB], int b) {
        const int n = min(QB, Q - b * QB);
        double hdc[NC][8];
#pragma unroll
        for (int i = 0; i < QB; i++) {
            if (i < n) {
                constexpr int RR = R;
                const int r = i % RR;
                if (r == 0) {
                    const int chunk = (((b * QB + i) / RR) << lrl) + s;
#pragma unroll
                    for (int c = 0; c < NC; c++) {
                        const float4* h4 = reinterpret_cast<const float4*>(hs + (size_t)c * K) + 2 * chunk;
                        const float4 lo = h4[0], hi = h4[1];
                        hdc[c][0] = lo.x; hdc[c][1] = lo.y; hdc[c][2] = lo.z; hdc[c][3] = lo.w;
                        hdc[c][4] = hi.x; hdc[c][5] = hi.y; hdc[c][6] = hi.z; hdc[c][7] = hi.w;
                    }
                }
                const uint32_t wu[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const double wd = (e & 1) ? bf_hi(wu[e >> 1]) : bf_lo(wu[e >> 1]);
#pragma unroll
                    for (int c = 0; c < NC; c++) acc[r][c] = fma(wd, hdc[c][e], acc[r][c]);
                }
            }
        }
    };

    // 4. finish a tile: reduce each row over its lr lanes, then the epilogue
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
                                const float g = rbf((float)acc[r][c]);
                                const float u = rbf((float)acc[r + 1][c]);
                                const double gd = (double)g;
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
                        } else if (EPI == EPI_RESIDUAL) {
                            const float y = rbf((float)acc[r][c]);
                            p.out[col * p.out_ld + row] = f2bf(xres[r][c] + y);
                        } else {  // EPI_LOGITS
                            const float v = (float)acc[r][c];
                            p.logits[(size_t)c * p.logits_ld + row] = v;
                            if (v > best_v[c] || (v == best_v[c] && row < best_i[c])) {
                                best_v[c] = v;
                                best_i[c] = row;
                            }
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

    // 5. the wave's batches, ping-ponging between two buffers: once a batch has
    //    landed, the next one is issued and only then is the landed one used
    int b = 0;
    while (tile < p.geo.n_tiles) {
        // bufA holds (tile, b)
        int nt = tile, nbt = b + 1;
        if (nbt == NB) {
            nt = tile + n_waves;
            nbt = 0;
        }
        batch_ready<QB>(bufA, min(QB, Q - b * QB));
        if (nt < p.geo.n_tiles) issue(bufB, nt, nbt);
        compute(bufA, b);
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
        batch_ready<QB>(bufB, min(QB, Q - b * QB));
        if (nt < p.geo.n_tiles) issue(bufA, nt, nbt);
        compute(bufB, b);
        if (b == NB - 1) {
            finish_tile(tile);
            if (nt < p.geo.n_tiles) load_res(nt);
        }
        tile = nt;
        b = nbt;
    }

    if (EPI == EPI_LOGITS) argmax_tail<NC>(p, best_v, best_i, bval, bidx, is_last, lane, wave, NW);
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV with the tile shape fixed at compile time: QT = J*R loads per
// lane per tile, all issued as one straight-line batch.  Each wave walks its
// tiles with two batch buffers: once the current batch has landed (one wait),
// the next tile's batch is issued and only then is the current one folded, so
// the stream never stops while the wave computes.
// ---------------------------------------------------------------------------
// Waves per workgroup of k_gemv1<R, J>: 8, or 4 where two batch buffers of
// J*R loads need more registers than two waves per SIMD leave.
__host__ __device__ constexpr int gemv1_waves(int r, int j) { return r * j > 16 ? 4 : 8; }

// KS = 2 splits each tile's chunks over two waves (static path only: at
// most one tile per pair of waves): waves 2m and 2m+1 fold the first and
// second half of tile m's chunks, and the second hands its row sums to the
// first through LDS, which adds them (first half + second half) and applies
// the epilogue.  For odd J both halves issue the same number of loads (the
// second repeats the last chunk and skips it) so the waits stay exact.
template <int R, int J, int EPI, int KS = 1>
__global__ __launch_bounds__(gemv1_waves(R, J) * 64) void k_gemv1(GemvPhase p)
{
    static_assert(KS == 1 || KS == 2, "K split of 1 or 2");
    constexpr int QT = J * R;
    constexpr int JH = (J + KS - 1) / KS;                  // chunk iterations per wave
    constexpr int QH = JH * R;                             // loads per wave per tile
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int NW = gemv1_waves(R, J);
    __shared__ double red[NW];
    __shared__ float bval[NW][1];
    __shared__ int bidx[NW][1];
    __shared__ int tile_next;
    __shared__ int is_last;
    float* hs = reinterpret_cast<float*>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int n_tiles = p.geo.n_tiles;
    const int N = p.geo.n_rows;
    const int nw = blockDim.x >> 6;                        // <= NW (one tile per wave: 4)
    const int n_waves = gridDim.x * nw;
    const char* W = reinterpret_cast<const char*>(p.w);
    const uint32_t lane_off = (uint32_t)lane * 16u;

    // (issued in chunk order: an empty asm with a memory clobber keeps the
    // compiler from reordering them, so chunk i's wait leaves QT-1-i in flight)
    // (KS = 2: this wave's half of the chunks, the last repeated for odd J)
    const int half = (KS == 2) ? (wave & 1) : 0;
    auto issue = [&](uint4 (&buf)[QT], int t) {
        const char* wt = W + (int64_t)t * QT * 1024;
#pragma unroll
        for (int i = 0; i < QH; i++) {
            const int c = i / R;
            const int jj = (KS == 2) ? min(half * JH + c, J - 1) : c;
            buf[i] = ld_stream16(wt + lane_off + (jj * R + (i - c * R)) * 1024);
            asm volatile("" ::: "memory");
        }
    };

    // Tiles.  With at most one tile per wave: tile = global wave index.
    // Otherwise each workgroup owns a contiguous range of tiles and its waves
    // take them one at a time from an LDS counter, so waves that get more
    // of the CU's memory bandwidth do more tiles and all finish together
    // (which tile a wave computes does not change any result).
    const bool dyn = KS == 1 && n_tiles > n_waves;            // (KS = 2: the host launches >= 2 waves per tile)
    const int t_begin = dyn ? (int)((int64_t)blockIdx.x * n_tiles / gridDim.x) : 0;
    const int t_end = dyn ? (int)((int64_t)(blockIdx.x + 1) * n_tiles / gridDim.x) : n_tiles;
    int tile = dyn ? t_begin + wave : (blockIdx.x * nw + wave) / KS;   // dyn: each range holds >= nw tiles
    if (threadIdx.x == 0) tile_next = t_begin + nw;
    auto next_tile = [&](int t) __attribute__((always_inline)) {
        if (!dyn) return t + n_waves;
        int v = 0;
        if (lane == 0) v = atomicAdd(&tile_next, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };
    Staged<1> stg;
    issue_input<1>(p, stg, nw * 64);
    // every wave's input loads go out before any weight load of the
    // workgroup, so the input and its RMSNorm do not queue behind the CU's
    // first weight batches (a barrier without a fence: nothing waits for
    // the loads here; the empty asms keep the compiler from moving loads
    // across it)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    float xres[R];
    auto load_res = [&](int t) {
        if (EPI == EPI_RESIDUAL && s == 0) {
            const int row0 = t * G * R + grp * R;
#pragma unroll
            for (int r = 0; r < R; r++)
                xres[r] = (row0 + r < N) ? bf2f(p.out[(size_t)p.col0 * p.out_ld + row0 + r]) : 0.f;
        }
    };
    uint4 bufA[QT], bufB[QT];
    // the first weight batch is issued before the input is staged, so both
    // arrive in one round trip and the stream starts at once.  Unconditional
    // (a wave without a tile loads the last one and drops it): loads issued
    // on every path keep the compiler's wait counts exact, so the fold
    // below waits for each chunk's loads only.
    {
        const int t0 = min(tile, n_tiles - 1);
        load_res(t0);
        issue(bufA, t0);
    }
    finish_input<1>(p, stg, hs, red, nw * 64);
    lds_barrier();   // publishes the staged input and tile_next (LDS only: the weights keep arriving)

    float best_v = -INFINITY;
    int best_i = 0x7fffffff;

    // independent partial sums per row (4 chains in flight per lane)
    constexpr int A = (R >= 4) ? 1 : 4 / R;
    // row sums of this wave's chunks of a tile: chunk c of the batch is
    // chunk j0 + c of the tile (n of them)
    auto dot = [&](const uint4 (&buf)[QT], double (&acc)[R], int j0, int n) __attribute__((always_inline)) {
        double part[R][A];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int a = 0; a < A; a++) part[r][a] = 0.0;
#pragma unroll
        for (int c = 0; c < JH; c++) {
            if (c >= n) break;   // (wave-uniform: only the second half of an odd J)
            const int j = j0 + c;
            const float4* h4 = reinterpret_cast<const float4*>(hs) + 2 * ((j << lrl) + s);
            const float4 hl = h4[0], hh = h4[1];
            const double hd[8] = {hl.x, hl.y, hl.z, hl.w, hh.x, hh.y, hh.z, hh.w};
            // Fold the chunks in load order, each waiting only for its own
            // load: empty asms that may rewrite the accumulators (so chunk
            // j's FMAs stay after chunk j-1's) and the chunk (so its uses stay
            // after that point).
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int a = 0; a < A; a++) asm volatile("" : "+v"(part[r][a]));
#pragma unroll
            for (int r = 0; r < R; r++) {
                uint4 w = buf[c * R + r];
                asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
                const uint32_t wu[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 8; e++)
                    part[r][e % A] = fma((e & 1) ? (double)bf_hi(wu[e >> 1]) : (double)bf_lo(wu[e >> 1]), hd[e],
                                         part[r][e % A]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            acc[r] = part[r][0];
#pragma unroll
            for (int a = 1; a < A; a++) acc[r] += part[r][a];
            acc[r] = group_sum_rt(acc[r], lrl);
        }
    };
    // epilogue of tile t from its row sums (lanes with s == 0)
    auto emit = [&](const double (&acc)[R], int t) __attribute__((always_inline)) {
        if (s != 0) return;
        const int row0 = t * G * R + grp * R;
        const size_t col = (size_t)p.col0;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int r = 0; r + 1 < R; r += 2) {
                if (row0 + r < N) {
                    const float g = rbf((float)acc[r]);
                    const float u = rbf((float)acc[r + 1]);
                    const double gd = (double)g;
                    const float z = rbf((float)(gd / (1.0 + exp(-gd))));
                    p.out[col * p.out_ld + ((row0 + r) >> 1)] = f2bf(z * u);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = row0 + r;
                if (row >= N) continue;
                if (EPI == EPI_STORE) {
                    p.out[col * p.out_ld + row] = f2bf((float)acc[r]);
                } else if (EPI == EPI_RESIDUAL) {
                    p.out[col * p.out_ld + row] = f2bf(xres[r] + rbf((float)acc[r]));
                } else {
                    const float v = (float)acc[r];
                    p.logits[row] = v;
                    if (v > best_v || (v == best_v && row < best_i)) {
                        best_v = v;
                        best_i = row;
                    }
                }
            }
        }
    };

    auto fold = [&](const uint4 (&buf)[QT], int t) __attribute__((always_inline)) {
        double acc[R];
        dot(buf, acc, 0, J);
        emit(acc, t);
    };

    if (!dyn) {
        // at most one tile per wave: fold it straight after staging, outside
        // any loop, so that each chunk iteration waits only for its own loads
        // (straight-line code gets per-load wait counts) and the arithmetic
        // of the first chunks overlaps the arrival of the last
        if constexpr (KS == 1) {
            if (tile < t_end) fold(bufA, tile);
        } else {
            // (waves without a tile fold their repeated data and drop it, so
            // every wave reaches the barrier)
            __shared__ double xch[4][64][R];
            double acc[R];
            dot(bufA, acc, half * JH, half ? J - JH : JH);
            if (half == 1 && s == 0) {
#pragma unroll
                for (int r = 0; r < R; r++) xch[wave >> 1][grp][r] = acc[r];
            }
            lds_barrier();
            if (half == 0 && tile < t_end) {
                if (s == 0) {
#pragma unroll
                    for (int r = 0; r < R; r++) acc[r] += xch[wave >> 1][grp][r];
                }
                emit(acc, tile);
            }
        }
    } else if constexpr (KS == 1) {
        while (tile < t_end) {
            int nt = next_tile(tile);
            batch_ready<QT>(bufA, QT);
            if (nt < t_end) issue(bufB, nt);
            fold(bufA, tile);
            if (nt < t_end) load_res(nt);
            tile = nt;
            if (tile >= t_end) break;
            nt = next_tile(tile);
            batch_ready<QT>(bufB, QT);
            if (nt < t_end) issue(bufA, nt);
            fold(bufB, tile);
            if (nt < t_end) load_res(nt);
            tile = nt;
        }
    }
    if (EPI == EPI_LOGITS) argmax_tail<1>(p, &best_v, &best_i, bval, bidx, is_last, lane, wave, nw);
}

}  // namespace mak

// Tile shapes (R rows per lane group, J chunk iterations) with a compiled
// batch-1 kernel; other shapes and multi-column phases use k_gemv.
#define MAK_GEMV1_SHAPES(X)                                                                     \
    X(1, 1) X(2, 1) X(4, 1) X(1, 2) X(2, 2) X(4, 2) X(1, 3) X(2, 3) X(4, 3) X(1, 4) X(2, 4) X(4, 4) \
    X(1, 6) X(2, 6) X(1, 9) X(2, 9) X(1, 11) X(1, 16)
// gate/up pairs need an even R
#define MAK_GEMV1_PAIR_SHAPES(X) X(2, 1) X(4, 1) X(2, 2) X(4, 2) X(2, 3) X(4, 3) X(2, 4) X(4, 4) X(2, 6) X(2, 9)
// shapes that also have a K-split (KS = 2) kernel: three or more chunk iterations
#define MAK_GEMV1_KS_SHAPES(X) \
    X(1, 3) X(2, 3) X(4, 3) X(1, 4) X(2, 4) X(4, 4) X(1, 6) X(2, 6) X(1, 9) X(2, 9) X(1, 11) X(1, 16)
#define MAK_GEMV1_KS_PAIR_SHAPES(X) X(2, 3) X(4, 3) X(2, 4) X(4, 4) X(2, 6) X(2, 9)

// defined in gemv1_*.hip: the compiled kernel for (r, j) and K split ks (1
// or 2), or nullptr
const void* mak_gemv1_fn_store(int r, int j, int ks = 1);
const void* mak_gemv1_fn_residual(int r, int j, int ks = 1);
const void* mak_gemv1_fn_swiglu(int r, int j, int ks = 1);
const void* mak_gemv1_fn_logits(int r, int j, int ks = 1);
