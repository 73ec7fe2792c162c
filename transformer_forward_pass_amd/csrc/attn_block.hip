// attn_block.hip -- blockwise causal attention for prompt chunks (gfx950).
//
// A prompt chunk's T columns are consecutive positions fp .. fp+T-1 of one
// sequence.  The split-KV kernels (attn_split.hip) give every (column, query
// head, position chunk) its own workgroup, so each K and V row is read once
// per column and head, and each P.V workgroup recomputes the softmax sum over
// every position.  Here a workgroup owns a (query head, 128-position chunk)
// block and serves all T columns from one copy of the chunk's K or V rows
// in LDS; the causal limit (column t sees positions <= fp + t) is applied per
// column ("CuTeDSL at Perplexity", section on prefill and decode
// specialization: prefill kernels get their own grid and block assignment;
// "model-as-a-kernel", Method section: exact split-KV with a deterministic
// combine):
//
//   A  k_attn_blk_scores  (head, chunk): the chunk's cached K rows and the
//      step's own k rows (qk-norm, rope at their positions) into LDS, the
//      columns' q (qk-norm, rope) into LDS, the step rows' KV append (first
//      head of each kv group), then each thread owns one row and computes
//      whole dot products for the columns of its half of the workgroup:
//      sigma_j = bf16(bf16(q'.K_j) * scale) -> global scratch, chunk maximum;
//   S  k_attn_blk_softmax (column, head): max over the chunk maxima,
//      Z = fp32(sum_j fp32(exp(sigma_j - max))), P_j = bf16(e_j / Z)
//      written over the scores, once per row;
//   B  k_attn_blk_pv      (head, chunk): the chunk's V rows and every
//      column's P into LDS; wave w accumulates o_c = sum_j P_j V_j in fp64
//      for its columns t = w (mod 4) together -> global scratch;
//   C  k_attn_combine (attn_split.hip): chunks summed in order, bf16.
//
// The arithmetic is the split-KV kernels' (products exact in fp64, sums
// exact before their single rounding), so the results are bitwise theirs.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "mak_internal.h"

namespace mak {

constexpr int kBlkWaves = 4;
constexpr int kBlkThreads = kBlkWaves * 64;

template <int D>
struct BlkGeom {
    static constexpr int LP = D / 8;                      // lanes per K/V row (16 B each)
    static constexpr int LPL = __builtin_ctz(LP);
    static constexpr int RW = 64 / LP;                    // rows per wave pass
    static constexpr int PASSES = MAK_ATTN_CHUNK / RW;    // passes over a chunk
    static constexpr int UK = MAK_ATTN_CHUNK * LP / kBlkThreads;   // 16-byte chunk pieces per thread
    static_assert(PASSES * RW == MAK_ATTN_CHUNK && PASSES % 4 == 0, "chunk must be whole groups of 4 passes");
    static_assert(UK >= 1 && UK * kBlkThreads == MAK_ATTN_CHUNK * LP, "chunk must be whole loads");
    static_assert(MAK_MAX_COLS * LP <= kBlkThreads, "one 16-byte piece of the step's rows per thread");
    // K rows in LDS are padded by 16 bytes, so the scores' one-row-per-lane
    // 16-byte reads of eight consecutive rows fall in distinct banks
    static constexpr int KSD = D + 8;
};

// P values staged per thread by the P.V kernel: every column's chunk row
constexpr int kBlkPLoads = MAK_MAX_COLS * MAK_ATTN_CHUNK / kBlkThreads;
static_assert(kBlkPLoads * kBlkThreads == MAK_MAX_COLS * MAK_ATTN_CHUNK, "whole P loads");

// the chunk's position range for a (head, chunk) workgroup
struct BlkRange {
    int fp, slot, T, j0, j1, cend, s0, n_s;
};

__device__ __forceinline__ bool blk_range(const AttnPhase& p, int c, BlkRange& r)
{
    const ColState c0 = p.ctl->cols[0];
    r.fp = c0.pos;
    r.slot = c0.slot;
    r.T = p.ncols;
    const int n_max = r.fp + r.T;                          // the last column sees positions < n_max
    r.j0 = c * MAK_ATTN_CHUNK;
    if (r.j0 >= n_max) return false;
    r.j1 = min(n_max, r.j0 + MAK_ATTN_CHUNK);
    r.cend = min(r.j1, r.fp);                              // cached rows [j0, cend)
    r.s0 = max(r.j0, r.fp);                                // the step's rows [s0, j1)
    r.n_s = max(0, r.j1 - r.s0);
    return true;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// The chunk's cached K or V rows [j0, cend): UK 16-byte pieces per thread,
// all issued before any is used.
template <int D>
__device__ __forceinline__ void load_chunk(const uint16_t* cache_h, const BlkRange& r, uint4 (&v)[BlkGeom<D>::UK])
{
    constexpr int LP = BlkGeom<D>::LP;
#pragma unroll
    for (int u = 0; u < BlkGeom<D>::UK; u++) {
        const int i = threadIdx.x + u * kBlkThreads, row = i / LP, q = i - row * LP;
        v[u] = (r.j0 + row < r.cend) ? *reinterpret_cast<const uint4*>(cache_h + (size_t)(r.j0 + row) * D + q * 8)
                                     : zero4();
    }
}

// Only the cached rows go to LDS: the rows past them belong to the step and
// are written by other threads.
template <int D, int STRIDE>
__device__ __forceinline__ void store_chunk(uint16_t* lds, const BlkRange& r, const uint4 (&v)[BlkGeom<D>::UK])
{
    constexpr int LP = BlkGeom<D>::LP;
#pragma unroll
    for (int u = 0; u < BlkGeom<D>::UK; u++) {
        const int i = threadIdx.x + u * kBlkThreads, row = i / LP, q = i - row * LP;
        if (r.j0 + row < r.cend) reinterpret_cast<uint4*>(lds + row * STRIDE)[q] = v[u];
    }
}

// ---------------------------------------------------------------------------
// A: scores of a (query head, chunk) block for every column
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBlkThreads) void k_attn_blk_scores(AttnPhase p)
{
    using Gm = BlkGeom<D>;
    constexpr int d = D, half = D / 2, LP = Gm::LP, KSD = Gm::KSD;
    __shared__ __attribute__((aligned(16))) uint16_t ks[MAK_ATTN_CHUNK * KSD];  // K rows j0 .. j1-1 (padded)
    __shared__ __attribute__((aligned(16))) float qs[MAK_MAX_COLS * D];         // the columns' q (norm, rope)
    __shared__ __attribute__((aligned(16))) double qd[MAK_MAX_COLS * D];        // q' in fp64
    __shared__ float redm[kBlkWaves][8];                                         // per-wave column maxima
    __shared__ __attribute__((aligned(16))) uint16_t rc[MAK_MAX_COLS * half];   // rope rows fp .. fp+T-1
    __shared__ __attribute__((aligned(16))) uint16_t rs[MAK_MAX_COLS * half];

    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, rep = Hq / Hkv;
    const int h = blockIdx.x / p.n_chunks, c = blockIdx.x - h * p.n_chunks;
    const int g = h / rep;
    const bool owner = (h - g * rep) == 0;
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    BlkRange r;
    if (!blk_range(p, c, r)) return;
    const size_t head_base = ((size_t)r.slot * Hkv + g) * p.max_seq;

    // 1. every global load first: cached K rows, the columns' q, the step's
    //    k (and v, for the append) rows, the rope rows of positions fp ..
    //    fp+T-1 (which hold the step rows' positions too)
    uint4 kr[Gm::UK];
    load_chunk<D>(p.kc + head_base * d, r, kr);
    const int qi = tid / LP, qq = tid - qi * LP;          // (column or step row, 16-byte piece)
    const uint4 qv = (qi < r.T) ? *reinterpret_cast<const uint4*>(p.qkv + (size_t)qi * p.qkv_ld + h * d + qq * 8)
                                : zero4();
    const size_t srow = (size_t)(r.s0 - r.fp + qi) * p.qkv_ld;
    const uint4 kv = (qi < r.n_s) ? *reinterpret_cast<const uint4*>(p.qkv + srow + q_dim + g * d + qq * 8) : zero4();
    const uint4 vv = (owner && qi < r.n_s)
                         ? *reinterpret_cast<const uint4*>(p.qkv + srow + q_dim + kv_dim + g * d + qq * 8)
                         : zero4();
    constexpr int RP = half / 8 > 0 ? half / 8 : 1;       // 16-byte pieces per rope row
    const int ri = tid / RP, rq = tid - ri * RP;
    const bool rope_ld = ri < r.T && rq * 8 < half;
    const size_t roff = (size_t)(r.fp + ri) * half + rq * 8;
    const uint4 cv = rope_ld ? *reinterpret_cast<const uint4*>(p.cos_t + roff) : zero4();
    const uint4 sv = rope_ld ? *reinterpret_cast<const uint4*>(p.sin_t + roff) : zero4();

    store_chunk<D, KSD>(ks, r, kr);
    if (qi < r.T) {
        const uint32_t u[4] = {qv.x, qv.y, qv.z, qv.w};
        float* qp = qs + qi * d + qq * 8;
#pragma unroll
        for (int e = 0; e < 8; e++) qp[e] = (e & 1) ? bf_hi(u[e >> 1]) : bf_lo(u[e >> 1]);
    }
    if (qi < r.n_s) reinterpret_cast<uint4*>(ks + (r.s0 - r.j0 + qi) * KSD)[qq] = kv;
    if (rope_ld) {
        reinterpret_cast<uint4*>(rc + ri * half)[rq] = cv;
        reinterpret_cast<uint4*>(rs + ri * half)[rq] = sv;
    }
    lds_barrier();

    // 2. per-head qk RMSNorm (one wave per vector: the columns' q, then the
    //    step's k rows), then rope: q of column t at fp + t, k row at s0 + row
    const int nv = r.T + r.n_s;
    if (p.q_norm) {
        for (int vi = wave; vi < nv; vi += kBlkWaves) {
            uint16_t* kp = ks + (r.s0 - r.j0 + vi - r.T) * KSD;
            double ss = 0.0;
            for (int e = lane; e < d; e += 64) {
                const double x = (vi < r.T) ? (double)qs[vi * d + e] : (double)bf2f(kp[e]);
                ss = fma(x, x, ss);
            }
            ss = wave_sum(ss);
            const float rr = rms_scale(ss, d, p.eps);
            for (int e = lane; e < d; e += 64) {
                if (vi < r.T) qs[vi * d + e] = bf2f(rms_apply(qs[vi * d + e], rr, bf2f(p.q_norm[e])));
                else kp[e] = rms_apply(bf2f(kp[e]), rr, bf2f(p.k_norm[e]));
            }
        }
        lds_barrier();
    }
    for (int i = tid; i < nv * half; i += kBlkThreads) {
        const int vi = i / half, e = i - vi * half;
        const int at = (vi < r.T) ? vi : r.s0 - r.fp + vi - r.T;   // rope row (position - fp)
        const float cf = bf2f(rc[at * half + e]);
        const float sf = bf2f(rs[at * half + e]);
        if (vi < r.T) {
            const float* qp = qs + vi * d;
            const float a = qp[e], b = qp[e + half];
            qd[vi * d + e] = (double)rbf(rbf(a * cf) - rbf(b * sf));
            qd[vi * d + e + half] = (double)rbf(rbf(b * cf) + rbf(a * sf));
        } else {
            uint16_t* kp = ks + (r.s0 - r.j0 + vi - r.T) * KSD;
            const float a = bf2f(kp[e]), b = bf2f(kp[e + half]);
            kp[e] = f2bf(rbf(a * cf) - rbf(b * sf));
            kp[e + half] = f2bf(rbf(b * cf) + rbf(a * sf));
        }
    }
    lds_barrier();

    // 3. KV append of the step's rows in this chunk (one head per kv group)
    if (owner && qi < r.n_s) {
        const size_t at = (head_base + r.s0 + qi) * d + qq * 8;
        *reinterpret_cast<uint4*>(p.kc + at) = reinterpret_cast<const uint4*>(ks + (r.s0 - r.j0 + qi) * KSD)[qq];
        *reinterpret_cast<uint4*>(p.vc + at) = vv;
    }

    // 4. scores: thread i owns row i % 128 of the chunk and computes whole dot
    //    products (elements in order, one fp64 chain per column) for the
    //    columns of its half: half 0 (waves 0-1) takes the first ceil(T/2)
    //    columns, half 1 the rest.  The q' values are the same for every lane
    //    of a wave (broadcast LDS reads); column t keeps rows < fp + t + 1.
    {
        const int row = tid & (MAK_ATTN_CHUNK - 1), hh = tid >> 7;
        const int cpg = (r.T + 1) >> 1;
        const int t0 = hh * cpg, nt = min(cpg, r.T - t0);   // (wave-uniform)
        const int j = r.j0 + row;
        double acc[8];
#pragma unroll
        for (int tt = 0; tt < 8; tt++) acc[tt] = 0.0;
        if (nt > 0) {
            const uint4* krow = reinterpret_cast<const uint4*>(ks + row * KSD);
#pragma unroll
            for (int q = 0; q < LP; q++) {
                const uint4 kk = krow[q];
                const uint32_t ku[4] = {kk.x, kk.y, kk.z, kk.w};
                double kd[8];
#pragma unroll
                for (int e = 0; e < 8; e++) kd[e] = (double)((e & 1) ? bf_hi(ku[e >> 1]) : bf_lo(ku[e >> 1]));
#pragma unroll
                for (int tt = 0; tt < 8; tt++) {
                    if (tt < nt) {
                        const double2* qp = reinterpret_cast<const double2*>(qd + (t0 + tt) * d + q * 8);
                        const double2 q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];
                        acc[tt] = fma(q0.x, kd[0], acc[tt]);
                        acc[tt] = fma(q0.y, kd[1], acc[tt]);
                        acc[tt] = fma(q1.x, kd[2], acc[tt]);
                        acc[tt] = fma(q1.y, kd[3], acc[tt]);
                        acc[tt] = fma(q2.x, kd[4], acc[tt]);
                        acc[tt] = fma(q2.y, kd[5], acc[tt]);
                        acc[tt] = fma(q3.x, kd[6], acc[tt]);
                        acc[tt] = fma(q3.y, kd[7], acc[tt]);
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < 8; tt++) {
            float m = -INFINITY;
            if (tt < nt) {
                const int t = t0 + tt;
                if (j < min(r.j1, r.fp + t + 1)) {
                    const float sv2 = rbf(rbf((float)acc[tt]) * p.scale);
                    p.sc[((size_t)t * Hq + h) * p.max_seq + j] = sv2;
                    m = sv2;
                }
            }
            m = wave_max(m);
            if (lane == 0) redm[wave][tt] = m;
        }
    }
    lds_barrier();
    if (tid < r.T) {
        const int t = tid, cpg = (r.T + 1) >> 1, hh = t >= cpg, tt = t - hh * cpg;
        p.cmax[((size_t)t * Hq + h) * p.n_chunks + c] = fmaxf(redm[2 * hh][tt], redm[2 * hh + 1][tt]);
    }
}

// ---------------------------------------------------------------------------
// S: softmax of one (column, head) row, probabilities over the scores.
// Each thread sums its entries j = tid, tid + 256, ... in that order, so Z
// is the per-column split kernel's.  The first kSoftBatch entries per thread
// are loaded before the maximum is known and their exponentials kept for the
// probabilities; later ones (rows past 2048 positions) are loaded eight at a
// time and recomputed.
// ---------------------------------------------------------------------------
constexpr int kSoftBatch = 8;

__global__ __launch_bounds__(kBlkThreads) void k_attn_blk_softmax(AttnPhase p)
{
    __shared__ float redf[kBlkWaves];
    __shared__ double redd[kBlkWaves];
    constexpr int SB = kSoftBatch * kBlkThreads;
    const int Hq = p.n_q_heads;
    const int t = blockIdx.x / Hq, h = blockIdx.x - t * Hq;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = p.ctl->cols[t].pos + 1;
    const int n_used = (n + MAK_ATTN_CHUNK - 1) / MAK_ATTN_CHUNK;
    const float* cm = p.cmax + ((size_t)t * Hq + h) * p.n_chunks;
    float* sc = p.sc + ((size_t)t * Hq + h) * p.max_seq;
    float e0[kSoftBatch];
#pragma unroll
    for (int u = 0; u < kSoftBatch; u++) e0[u] = (tid + u * kBlkThreads < n) ? sc[tid + u * kBlkThreads] : 0.0f;
    float m = -INFINITY;
    for (int i = tid; i < n_used; i += kBlkThreads) m = fmaxf(m, cm[i]);
    m = wave_max(m);
    if (lane == 0) redf[wave] = m;
    lds_barrier();
    m = redf[0];
    for (int w = 1; w < kBlkWaves; w++) m = fmaxf(m, redf[w]);
    double z = 0.0;
#pragma unroll
    for (int u = 0; u < kSoftBatch; u++)
        if (tid + u * kBlkThreads < n) {
            e0[u] = (float)exp((double)e0[u] - (double)m);
            z += (double)e0[u];
        }
    for (int b = tid + SB; b < n; b += SB) {
        float v[kSoftBatch];
#pragma unroll
        for (int u = 0; u < kSoftBatch; u++) v[u] = (b + u * kBlkThreads < n) ? sc[b + u * kBlkThreads] : 0.0f;
#pragma unroll
        for (int u = 0; u < kSoftBatch; u++)
            if (b + u * kBlkThreads < n) z += (double)(float)exp((double)v[u] - (double)m);
    }
    // (e / Z below: the correctly rounded fp32 division, equal to the fp64
    // quotient rounded to fp32)
    const float Z = (float)block_sum_lds(z, redd, kBlkWaves);
    // (each thread rewrites only the entries it read)
#pragma unroll
    for (int u = 0; u < kSoftBatch; u++)
        if (tid + u * kBlkThreads < n) sc[tid + u * kBlkThreads] = rbf(e0[u] / Z);
    for (int b = tid + SB; b < n; b += SB) {
        float v[kSoftBatch];
#pragma unroll
        for (int u = 0; u < kSoftBatch; u++) v[u] = (b + u * kBlkThreads < n) ? sc[b + u * kBlkThreads] : 0.0f;
#pragma unroll
        for (int u = 0; u < kSoftBatch; u++)
            if (b + u * kBlkThreads < n) {
                const float e = (float)exp((double)v[u] - (double)m);
                sc[b + u * kBlkThreads] = rbf(e / Z);
            }
    }
}

// ---------------------------------------------------------------------------
// B: P.V of a (query head, chunk) block for every column
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBlkThreads) void k_attn_blk_pv(AttnPhase p)
{
    using Gm = BlkGeom<D>;
    constexpr int d = D, LP = Gm::LP;
    __shared__ __attribute__((aligned(16))) uint16_t vs[MAK_ATTN_CHUNK * D];   // V rows j0 .. j1-1
    __shared__ float ps[MAK_MAX_COLS * MAK_ATTN_CHUNK];                          // P of every column

    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, rep = Hq / Hkv;
    const int h = blockIdx.x / p.n_chunks, c = blockIdx.x - h * p.n_chunks;
    const int g = h / rep;
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    BlkRange r;
    if (!blk_range(p, c, r)) return;
    const size_t head_base = ((size_t)r.slot * Hkv + g) * p.max_seq;

    // every global load first: cached V rows, the step's v rows, P of every
    // column over the chunk (entries past a column's limit read as 0)
    uint4 vr[Gm::UK];
    load_chunk<D>(p.vc + head_base * d, r, vr);
    const int qi = tid / LP, qq = tid - qi * LP;
    const uint4 sv = (qi < r.n_s) ? *reinterpret_cast<const uint4*>(p.qkv + (size_t)(r.s0 - r.fp + qi) * p.qkv_ld +
                                                                   q_dim + kv_dim + g * d + qq * 8)
                                  : zero4();
    float pl[kBlkPLoads];
#pragma unroll
    for (int u = 0; u < kBlkPLoads; u++) {
        const int i = tid + u * kBlkThreads, t = i / MAK_ATTN_CHUNK, j = r.j0 + (i - t * MAK_ATTN_CHUNK);
        pl[u] = (t < r.T && j < min(r.j1, r.fp + t + 1)) ? p.sc[((size_t)t * Hq + h) * p.max_seq + j] : 0.0f;
    }
    store_chunk<D, D>(vs, r, vr);
    if (qi < r.n_s) reinterpret_cast<uint4*>(vs + (r.s0 - r.j0 + qi) * d)[qq] = sv;
#pragma unroll
    for (int u = 0; u < kBlkPLoads; u++) ps[tid + u * kBlkThreads] = pl[u];
    lds_barrier();

    // wave w accumulates its columns t = w + 4i (i < 4) together: each V
    // piece is converted once for all of them.  Per column the sums run in
    // pass order; rows past a column's limit have P = 0, rows past the
    // chunk's end (stale LDS) a zeroed V.
    const int sub = lane >> Gm::LPL, ch = lane & (LP - 1);
    const int nw = (r.T - wave + kBlkWaves - 1) / kBlkWaves;   // this wave's columns (wave-uniform)
    if (nw > 0) {
        const int je_w = min(r.j1, r.fp + wave + kBlkWaves * (nw - 1) + 1);   // its last column's limit
        double acc[4][8];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int e = 0; e < 8; e++) acc[i][e] = 0.0;
        for (int u0 = 0; u0 < Gm::PASSES; u0 += 4) {
            if (r.j0 + u0 * Gm::RW >= je_w) break;         // wave-uniform
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int jj = (u0 + k) * Gm::RW + sub;
                uint4 vv = reinterpret_cast<const uint4*>(vs + jj * d)[ch];
                if (r.j0 + jj >= r.j1) vv = zero4();
                const uint32_t vu[4] = {vv.x, vv.y, vv.z, vv.w};
                double vd[8];
#pragma unroll
                for (int e = 0; e < 8; e++) vd[e] = (double)((e & 1) ? bf_hi(vu[e >> 1]) : bf_lo(vu[e >> 1]));
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (i < nw) {
                        const double pj = (double)ps[(wave + kBlkWaves * i) * MAK_ATTN_CHUNK + jj];
#pragma unroll
                        for (int e = 0; e < 8; e++) acc[i][e] = fma(pj, vd[e], acc[i][e]);
                    }
                }
            }
        }
        // sum over the wave's row groups (lanes with the same piece ch)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i >= nw) continue;
            const int t = wave + kBlkWaves * i;
            if (r.j0 >= min(r.j1, r.fp + t + 1)) continue;   // (wave-uniform) the column does not reach this chunk
#pragma unroll
            for (int e = 0; e < 8; e++) {
                double v = acc[i][e];
                for (int off = LP; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
                acc[i][e] = v;
            }
            if (sub == 0) {
                double* op = p.opart + (((size_t)t * Hq + h) * p.n_chunks + c) * d + ch * 8;
#pragma unroll
                for (int e = 0; e < 8; e++) op[e] = acc[i][e];
            }
        }
    }
}

}  // namespace mak

using namespace mak;

int mak_check_launch(const void* fn, dim3 grid, dim3 block, size_t lds);

// stage 0 = scores, 1 = softmax, 2 = P.V (the combine is the split path's)
hipError_t mak_launch_attn_block(const AttnPhase& p, int stage, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const void* fn = nullptr;
    dim3 grid(p.n_q_heads * p.n_chunks);
    if (stage == 1) {
        fn = reinterpret_cast<const void*>(&k_attn_blk_softmax);
        grid = dim3(p.ncols * p.n_q_heads);
    } else {
#define X(D)                                                                                               \
    if (p.head_dim == D)                                                                                   \
        fn = stage == 0 ? reinterpret_cast<const void*>(&k_attn_blk_scores<D>)                             \
                        : reinterpret_cast<const void*>(&k_attn_blk_pv<D>);
        X(16) X(32) X(64) X(128)
#undef X
    }
    if (!fn) return hipErrorInvalidValue;
    if (mak_check_launch(fn, grid, dim3(kBlkThreads), 0)) return hipErrorInvalidConfiguration;
    AttnPhase q = p;
    void* args[] = {&q};
    if (e0 || e1) return hipExtLaunchKernel(fn, grid, dim3(kBlkThreads), args, 0, st, e0, e1, 0);
    return hipLaunchKernel(fn, grid, dim3(kBlkThreads), args, 0, st);
}
