// attn_split.hip -- exact split-KV attention for long contexts (gfx950).
//
// The single-pass kernel (k_attn) gives each query head one workgroup that
// walks every cached position; past a few hundred positions that walk is a
// chain of dependent round trips.  Here positions are cut into chunks of
// MAK_ATTN_CHUNK and the softmax stays exact (global max and sum before any
// probability is rounded, as the card's split-KV note requires for equality
// with eager execution -- "model-as-a-kernel", Method section):
//
//   A  k_attn_scores  (column, query head, chunk): qk-norm and rope of q and
//      of the step's own k rows, KV append (first head of each kv group, the
//      chunk holding the column's position), scores
//      sigma_j = bf16(bf16(q'.K_j) * scale) -> global scratch, chunk maximum;
//   B  k_attn_pv      (column, query head, chunk): global max over the chunk
//      maxima, Z = fp32(sum_j fp32(exp(sigma_j - max))) over all positions,
//      P_j = bf16(e_j / Z) for the chunk, partial o_c = sum_j P_j V_j
//      in fp64 -> global scratch;
//   C  k_attn_combine (column, query head): o = bf16(fp32(sum_c o_c)), chunks
//      in order.
//
// Kernel boundaries order the three (A's cache appends are visible to B).
// Every product is exact in fp64 and the sums are exact before their single
// rounding, so the result equals the single-pass kernel's.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "mak_internal.h"

namespace mak {

template <int D>
struct AttnGeom {
    static constexpr int d = D;
    static constexpr int half = D / 2;
    static constexpr int LP = D / 8;                       // lanes per K/V row (16 B each)
    static constexpr int LPL = __builtin_ctz(LP);
    static constexpr int ROWS_W = 64 / LP;                 // rows per wave per pass
    static constexpr int ROWS_IT = (MAK_BLOCK / 64) * ROWS_W;
    static constexpr int U = MAK_ATTN_CHUNK / ROWS_IT;      // rows per lane per chunk
    static_assert(U * ROWS_IT == MAK_ATTN_CHUNK, "chunk must be whole passes");
};

__device__ __forceinline__ void split_index(const AttnPhase& p, int& col, int& h, int& c)
{
    const int per_col = p.n_q_heads * p.n_chunks;
    col = blockIdx.x / per_col;
    const int r = blockIdx.x - col * per_col;
    h = r / p.n_chunks;
    c = r - h * p.n_chunks;
}

// ---------------------------------------------------------------------------
// A: scores of one chunk
// LDS: qf[d] f32 | kin[MAK_MAX_COLS][d] bf16 | cos, sin [1 + MAK_MAX_COLS][d/2]
//      bf16 | red[4] f32
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(MAK_BLOCK) void k_attn_scores(AttnPhase p)
{
    using Gm = AttnGeom<D>;
    constexpr int d = D, half = Gm::half, LP = Gm::LP, U = Gm::U;
    __shared__ float qf[d];
    __shared__ uint16_t kin[MAK_MAX_COLS * d];
    __shared__ uint16_t rc[(MAK_MAX_COLS + 1) * half];
    __shared__ uint16_t rsn[(MAK_MAX_COLS + 1) * half];
    __shared__ float red[MAK_BLOCK / 64];

    int col, h, c;
    split_index(p, col, h, c);
    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, rep = Hq / Hkv;
    const int g = h / rep;
    const bool owner = (h - g * rep) == 0;
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = lane >> Gm::LPL, ch = lane & (LP - 1);
    const int my_row = wave * Gm::ROWS_W + sub;

    const ColState cs = p.ctl->cols[col];
    const int pos = cs.pos, fp = cs.first_pos, n = pos + 1;
    const int j0 = c * MAK_ATTN_CHUNK;
    if (j0 >= n) return;                                    // the whole block leaves
    const int j1 = min(n, j0 + MAK_ATTN_CHUNK);
    const int cend = min(j1, fp);                           // cached rows [j0, cend)
    const int s0 = max(j0, fp);                             // the step's rows [s0, j1)
    const int n_s = max(0, j1 - s0);
    const bool own = owner && pos >= j0 && pos < j1;        // this chunk holds the column's own row
    const size_t head_base = ((size_t)cs.slot * Hkv + g) * p.max_seq;
    const uint16_t* kc_h = p.kc + head_base * d;

    // cached K rows of the chunk (independent of this step), then q, the
    // step's k rows and the rope rows
    uint4 kr[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = j0 + u * Gm::ROWS_IT + my_row;
        kr[u] = make_uint4(0, 0, 0, 0);
        if (j < cend) kr[u] = *reinterpret_cast<const uint4*>(kc_h + (size_t)j * d + ch * 8);
    }
    for (int t = tid; t < d; t += MAK_BLOCK) qf[t] = bf2f(p.qkv[(size_t)col * p.qkv_ld + h * d + t]);
    for (int t = tid; t < n_s * d; t += MAK_BLOCK) {
        const int ri = t / d, i = t - ri * d;
        const size_t base = (size_t)(cs.first_col + (s0 - fp) + ri) * p.qkv_ld;
        kin[t] = p.qkv[base + q_dim + g * d + i];
    }
    for (int t = tid; t < (1 + n_s) * half; t += MAK_BLOCK) {
        const int ri = t / half, i = t - ri * half;
        const int at = (ri == 0) ? pos : s0 + ri - 1;
        rc[t] = p.cos_t[(size_t)at * half + i];
        rsn[t] = p.sin_t[(size_t)at * half + i];
    }
    __syncthreads();

    // per-head qk RMSNorm (one wave per vector)
    if (p.q_norm) {
        for (int vi = wave; vi < 1 + n_s; vi += MAK_BLOCK / 64) {
            double ss = 0.0;
            for (int i = lane; i < d; i += 64) {
                const double x = (vi == 0) ? (double)qf[i] : (double)bf2f(kin[(vi - 1) * d + i]);
                ss = fma(x, x, ss);
            }
            ss = wave_sum(ss);
            const float r = rms_scale(ss, d, p.eps);
            for (int i = lane; i < d; i += 64) {
                if (vi == 0) {
                    qf[i] = bf2f(rms_apply(qf[i], r, bf2f(p.q_norm[i])));
                } else {
                    uint16_t* kp = &kin[(vi - 1) * d + i];
                    *kp = rms_apply(bf2f(*kp), r, bf2f(p.k_norm[i]));
                }
            }
        }
        __syncthreads();
    }

    // rope (pairs i, i + d/2): q at pos, step row ri at s0 + ri
    for (int t = tid; t < (1 + n_s) * half; t += MAK_BLOCK) {
        const int vi = t / half, i = t - vi * half;
        const float cv = bf2f(rc[vi * half + i]);
        const float sv = bf2f(rsn[vi * half + i]);
        if (vi == 0) {
            const float a = qf[i], b = qf[i + half];
            qf[i] = rbf(rbf(a * cv) - rbf(b * sv));
            qf[i + half] = rbf(rbf(b * cv) + rbf(a * sv));
        } else {
            uint16_t* kp = &kin[(vi - 1) * d];
            const float a = bf2f(kp[i]), b = bf2f(kp[i + half]);
            kp[i] = f2bf(rbf(a * cv) - rbf(b * sv));
            kp[i + half] = f2bf(rbf(b * cv) + rbf(a * sv));
        }
    }
    __syncthreads();

    // KV append of this column's k', v at pos
    if (own) {
        for (int i = tid; i < d; i += MAK_BLOCK) {
            p.kc[(head_base + pos) * d + i] = kin[(pos - s0) * d + i];
            p.vc[(head_base + pos) * d + i] = p.qkv[(size_t)col * p.qkv_ld + q_dim + kv_dim + g * d + i];
        }
    }

    // scores of the chunk's rows
    double qreg[8];
#pragma unroll
    for (int e = 0; e < 8; e++) qreg[e] = (double)qf[ch * 8 + e];
    float* sc = p.sc + ((size_t)col * Hq + h) * p.max_seq;
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = j0 + u * Gm::ROWS_IT + my_row;
        uint4 kv = kr[u];
        if (j >= cend && j < j1) kv = *reinterpret_cast<const uint4*>(kin + (j - s0) * d + ch * 8);
        const uint32_t ku[4] = {kv.x, kv.y, kv.z, kv.w};
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < 8; e++) a = fma(qreg[e], (double)((e & 1) ? bf_hi(ku[e >> 1]) : bf_lo(ku[e >> 1])), a);
        a = group_sum<Gm::LPL>(a);
        if (j < j1) {
            const float s = rbf(rbf((float)a) * p.scale);
            if (ch == 0) sc[j] = s;
            mloc = fmaxf(mloc, s);
        }
    }
    mloc = wave_max(mloc);
    if (lane == 0) red[wave] = mloc;
    __syncthreads();
    if (tid == 0) {
        float m = red[0];
        for (int w = 1; w < MAK_BLOCK / 64; w++) m = fmaxf(m, red[w]);
        p.cmax[((size_t)col * Hq + h) * p.n_chunks + c] = m;
    }
}

// ---------------------------------------------------------------------------
// B: probabilities and P.V of one chunk
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(MAK_BLOCK) void k_attn_pv(AttnPhase p)
{
    using Gm = AttnGeom<D>;
    constexpr int d = D, LP = Gm::LP, U = Gm::U;
    __shared__ float pc[MAK_ATTN_CHUNK];
    __shared__ double pv[16 * d];
    __shared__ double redd[MAK_BLOCK / 64];
    __shared__ float redf[MAK_BLOCK / 64];

    int col, h, c;
    split_index(p, col, h, c);
    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, rep = Hq / Hkv;
    const int g = h / rep;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = lane >> Gm::LPL, ch = lane & (LP - 1);
    const int my_row = wave * Gm::ROWS_W + sub;

    const ColState cs = p.ctl->cols[col];
    const int n = cs.pos + 1;
    const int j0 = c * MAK_ATTN_CHUNK;
    if (j0 >= n) return;
    const int j1 = min(n, j0 + MAK_ATTN_CHUNK);
    const int n_used = (n + MAK_ATTN_CHUNK - 1) / MAK_ATTN_CHUNK;
    const size_t head_base = ((size_t)cs.slot * Hkv + g) * p.max_seq;
    const uint16_t* vc_h = p.vc + head_base * d;

    // V rows of the chunk first: their latency overlaps the softmax statistics
    uint4 vr[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = j0 + u * Gm::ROWS_IT + my_row;
        vr[u] = make_uint4(0, 0, 0, 0);
        if (j < j1) vr[u] = *reinterpret_cast<const uint4*>(vc_h + (size_t)j * d + ch * 8);
    }

    // global max over the chunk maxima, then Z over every position
    const float* cm = p.cmax + ((size_t)col * Hq + h) * p.n_chunks;
    float m = -INFINITY;
    for (int i = tid; i < n_used; i += MAK_BLOCK) m = fmaxf(m, cm[i]);
    m = wave_max(m);
    if (lane == 0) redf[wave] = m;
    __syncthreads();
    m = redf[0];
    for (int w = 1; w < MAK_BLOCK / 64; w++) m = fmaxf(m, redf[w]);
    const float* sc = p.sc + ((size_t)col * Hq + h) * p.max_seq;
    // each thread sums j = tid, tid + MAK_BLOCK, ... in that order, its loads
    // issued eight at a time
    double z = 0.0;
    for (int b = tid; b < n; b += 8 * MAK_BLOCK) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = (b + u * MAK_BLOCK < n) ? sc[b + u * MAK_BLOCK] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (b + u * MAK_BLOCK < n) z += (double)(float)exp((double)v[u] - (double)m);
    }
    // (e / Z: the correctly rounded fp32 division, equal to the fp64 quotient
    // rounded to fp32)
    const float Z = (float)block_sum_rt(z, redd, MAK_BLOCK / 64);
    for (int j = j0 + tid; j < j1; j += MAK_BLOCK) {
        const float e = (float)exp((double)sc[j] - (double)m);
        pc[j - j0] = rbf(e / Z);
    }
    __syncthreads();

    // partial o = sum_j P_j V_j over the chunk: per-lane sums, folded within
    // each 16-lane row, then over the block's 16 rows through LDS
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = j0 + u * Gm::ROWS_IT + my_row;
        const double pj = (j < j1) ? (double)pc[j - j0] : 0.0;
        const uint32_t vu[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] = fma(pj, (double)((e & 1) ? bf_hi(vu[e >> 1]) : bf_lo(vu[e >> 1])), acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
        double v = acc[e];
        if (Gm::LPL <= 1) v += dpp_d<0x122>(v);   // row_ror:2
        if (Gm::LPL <= 2) v += dpp_d<DPP_ROR4>(v);
        if (Gm::LPL <= 3) v += dpp_d<DPP_ROR8>(v);
        acc[e] = v;
    }
    if ((lane & 15) < LP) {
        const int grp16 = wave * 4 + (lane >> 4);
#pragma unroll
        for (int e = 0; e < 8; e++) pv[grp16 * d + ch * 8 + e] = acc[e];
    }
    __syncthreads();
    double* op = p.opart + (((size_t)col * Hq + h) * p.n_chunks + c) * d;
    for (int i = tid; i < d; i += MAK_BLOCK) {
        double v = 0.0;
#pragma unroll
        for (int gi = 0; gi < 16; gi++) v += pv[gi * d + i];
        op[i] = v;
    }
}

// ---------------------------------------------------------------------------
// C: o = bf16(fp32(sum over chunks, in chunk order))
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(MAK_BLOCK) void k_attn_combine(AttnPhase p)
{
    const int Hq = p.n_q_heads, d = p.head_dim;
    const int col = blockIdx.x / Hq, h = blockIdx.x - col * Hq;
    const int n = p.ctl->cols[col].pos + 1;
    const int n_used = (n + MAK_ATTN_CHUNK - 1) / MAK_ATTN_CHUNK;
    const double* op = p.opart + ((size_t)col * Hq + h) * p.n_chunks * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        // chunks summed in order, their loads issued eight at a time
        double v = 0.0;
        for (int c0 = 0; c0 < n_used; c0 += 8) {
            double x[8];
#pragma unroll
            for (int u = 0; u < 8; u++) x[u] = (c0 + u < n_used) ? op[(size_t)(c0 + u) * d + i] : 0.0;
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (c0 + u < n_used) v += x[u];
        }
        p.o[(size_t)col * Hq * d + h * d + i] = f2bf((float)v);
    }
}

}  // namespace mak

using namespace mak;

#define MAK_SPLIT_DIMS(X) X(16) X(32) X(64) X(128)

int mak_check_launch(const void* fn, dim3 grid, dim3 block, size_t lds);

static hipError_t launch3(const void* fn, dim3 grid, dim3 block, const AttnPhase& p, hipStream_t st, hipEvent_t e0,
                          hipEvent_t e1)
{
    if (mak_check_launch(fn, grid, block, 0)) return hipErrorInvalidConfiguration;
    AttnPhase q = p;
    void* args[] = {&q};
    if (e0 || e1) return hipExtLaunchKernel(fn, grid, block, args, 0, st, e0, e1, 0);
    return hipLaunchKernel(fn, grid, block, args, 0, st);
}

// stage 0 = scores, 1 = P.V, 2 = combine
hipError_t mak_launch_attn_split(const AttnPhase& p, int stage, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const void* fn = nullptr;
    if (stage == 2) {
        fn = reinterpret_cast<const void*>(&k_attn_combine);
        return launch3(fn, dim3(p.ncols * p.n_q_heads), dim3(128), p, st, e0, e1);
    }
#define X(D)                                                                                         \
    if (p.head_dim == D)                                                                             \
        fn = stage == 0 ? reinterpret_cast<const void*>(&k_attn_scores<D>) : reinterpret_cast<const void*>(&k_attn_pv<D>);
    MAK_SPLIT_DIMS(X)
#undef X
    if (!fn) return hipErrorInvalidValue;
    return launch3(fn, dim3(p.ncols * p.n_q_heads * p.n_chunks), dim3(MAK_BLOCK), p, st, e0, e1);
}
