// kernels.hip -- gfx950 kernels of the decode program and their launchers.
//
// Phases of one step (B columns = batch rows or prefill tokens):
//   per layer: [RMSNorm + QKV GEMV] -> [attention: qk-norm, rope, KV append,
//   scores, softmax, P.V] -> [O GEMV + residual] -> [RMSNorm + gate/up GEMV +
//   SwiGLU] -> [down GEMV + residual]; then [final RMSNorm + LM head (fp32
//   logits) + greedy argmax with on-device token feedback].
// ("model-as-a-kernel", Method and API sections; RMSNorm as in "Building a GPU
// compiler from scratch ... (Emmy)", Tensor IR section.)
//
// GEMV: weights stream once from HBM in a packed order (mak_internal.h) so
// each wave instruction loads 1 KiB contiguous (16 B per lane).  The GEMV's
// input vectors sit in LDS as bf16; products and sums are fp64; each output
// row is reduced across the lanes that share it with a fixed xor tree.  No
// floating-point atomics anywhere: the only atomic is the integer ticket that
// elects the last workgroup of the LM head to finish the argmax.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "device_math.h"
#include "mak_internal.h"

#include "gemv_kernels.h"
#include "gemvn_kernels.h"

namespace mak {

constexpr int kAttnWaves = 8;                       // waves per attention workgroup
constexpr int kAttnBlock = kAttnWaves * 64;

// ---------------------------------------------------------------------------
// attention: one workgroup per (column, query head)
// ---------------------------------------------------------------------------
// For query head h of a column (kv group g = h / rep): per-head qk RMSNorm,
// rope at the column's position, then softmax(q'K^T * scale) V over
// positions 0..pos.  The first head of each group also appends the column's
// k', v at pos.  Positions before the first column of this sequence in the
// step come from the KV cache; the step's own earlier columns (a prefill
// chunk) are rebuilt in LDS from the raw projections, so no workgroup reads a
// cache row another one writes in the same launch.
//
// Lanes split a K/V row into 16-byte chunks (LP = d/8 lanes per row); rows
// spread over lane groups and the kAttnWaves waves (two per SIMD, so one
// wave's dependent steps overlap the other's); each lane keeps U rows in
// flight.
//
// LDS (dynamic): pv[4 * kAttnWaves][d] f64 | qf[d] f32 | kin[8][d] bf16 | vin[8][d] bf16 |
//                rope cos, sin [9][d/2] bf16 | S[max_seq] f32
// XM (Hq a multiple of 8 only): workgroups go to the 8 XCDs round-robin
// (blockIdx % 8), so XCD x takes the query heads x*Hq/8 .. x*Hq/8 + Hq/8 - 1,
// consecutive heads that share kv heads, and each XCD's L2 fetches the K/V
// rows of as few kv heads as possible.
template <int D_, bool XM = false>
__global__ __launch_bounds__(kAttnBlock) void k_attn(AttnPhase p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int d = D_ > 0 ? D_ : p.head_dim;
    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, half = d >> 1;
    const int rep = Hq / Hkv;
    const int col = blockIdx.x / Hq;
    const int hr = blockIdx.x - col * Hq;
    const int h = XM ? (hr & 7) * (Hq >> 3) + (hr >> 3) : hr;
    const int g = h / rep;
    const bool owner = (h - g * rep) == 0;        // appends the group's k', v
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    double* pv = reinterpret_cast<double*>(smem);
    float* qf = reinterpret_cast<float*>(pv + 4 * kAttnWaves * d);
    uint16_t* kin = reinterpret_cast<uint16_t*>(qf + d);
    uint16_t* vin = kin + MAK_MAX_COLS * d;
    uint16_t* rc = vin + MAK_MAX_COLS * d;            // rope rows: 0 = pos, 1 + ci = fp + ci
    uint16_t* rsn = rc + (MAK_MAX_COLS + 1) * half;
    float* S = reinterpret_cast<float*>(rsn + (MAK_MAX_COLS + 1) * half);

    const int lp_log2 = __builtin_ctz(d >> 3);
    const int LP = 1 << lp_log2;
    const int rows_w = 64 >> lp_log2;
    const int rows_it = kAttnWaves * rows_w;
    const int sub = lane >> lp_log2, ch = lane & (LP - 1);
    const int my_row = wave * rows_w + sub;
    constexpr int U = 8;   // rows per lane per pass: 512 positions per round trip at d = 64

    // ---- round trip 1: this column's state
    const ColState cs = p.ctl->cols[col];
    const int pos = cs.pos, fp = cs.first_pos, n = pos + 1, n_in = pos - fp + 1;
    const size_t head_base = ((size_t)cs.slot * Hkv + g) * p.max_seq;
    const uint16_t* kc_h = p.kc + head_base * d;
    const uint16_t* vc_h = p.vc + head_base * d;

    // ---- round trip 2: the leading cached K and V rows (they do not depend on
    // this step), then the raw q head, the step's k/v rows and rope rows
    uint4 kpre[U], vpre[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = u * rows_it + my_row;
        kpre[u] = make_uint4(0, 0, 0, 0);
        vpre[u] = make_uint4(0, 0, 0, 0);
        if (u * rows_it < fp && j < fp) {   // (the first test is block-uniform: whole passes skip)
            kpre[u] = *reinterpret_cast<const uint4*>(kc_h + (size_t)j * d + ch * 8);
            vpre[u] = *reinterpret_cast<const uint4*>(vc_h + (size_t)j * d + ch * 8);
        }
    }
    if (!p.q_norm) {
        // no qk-norm: rope straight from the loaded pairs (i, i + d/2) and
        // their table entries, before the one barrier -- q at pos, the
        // step's k rows at fp + ci; v rows as loaded
        for (int t = tid; t < (1 + n_in) * half; t += kAttnBlock) {
            const int vi = t / half, i = t - vi * half;
            const int at = (vi == 0) ? pos : fp + vi - 1;
            const float c = bf2f(p.cos_t[(size_t)at * half + i]);
            const float sn = bf2f(p.sin_t[(size_t)at * half + i]);
            const uint16_t* src = (vi == 0) ? p.qkv + (size_t)col * p.qkv_ld + h * d
                                            : p.qkv + (size_t)(cs.first_col + vi - 1) * p.qkv_ld + q_dim + g * d;
            const float a = bf2f(src[i]), b = bf2f(src[i + half]);
            const float ra = rbf(rbf(a * c) - rbf(b * sn));
            const float rb = rbf(rbf(b * c) + rbf(a * sn));
            if (vi == 0) {
                qf[i] = ra;
                qf[i + half] = rb;
            } else {
                kin[(vi - 1) * d + i] = f2bf(ra);
                kin[(vi - 1) * d + i + half] = f2bf(rb);
            }
        }
        for (int t = tid; t < n_in * d; t += kAttnBlock) {
            const int ci = t / d, i = t - ci * d;
            vin[t] = p.qkv[(size_t)(cs.first_col + ci) * p.qkv_ld + q_dim + kv_dim + g * d + i];
        }
        lds_barrier();
    } else {
    for (int t = tid; t < d; t += kAttnBlock) qf[t] = bf2f(p.qkv[(size_t)col * p.qkv_ld + h * d + t]);
    for (int t = tid; t < n_in * d; t += kAttnBlock) {
        const int ci = t / d, i = t - ci * d;
        const size_t base = (size_t)(cs.first_col + ci) * p.qkv_ld;
        kin[t] = p.qkv[base + q_dim + g * d + i];
        vin[t] = p.qkv[base + q_dim + kv_dim + g * d + i];
    }
    for (int t = tid; t < (1 + n_in) * half; t += kAttnBlock) {
        const int ri = t / half, i = t - ri * half;
        const int at = (ri == 0) ? pos : fp + ri - 1;
        rc[t] = p.cos_t[(size_t)at * half + i];
        rsn[t] = p.sin_t[(size_t)at * half + i];
    }
    lds_barrier();

    // per-head qk RMSNorm (one wave per vector: q, then the step's k rows)
    {
        for (int vi = wave; vi < 1 + n_in; vi += kAttnWaves) {
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
        lds_barrier();
    }

    // rope (pairs i, i + d/2): q at pos, the step's k rows at fp + ci
    for (int t = tid; t < (1 + n_in) * half; t += kAttnBlock) {
        const int vi = t / half, i = t - vi * half;
        const float c = bf2f(rc[vi * half + i]);
        const float sn = bf2f(rsn[vi * half + i]);
        if (vi == 0) {
            const float a = qf[i], b = qf[i + half];
            qf[i] = rbf(rbf(a * c) - rbf(b * sn));
            qf[i + half] = rbf(rbf(b * c) + rbf(a * sn));
        } else {
            uint16_t* kp = &kin[(vi - 1) * d];
            const float a = bf2f(kp[i]), b = bf2f(kp[i + half]);
            kp[i] = f2bf(rbf(a * c) - rbf(b * sn));
            kp[i + half] = f2bf(rbf(b * c) + rbf(a * sn));
        }
    }
    lds_barrier();
    }

    // append this column's k', v at pos (single owner per kv group)
    if (owner) {
        for (int i = tid; i < d; i += kAttnBlock) {
            p.kc[(head_base + pos) * d + i] = kin[(n_in - 1) * d + i];
            p.vc[(head_base + pos) * d + i] = vin[(n_in - 1) * d + i];
        }
    }

    // scores sigma_j = bf16(bf16(q'.K_j) * scale); the lane's q chunk in registers
    double qreg[8];
#pragma unroll
    for (int e = 0; e < 8; e++) qreg[e] = (double)qf[ch * 8 + e];
    for (int j0 = 0; j0 < n; j0 += U * rows_it) {
        uint4 kv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + u * rows_it + my_row;
            if (j0 + u * rows_it >= n) continue;   // block-uniform: a pass past the last position
            if (j0 == 0) kv[u] = kpre[u];
            else kv[u] = (j < fp) ? *reinterpret_cast<const uint4*>(kc_h + (size_t)j * d + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
            if (j >= fp && j < n) kv[u] = *reinterpret_cast<const uint4*>(kin + (j - fp) * d + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (j0 + u * rows_it >= n) continue;
            const uint32_t ku[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
            double a = 0.0;
#pragma unroll
            for (int e = 0; e < 8; e++)
                a = fma(qreg[e], (double)((e & 1) ? bf_hi(ku[e >> 1]) : bf_lo(ku[e >> 1])), a);
            a = (D_ > 0) ? group_sum<(D_ > 0 ? __builtin_ctz(D_ >> 3) : 0)>(a) : group_sum_rt(a, lp_log2);
            const int j = j0 + u * rows_it + my_row;
            if (ch == 0 && j < n) S[j] = rbf(rbf((float)a) * p.scale);
        }
    }
    lds_barrier();

    // softmax over the block: max, e_j = fp32(exp(sigma_j - max)),
    // Z = fp32(sum e_j), P_j = bf16(e_j / Z) with the correctly rounded fp32
    // division (the fp64 quotient of two fp32 values rounded to fp32 is that
    // same value); each thread rewrites only the entries it reads
    if (n <= 256) {   // a short row: one wave, no extra barriers, four entries per lane
        if (wave == 0) {
            float sv[4];
#pragma unroll
            for (int u = 0; u < 4; u++) sv[u] = (lane + 64 * u < n) ? S[lane + 64 * u] : -INFINITY;
            float m = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            m = wave_max(m);
            double z = 0.0;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                sv[u] = (float)exp((double)sv[u] - (double)m);
                if (lane + 64 * u < n) z += (double)sv[u];
            }
            const float Z = (float)wave_sum(z);
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (lane + 64 * u < n) S[lane + 64 * u] = rbf(sv[u] / Z);
        }
    } else {
        __shared__ float redf[kAttnBlock / 64];
        __shared__ double redd[kAttnBlock / 64];
        float m = -INFINITY;
        for (int j = tid; j < n; j += kAttnBlock) m = fmaxf(m, S[j]);
        m = wave_max(m);
        if (lane == 0) redf[wave] = m;
        lds_barrier();
        m = redf[0];
        for (int w = 1; w < kAttnBlock / 64; w++) m = fmaxf(m, redf[w]);
        double z = 0.0;
        for (int j = tid; j < n; j += kAttnBlock) {
            const float e = (float)exp((double)S[j] - (double)m);
            S[j] = e;
            z += (double)e;
        }
        const float Z = (float)block_sum_lds(z, redd, kAttnBlock / 64);
        for (int j = tid; j < n; j += kAttnBlock) S[j] = rbf(S[j] / Z);
    }
    lds_barrier();

    // o = bf16(sum_j P_j V_j): per-lane partial sums over its rows, folded
    // within each 16-lane row (DPP), then the block's 4 * kAttnWaves rows through LDS
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0;
    for (int j0 = 0; j0 < n; j0 += U * rows_it) {
        uint4 vv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + u * rows_it + my_row;
            if (j0 + u * rows_it >= n) continue;   // block-uniform
            if (j0 == 0) vv[u] = vpre[u];
            else vv[u] = (j < fp) ? *reinterpret_cast<const uint4*>(vc_h + (size_t)j * d + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
            if (j >= fp && j < n) vv[u] = *reinterpret_cast<const uint4*>(vin + (j - fp) * d + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (j0 + u * rows_it >= n) continue;
            const int j = j0 + u * rows_it + my_row;
            const double pj = (j < n) ? (double)S[j] : 0.0;
            const uint32_t vu[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                acc[e] = fma(pj, (double)((e & 1) ? bf_hi(vu[e >> 1]) : bf_lo(vu[e >> 1])), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
        double v = acc[e];
        if (lp_log2 <= 1) v += dpp_d<0x122>(v);   // row_ror:2
        if (lp_log2 <= 2) v += dpp_d<DPP_ROR4>(v);
        if (lp_log2 <= 3) v += dpp_d<DPP_ROR8>(v);
        acc[e] = v;
    }
    if ((lane & 15) < LP) {
        const int grp16 = wave * 4 + (lane >> 4);
#pragma unroll
        for (int e = 0; e < 8; e++) pv[grp16 * d + ch * 8 + e] = acc[e];
    }
    lds_barrier();
    for (int i = tid; i < d; i += kAttnBlock) {
        double v = 0.0;
#pragma unroll
        for (int gi = 0; gi < 4 * kAttnWaves; gi++) v += pv[gi * d + i];
        p.o[(size_t)col * q_dim + h * d + i] = f2bf((float)v);
    }
}

// ---------------------------------------------------------------------------
// control block
// ---------------------------------------------------------------------------
struct CtlInit {
    ColState cols[MAK_MAX_COLS];
    int32_t ncols, step;
};

__global__ void k_set_ctl(Ctl* ctl, CtlInit in)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        for (int c = 0; c < MAK_MAX_COLS; c++) ctl->cols[c] = in.cols[c];
        ctl->ncols = in.ncols;
        ctl->step = in.step;
        ctl->ticket = 0;
        ctl->err = 0;
    }
}

}  // namespace mak

// ---------------------------------------------------------------------------
// launchers (host)
// ---------------------------------------------------------------------------
using namespace mak;

// batch-1 GEMV for tile shapes without a compiled k_gemv1
template <int R>
static const void* gemv_fn_r1(int epi)
{
    switch (epi) {
    case EPI_STORE: return reinterpret_cast<const void*>(&k_gemv<R, 1, EPI_STORE>);
    case EPI_RESIDUAL: return reinterpret_cast<const void*>(&k_gemv<R, 1, EPI_RESIDUAL>);
    case EPI_SWIGLU: return reinterpret_cast<const void*>(&k_gemv<R, 1, EPI_SWIGLU>);
    case EPI_LOGITS: return reinterpret_cast<const void*>(&k_gemv<R, 1, EPI_LOGITS>);
    }
    return nullptr;
}

// gemm16.hip: the multi-column GEMM on the fp64 matrix cores
const void* mak_gemm16_fn(int rt, int epi, bool staged);
const void* mak_gemm8_fn(int rt, int epi, bool staged, bool half, int ng);
size_t mak_gemm8_lds(int rt, int k, bool staged, bool single_round, int ng);
size_t mak_gemm16_lds(int rt, int k, bool staged, bool single_round);
int mak_gemm16_threads(int rt, bool staged);

// gemv4.hip: the GEMV over 4-bit (MXFP4) weights
const void* mak_gemv4_fn(int r, int nc, int epi);
size_t mak_gemv4_lds(int k, int nc);
hipError_t mak_gemv4_set_lds_limit(int bytes);
// gemv41.hip: the batch-1 4-bit GEMV with a compile-time tile shape
const void* mak_gemv41_fn(int r, int j, int epi);
hipError_t mak_gemv41_set_lds_limit(int bytes);

// k_gemv41 for a one-column 4-bit phase (one tile per wave, so the grid
// covers every tile), or nullptr
static const void* gemv41_fn(const GemvPhase& p)
{
    if (p.ncols != 1 || p.geo.n_tiles > 4 * 16384) return nullptr;
    return mak_gemv41_fn(p.geo.r, (p.geo.k / MAK_MX_BLOCK) >> p.geo.lr_log2, p.epi);
}

// Column capacity (template NC) for n active columns.
int mak_gemv_nc(int ncols) { return ncols <= 1 ? 1 : ncols <= 2 ? 2 : ncols <= 4 ? 4 : ncols <= 8 ? 8 : 16; }

static const void* gemvn_fn(int rr, int nc, int epi)
{
    switch (epi) {
    case EPI_STORE: return mak_gemvn_fn_store(rr, nc);
    case EPI_RESIDUAL: return mak_gemvn_fn_residual(rr, nc);
    case EPI_SWIGLU: return mak_gemvn_fn_swiglu(rr, nc);
    case EPI_LOGITS: return mak_gemvn_fn_logits(rr, nc);
    }
    return nullptr;
}

static const void* gemv1_fn_ks(const GemvPhase& p, int ks)
{
    const int j = (p.geo.k >> 3) >> p.geo.lr_log2;
    switch (p.epi) {
    case EPI_STORE: return mak_gemv1_fn_store(p.geo.r, j, ks);
    case EPI_RESIDUAL: return mak_gemv1_fn_residual(p.geo.r, j, ks);
    case EPI_SWIGLU: return mak_gemv1_fn_swiglu(p.geo.r, j, ks);
    case EPI_LOGITS: return mak_gemv1_fn_logits(p.geo.r, j, ks);
    }
    return nullptr;
}

static const void* gemv1_fn(const GemvPhase& p) { return gemv1_fn_ks(p, p.ks == 2 ? 2 : 1); }

static bool gemv1_compiled(const GemvPhase& p) { return gemv1_fn_ks(p, 1) != nullptr; }

static const void* gemv_fn(const GemvPhase& p)
{
    if (p.geo.fmt == MAK_FMT_MXFP4) {
        if (const void* f = gemv41_fn(p)) return f;
        return mak_gemv4_fn(p.geo.r, mak_gemv_nc(p.ncols), p.epi);
    }
    if (p.multi == 2) return mak_gemm16_fn(p.rr, p.epi, p.in_kind != IN_RAW);
    if (p.multi == 3) return mak_gemm8_fn(p.rr, p.epi, p.in_kind != IN_RAW, p.jw == 2, p.ncols > 8 ? 4 : 2);
    if (p.multi) return gemvn_fn(p.rr, mak_gemv_nc(p.ncols), p.epi);
    if (const void* f = gemv1_fn(p)) return f;
    switch (p.geo.r) {
    case 1: return gemv_fn_r1<1>(p.epi);
    case 2: return gemv_fn_r1<2>(p.epi);
    case 4: return gemv_fn_r1<4>(p.epi);
    }
    return nullptr;
}

static int gemv_threads(const GemvPhase& p) { return p.threads; }

size_t mak_gemv_lds(const GemvPhase& p)
{
    if (p.geo.fmt == MAK_FMT_MXFP4) return mak_gemv4_lds(p.geo.k, mak_gemv_nc(p.ncols));
    if (p.multi == 2 || p.multi == 3) {
        const int tr = (p.multi == 3 && p.jw == 2) ? 8 : 16;   // rows per tile (k_gemm8 half-height: jw = 2)
        const int64_t groups = (p.geo.n_rows + tr * p.rr - 1) / (tr * p.rr);
        return p.multi == 2 ? mak_gemm16_lds(p.rr, p.geo.k, p.in_kind != IN_RAW, groups <= p.n_blocks)
                            : mak_gemm8_lds(p.rr, p.geo.k, p.in_kind != IN_RAW, groups <= p.n_blocks,
                                            p.ncols > 8 ? 4 : 2);
    }
    if (p.multi)
        return gemvn_lds(mak_gemv_nc(p.ncols), p.geo.k, p.rr, p.jw, p.geo.lr_log2, p.epi == EPI_SWIGLU);
    return (size_t)p.geo.k * sizeof(float);
}

static int device_cus()
{
    static int n_cu = 0;
    if (!n_cu) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
            n_cu = 256;
    }
    return n_cu;
}

// resident workgroups per CU of `fn` with `lds` bytes of dynamic LDS (cached)
static int resident_blocks(const void* fn, int threads, size_t lds)
{
    struct OccEntry {
        const void* fn;
        size_t lds;
        int occ;
    };
    static OccEntry cache[256];
    static int n_cache = 0;
    for (int i = 0; i < n_cache; i++)
        if (cache[i].fn == fn && cache[i].lds == lds) return cache[i].occ;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads, lds) != hipSuccess || occ <= 0) occ = 1;
    if (n_cache < 256) cache[n_cache++] = {fn, lds, occ};
    return occ;
}

// Multi-column work split: rows per lane rr (as many as keep >= 1024 tile
// groups), then waves per group jw (a power of two <= the chunk iterations,
// within the LDS budget) until about 2048 waves are busy.
// Work split of a multi-column GEMV: RR rows per lane (rr) and waves per
// group along K (jw).  Each wave streams its units in batches of QB 16-byte
// loads per lane (the same bytes for every rr), one batch in flight while it
// folds the other.  Among the compiled shapes that fit the LDS budget, the
// plan takes, in this order of priority (measured over the QKV, O, gate/up,
// down and LM-head matrices of the 135M-1.1B shapes at 8 columns):
//   1. the fewest rounds of groups (each round ends in a reduce-scatter and
//      an epilogue that the next round's loads cannot hide: ~2.5 us);
//   2. the fewest workgroups on the busiest CU (a CU holding two shares the
//      fp64 arithmetic and the input staging of both);
//   3. the fewest batches per wave (each is about a memory round trip);
//   4. the most workgroups (more CUs streaming);
//   5. rr = 2, then 4, then 1 (rr = 1 converts every input for each row,
//      rr = 4 holds twice the accumulators);
//   6. the smallest jw (less LDS combining).
// MAK_GEMVN_PLAN=0 selects the earlier rule (rr for >= 1024 groups, then jw
// up to ~2048 waves) for comparison.
static int gemvn_qb(int nc) { return nc <= 2 ? 16 : nc <= 4 ? 8 : 4; }   // k_gemvn's QB

static void gemvn_plan_auto(GemvPhase& p, size_t lds_budget, int cap);

// Tuning knob: MAK_GEMVN_FORCE="n,k,rr,jw;..." sets (rr, jw) for matrices of
// n rows by k inputs, when that split is compiled and valid; read at every
// plan (plans are made when a step is recorded).
static void gemvn_plan(GemvPhase& p, size_t lds_budget, int cap)
{
    gemvn_plan_auto(p, lds_budget, cap);
    const char* e = getenv("MAK_GEMVN_FORCE");
    if (!e) return;
    const int nc = mak_gemv_nc(p.ncols);
    const int R = p.geo.r, J = (p.geo.k >> 3) >> p.geo.lr_log2;
    while (*e) {
        int n = 0, k = 0, rr = 0, jw = 0, used = 0;
        if (sscanf(e, "%d,%d,%d,%d%n", &n, &k, &rr, &jw, &used) != 4) return;
        e += used;
        if (*e == ';') e++;
        if (n != p.geo.n_rows || k != p.geo.k) continue;
        const bool ok = (rr == 1 || rr == 2 || rr == 4) && rr >= R && rr % R == 0 && gemvn_fn(rr, nc, p.epi) &&
                        (jw == 1 || jw == 2 || jw == 4 || jw == 8) && jw <= J && jw <= MAK_NBLOCK / 64 &&
                        gemvn_lds(nc, p.geo.k, rr, jw, p.geo.lr_log2, p.epi == EPI_SWIGLU) <= lds_budget;
        if (ok) {
            p.rr = rr;
            p.jw = jw;
        }
        return;
    }
}

static void gemvn_plan_auto(GemvPhase& p, size_t lds_budget, int cap)
{
    const int nc = mak_gemv_nc(p.ncols);
    const int R = p.geo.r, lrl = p.geo.lr_log2;
    const int J = (p.geo.k >> 3) >> lrl;
    const int64_t tiles = p.geo.n_tiles;
    const bool pairs = p.epi == EPI_SWIGLU;
    static int mode = -1;
    if (mode < 0) {
        const char* e = getenv("MAK_GEMVN_PLAN");
        mode = (e && atoi(e) == 0) ? 0 : 1;
    }
    if (mode == 0) {
        int rr = R;
        for (int cand : {4, 2}) {
            if (cand < R || cand % R) continue;
            if ((tiles + cand / R - 1) / (cand / R) >= 1024) {
                rr = cand;
                break;
            }
        }
        const int64_t ng = (tiles + rr / R - 1) / (rr / R);
        int jw = 1;
        while (jw * 2 <= MAK_NBLOCK / 64 && jw * 2 <= J && ng * jw < 2048 &&
               gemvn_lds(nc, p.geo.k, rr, jw * 2, lrl, pairs) <= lds_budget)
            jw *= 2;
        p.rr = rr;
        p.jw = jw;
        return;
    }
    const int n_cu = device_cus();
    const int qb = gemvn_qb(nc);
    const int nw = MAK_NBLOCK / 64;
    auto rr_rank = [](int rr) { return rr == 2 ? 0 : rr == 4 ? 1 : 2; };
    bool have = false;
    int64_t b_rounds = 0, b_per_cu = 0, b_batches = 0, b_blocks = 0;
    int b_rank = 0, b_jw = 0;
    p.rr = R;
    p.jw = 1;
    for (int rr : {4, 2, 1}) {
        if (rr < R || rr % R) continue;
        const void* fn = gemvn_fn(rr, nc, p.epi);
        if (!fn) continue;
        const int ub = std::max(1, qb / rr);
        const int64_t ng = (tiles + rr / R - 1) / (rr / R);
        for (int jw = 1; jw <= nw && jw <= J; jw *= 2) {
            const size_t lds = gemvn_lds(nc, p.geo.k, rr, jw, lrl, pairs);
            if (lds > lds_budget) break;
            const int occ = resident_blocks(fn, MAK_NBLOCK, lds);
            const int64_t gpr = nw / jw;
            const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((ng + gpr - 1) / gpr, std::min(occ * n_cu, cap)));
            const int64_t rounds = (ng + blocks * gpr - 1) / (blocks * gpr);
            const int64_t per_cu = (blocks + n_cu - 1) / n_cu;
            const int64_t batches = (rounds * ((J + jw - 1) / jw) + ub - 1) / ub;
            const int rank = rr_rank(rr);
            bool better = !have;
            if (have) {
                if (rounds != b_rounds) better = rounds < b_rounds;
                else if (per_cu != b_per_cu) better = per_cu < b_per_cu;
                else if (batches != b_batches) better = batches < b_batches;
                else if (blocks != b_blocks) better = blocks > b_blocks;
                else if (rank != b_rank) better = rank < b_rank;
                else better = jw < b_jw;
            }
            if (better) {
                have = true;
                b_rounds = rounds, b_per_cu = per_cu, b_batches = batches, b_blocks = blocks;
                b_rank = rank, b_jw = jw;
                p.rr = rr;
                p.jw = jw;
            }
        }
    }
}

// Grid of a GEMV phase.  Batch-1: one wave per tile while that fits on the
// chip at once; otherwise the resident capacity (occupancy x CUs), with the
// tiles spread evenly so that every wave streams the same number of tiles.
// Multi-column: the work split of gemvn_plan, one workgroup per group slot
// up to the resident capacity.
// Multi-column steps of at least this many columns run on the fp64 matrix
// cores (k_gemm16); MAK_GEMM_MFMA_COLS overrides (0: never).  fp64 MFMA
// sustains about 40 TFLOP/s here against 63 for fp64 VALU FMAs, so the
// matrix cores pay only where they take the most multiply-adds off the
// VALU: measured faster than k_gemvn for the 16-column groups (16-sequence
// decode 3.17 -> 2.78 ms per step, 16-token prefill chunks), slower at 8.
static int gemm16_min_cols()
{
    static int v = -1;
    if (v < 0) {
        const char* e = getenv("MAK_GEMM_MFMA_COLS");
        v = (e && atoi(e) >= 0) ? atoi(e) : 9;
    }
    return v;
}

// Tiles of 16 rows per k_gemm16 workgroup: as many as still leave two
// workgroups per CU, within the LDS budget.  Returns 0 if the kernel does
// not apply (too few columns, or RMSNorm inputs wider than 4096).
int mak_gemm16_plan(const GemvPhase& p, int ncols, size_t lds_budget)
{
    const int mc = gemm16_min_cols();
    if (mc == 0 || ncols < mc || ncols > 16) return 0;
    const bool staged = p.in_kind != IN_RAW;
    if (staged && p.geo.k > 4096) return 0;
    const int n_cu = device_cus();
    const int n16 = (p.geo.n_rows + 15) / 16;
    int rt = (n16 >= 8 * n_cu) ? 4 : (n16 >= 4 * n_cu) ? 2 : 1;
    // (sized for the worst case: partial tiles beside the inputs)
    while (rt > 1 && mak_gemm16_lds(rt, p.geo.k, staged, false) > lds_budget) rt >>= 1;
    return mak_gemm16_lds(rt, p.geo.k, staged, false) <= lds_budget ? rt : 0;
}

// Steps of 2..8 columns (at least MAK_GEMM8_COLS, default 2; 0: never) run
// on v_mfma_f64_4x4x4_4b_f64 (k_gemm8), which reaches the fp64 matrix rate
// with no padded half tile, where that measured faster than the vector
// GEMV: at least 2048 inputs and 2048 rows, and raw inputs only at 2048
// (shorter rows leave each wave too few 32-input blocks to cover the
// staging and the cross-wave sum; long raw rows over few row groups leave
// CUs idle).  Row tiles per workgroup as for k_gemm16, raw inputs at most
// two.  Raw inputs whose 16-row groups are fewer than the CUs take tiles of
// 8 rows (gemm8_half; MAK_GEMM8_HALF=0 turns them off), and with them any
// K; on such tiles 9..16 columns run here too, as four groups of four
// (MAK_GEMM8_WIDE=0 leaves them to k_gemm16).  Returns 0 if the kernel does
// not apply.
static bool gemm8_half(const GemvPhase& p)
{
    static int hv = -1;
    if (hv < 0) {
        const char* e = getenv("MAK_GEMM8_HALF");
        hv = (e && atoi(e) == 0) ? 0 : 1;
    }
    return hv && p.in_kind == IN_RAW && (p.geo.n_rows + 15) / 16 < device_cus();
}

int mak_gemm8_plan(const GemvPhase& p, int ncols, size_t lds_budget)
{
    static int mc = -1, wide = -1;
    if (mc < 0) {
        const char* e = getenv("MAK_GEMM8_COLS");
        mc = (e && atoi(e) >= 0) ? atoi(e) : 2;
        const char* e2 = getenv("MAK_GEMM8_WIDE");
        wide = (e2 && atoi(e2) == 0) ? 0 : 1;
    }
    const bool staged = p.in_kind != IN_RAW;
    const bool half = gemm8_half(p);
    if (mc == 0 || ncols < mc || ncols < 2 || ncols > 16) return 0;
    if (ncols > 8 && !(wide && half)) return 0;
    if (staged && p.geo.k > 4096) return 0;
    if (p.geo.k < 2048 || p.geo.n_rows < 2048 || (!staged && p.geo.k > 2048 && !half)) return 0;
    const int n_cu = device_cus();
    const int n16 = (p.geo.n_rows + 15) / 16;
    int rt = (n16 >= 8 * n_cu) ? 4 : (n16 >= 4 * n_cu) ? 2 : 1;
    if (!staged && rt > 2) rt = 2;
    if (half) rt = 1;
    const int ng = ncols > 8 ? 4 : 2;
    while (rt > 1 && mak_gemm8_lds(rt, p.geo.k, staged, false, ng) > lds_budget) rt >>= 1;
    return mak_gemm8_lds(rt, p.geo.k, staged, false, ng) <= lds_budget ? rt : 0;
}

int mak_gemv_blocks(GemvPhase& p, int cap, size_t lds_budget_n)
{
    const int n_cu = device_cus();
    if (p.geo.fmt == MAK_FMT_MXFP4) {
        // 4-bit weights: k_gemv4, workgroups of 4 waves, one tile per wave
        // up to 4096 workgroups (waves loop over the rest)
        p.multi = 0;
        p.ks = 1;
        p.rr = p.geo.r;
        p.jw = 1;
        p.threads = MAK_BLOCK;
        const int64_t wpb = MAK_BLOCK / 64;
        if (gemv41_fn(p)) return (int)((p.geo.n_tiles + wpb - 1) / wpb);   // one tile per wave
        return (int)std::max<int64_t>(1, std::min<int64_t>((p.geo.n_tiles + wpb - 1) / wpb, std::max(cap, 4096)));
    }
    // (splitting one-column tiles over several waves with this kernel was
    // measured slower: its staging and combine cost more than the fold)
    p.multi = p.ncols >= 2;
    if (p.multi) {
        if (const int rt = mak_gemm8_plan(p, p.ncols, lds_budget_n)) {
            // (as k_gemm16 below: resident workgroups, each staging its inputs once)
            p.multi = 3;
            p.rr = rt;
            const bool half = gemm8_half(p);
            p.jw = half ? 2 : 1;                      // (k_gemm8: 2 = tiles of 8 rows)
            const bool staged = p.in_kind != IN_RAW;
            p.threads = mak_gemm16_threads(rt, staged);
            const int tr = half ? 8 : 16;
            const int64_t groups = (p.geo.n_rows + tr * rt - 1) / (tr * rt);
            const int ng = p.ncols > 8 ? 4 : 2;
            const int occ = resident_blocks(mak_gemm8_fn(rt, p.epi, staged, half, ng), p.threads,
                                            mak_gemm8_lds(rt, p.geo.k, staged, false, ng));
            int64_t g = std::min<int64_t>(groups, (int64_t)occ * n_cu);
            if (p.epi == EPI_LOGITS) g = std::min<int64_t>(g, cap);
            return (int)std::max<int64_t>(1, g);
        }
        if (const int rt = mak_gemm16_plan(p, p.ncols, lds_budget_n)) {
            p.multi = 2;
            p.rr = rt;
            p.jw = 1;
            p.threads = mak_gemm16_threads(rt, p.in_kind != IN_RAW);
            const int64_t groups = (p.geo.n_rows + 16 * rt - 1) / (16 * rt);
            // As many workgroups as are resident at once (the staged inputs
            // take most of a CU's LDS): each stages its inputs once and loops
            // over row groups, issuing the next group's first batch before
            // reducing the current one.  (The LM head's argmax partials also
            // hold at most `cap` workgroups.)  MAK_GEMM16_RESIDENT=0 launches
            // one workgroup per row group instead.
            static int res_env = -1;
            if (res_env < 0) {
                const char* e = getenv("MAK_GEMM16_RESIDENT");
                res_env = (e && atoi(e) == 0) ? 0 : 1;
            }
            int64_t g = groups;
            if (res_env) {
                const bool staged = p.in_kind != IN_RAW;
                // (LDS sized for several rounds: partial tiles beside the inputs)
                const int occ = resident_blocks(mak_gemm16_fn(rt, p.epi, staged), p.threads,
                                                mak_gemm16_lds(rt, p.geo.k, staged, false));
                g = std::min<int64_t>(groups, (int64_t)occ * n_cu);
            }
            if (p.epi == EPI_LOGITS) g = std::min<int64_t>(g, cap);
            return (int)std::max<int64_t>(1, g);
        }
        gemvn_plan(p, lds_budget_n, cap);
        p.threads = MAK_NBLOCK;
        const void* fn = gemv_fn(p);
        if (!fn) return 0;
        const int occ = resident_blocks(fn, MAK_NBLOCK, mak_gemv_lds(p));
        const int64_t ng = (p.geo.n_tiles + p.rr / p.geo.r - 1) / (p.rr / p.geo.r);
        const int64_t gpr = (MAK_NBLOCK / 64) / p.jw;
        const int64_t want = (ng + gpr - 1) / gpr;
        return (int)std::max<int64_t>(1, std::min<int64_t>(want, std::min(occ * n_cu, cap)));
    }
    const void* fn = gemv_fn(p);
    if (!fn) return 0;
    // batch-1: one tile per wave in workgroups of 4 waves while that keeps
    // <= 8 waves per CU; beyond, one workgroup per CU (8 waves, or 4 for
    // shapes whose batch buffers need the registers of two waves) whose
    // waves share its tile range (k_gemv1 hands the tiles out dynamically,
    // k_gemv strides over them)
    static int per_cu = -1;   // optional override of workgroups per CU (tuning knob)
    if (per_cu < 0) {
        const char* e = getenv("MAK_GEMV_BLOCKS_PER_CU");
        per_cu = (e && atoi(e) > 0) ? atoi(e) : 1;
    }
    const int64_t tiles = p.geo.n_tiles;
    p.ks = 1;
    if (!gemv1_compiled(p)) {
        p.threads = MAK_GBLOCK;
        const int wpb = MAK_GBLOCK / 64;
        return (int)std::max<int64_t>(1, std::min<int64_t>((tiles + wpb - 1) / wpb, std::min(per_cu * n_cu, cap)));
    }
    // One tile per wave up to wpc waves per CU, beyond that the tile queue.
    // All such waves need not be resident at once (the static path has no
    // cross-workgroup waits): 32 waves per CU measured faster than 8 for the
    // 1B shape's QKV and gate/up GEMVs (1166 -> 1195 tok/s), but slower for
    // the LM head, which keeps 8 (MAK_GEMV_STATIC_WPC overrides the 32).
    // The grid cap rises to 4096 workgroups except for the LM head, whose
    // per-workgroup argmax partials are sized for `cap`.
    static int static_wpc = -1;
    if (static_wpc < 0) {
        const char* e = getenv("MAK_GEMV_STATIC_WPC");
        static_wpc = (e && atoi(e) >= 8 && atoi(e) <= 64) ? atoi(e) : 32;
    }
    const int wpc = (p.epi == EPI_LOGITS) ? 8 : static_wpc;
    if (p.epi != EPI_LOGITS) cap = std::max(cap, 4096);
    if (tiles <= (int64_t)wpc * n_cu) {
        // waves per workgroup: small matrices spread over more CUs in
        // workgroups of 2 waves (measured faster up to ~1024 tiles), larger
        // ones in workgroups of 4 (MAK_GEMV_STATIC_WAVES overrides: 1, 2, 4)
        static int sw = -1;
        if (sw < 0) {
            const char* e = getenv("MAK_GEMV_STATIC_WAVES");
            sw = (e && (atoi(e) == 1 || atoi(e) == 2 || atoi(e) == 4)) ? atoi(e) : 0;
        }
        // K split: with room for two waves per tile (up to ks_wpc waves per
        // CU: 16, measured faster than 8 on the 1B shape's O and down GEMVs,
        // whose 4096 waves no longer fit at once), each folds half of the
        // tile's chunks (MAK_GEMV_KSPLIT=0 turns it off; MAK_GEMV_KSPLIT_WPC
        // sets the waves per CU)
        static int ks_env = -1, ks_wpc = 16;
        if (ks_env < 0) {
            const char* e = getenv("MAK_GEMV_KSPLIT");
            ks_env = (e && atoi(e) == 0) ? 0 : 1;
            const char* e2 = getenv("MAK_GEMV_KSPLIT_WPC");
            if (e2 && atoi(e2) >= 2 && atoi(e2) <= 32) ks_wpc = atoi(e2);
        }
        const int64_t waves1 = tiles;
        int w = sw ? sw : (waves1 <= 1024 ? 2 : 4);
        if (ks_env && 2 * tiles <= (int64_t)ks_wpc * n_cu && w >= 2 && gemv1_fn_ks(p, 2)) p.ks = 2;
        const int64_t waves = tiles * p.ks;
        if (!sw) w = waves <= 2048 ? 2 : 4;   // (split waves: 2048 measured faster than 1024 for the 135M down GEMV's 1152)
        // RMSNorm staging holds 2 chunks of 8 inputs per thread
        while (p.in_kind != IN_RAW && w < 4 && 64 * w * 16 < p.geo.k) w *= 2;
        p.threads = 64 * w;
        const int64_t blocks = (waves + w - 1) / w;
        if (p.ks == 2 && blocks > cap) {   // (the K-split kernel has no tile loop: every tile needs its pair)
            p.ks = 1;
            return (int)std::min<int64_t>((tiles + w - 1) / w, cap);
        }
        return (int)std::min<int64_t>(blocks, cap);
    }
    const int j = (p.geo.k >> 3) >> p.geo.lr_log2;
    p.threads = gemv1_waves(p.geo.r, j) * 64;
    return (int)std::max(1, std::min(per_cu * n_cu, cap));
}

// Launch `fn`; with start/stop events, HIP stamps them at the kernel's own
// begin and end (the dispatch packet's timestamps), not around the launch.
// Launch-configuration check of `fn` (mak_launch_check with the kernel's own
// attributes, cached per kernel, and the device's LDS per workgroup).
// Returns 0 or the violated rule; `msg` receives a description.
static thread_local char g_launch_msg[256];

const char* mak_launch_check_msg() { return g_launch_msg; }

int mak_check_launch(const void* fn, dim3 grid, dim3 block, size_t lds)
{
    struct AttrEntry {
        const void* fn;
        int64_t max_threads, static_lds, max_dyn;
    };
    static AttrEntry cache[512];
    static int n_cache = 0;
    static int64_t lds_per_block = 0;
    if (!lds_per_block) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            lds_per_block = v;
        else
            lds_per_block = 160 * 1024;
    }
    const AttrEntry* e = nullptr;
    for (int i = 0; i < n_cache; i++)
        if (cache[i].fn == fn) e = &cache[i];
    AttrEntry fresh{};
    if (!e) {
        hipFuncAttributes a{};
        if (hipFuncGetAttributes(&a, fn) != hipSuccess) {
            snprintf(g_launch_msg, sizeof g_launch_msg, "hipFuncGetAttributes failed for a kernel");
            return 5;
        }
        fresh = {fn, a.maxThreadsPerBlock, (int64_t)a.sharedSizeBytes,
                 a.maxDynamicSharedSizeBytes > 0 ? (int64_t)a.maxDynamicSharedSizeBytes : lds_per_block};
        if (n_cache < 512) cache[n_cache++] = fresh;
        e = &fresh;
    }
    const int rc = mak_launch_check(grid.x, grid.y, grid.z, block.x, block.y, block.z, e->max_threads, e->static_lds,
                                    (int64_t)lds, e->max_dyn, lds_per_block);
    if (rc)
        snprintf(g_launch_msg, sizeof g_launch_msg,
                 "launch rejected (rule %d): grid %ux%ux%u, block %ux%ux%u of at most %lld threads, "
                 "LDS %zu dynamic (ceiling %lld) + %lld static of %lld",
                 rc, grid.x, grid.y, grid.z, block.x, block.y, block.z, (long long)e->max_threads, lds,
                 (long long)e->max_dyn, (long long)e->static_lds, (long long)lds_per_block);
    return rc;
}

static hipError_t launch_fn(const void* fn, dim3 grid, dim3 block, void** args, size_t lds, hipStream_t st,
                            hipEvent_t e0, hipEvent_t e1)
{
    if (!fn) return hipErrorInvalidValue;
    if (mak_check_launch(fn, grid, block, lds)) return hipErrorInvalidConfiguration;
    if (e0 || e1) return hipExtLaunchKernel(fn, grid, block, args, lds, st, e0, e1, 0);
    return hipLaunchKernel(fn, grid, block, args, lds, st);
}

hipError_t mak_launch_gemv(const GemvPhase& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    GemvPhase q = p;
    void* args[] = {&q};
    return launch_fn(gemv_fn(p), dim3(p.n_blocks), dim3(gemv_threads(p)), args, mak_gemv_lds(p), st, e0, e1);
}

// dynamic LDS of k_attn: pv[4 * kAttnWaves][d] f64 | qf[d] f32 | kin, vin [8][d] bf16 |
// rope [9][d/2] bf16 x 2 | S[s_cap] f32
size_t mak_attn_lds_for(int rep, int d, int max_seq)
{
    (void)rep;
    return (size_t)4 * kAttnWaves * d * 8 + (size_t)d * 4 + 2 * (size_t)MAK_MAX_COLS * d * 2 +
           2 * (size_t)(MAK_MAX_COLS + 1) * (d / 2) * 2 + (size_t)max_seq * 4;
}

size_t mak_attn_lds(const AttnPhase& p)
{
    return mak_attn_lds_for(p.n_q_heads / p.n_kv_heads, p.head_dim, p.s_cap);
}

#define MAK_ATTN_DIMS(X) X(32) X(64) X(128)

hipError_t mak_launch_attn(const AttnPhase& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const bool xm = p.n_q_heads % 8 == 0;
    const void* fn = xm ? reinterpret_cast<const void*>(&k_attn<0, true>) : reinterpret_cast<const void*>(&k_attn<0>);
#define X(D)                                                                                \
    if (p.head_dim == D)                                                                    \
        fn = xm ? reinterpret_cast<const void*>(&k_attn<D, true>) : reinterpret_cast<const void*>(&k_attn<D>);
    MAK_ATTN_DIMS(X)
#undef X
    AttnPhase q = p;
    void* args[] = {&q};
    return launch_fn(fn, dim3(p.ncols * p.n_q_heads), dim3(kAttnBlock), args, mak_attn_lds(p), st, e0, e1);
}

hipError_t mak_launch_set_ctl(Ctl* ctl, const ColState* cols, int ncols, int step, hipStream_t st, hipEvent_t e0,
                              hipEvent_t e1)
{
    CtlInit in = {};
    for (int c = 0; c < ncols && c < MAK_MAX_COLS; c++) in.cols[c] = cols[c];
    in.ncols = ncols;
    in.step = step;
    void* args[] = {&ctl, &in};
    return launch_fn(reinterpret_cast<const void*>(&k_set_ctl), dim3(1), dim3(64), args, 0, st, e0, e1);
}

// Raise the dynamic-LDS ceiling of the batch-1 GEMV instantiations to
// `bytes`, of the multi-column ones to `bytes_n` and of the attention kernel
// to `attn_bytes`.
hipError_t mak_set_lds_limit(int bytes, int bytes_n, int attn_bytes)
{
    auto set = [](const void* f, int b) {
        return f ? hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, b) : hipSuccess;
    };
    for (int r : {1, 2, 4})
        for (int epi : {(int)EPI_STORE, (int)EPI_RESIDUAL, (int)EPI_SWIGLU, (int)EPI_LOGITS}) {
            const void* f = (r == 1) ? gemv_fn_r1<1>(epi) : (r == 2) ? gemv_fn_r1<2>(epi) : gemv_fn_r1<4>(epi);
            hipError_t e = set(f, bytes);
            if (e != hipSuccess) return e;
            for (int nc : {2, 4, 8, 16}) {
                e = set(gemvn_fn(r, nc, epi), bytes_n);
                if (e != hipSuccess) return e;
            }
        }
    for (int rt : {1, 2, 4})
        for (int epi : {(int)EPI_STORE, (int)EPI_RESIDUAL, (int)EPI_SWIGLU, (int)EPI_LOGITS})
            for (bool staged : {true, false}) {
                hipError_t e = set(mak_gemm16_fn(rt, epi, staged), bytes_n);
                if (e != hipSuccess) return e;
                for (bool half : {false, true})
                    for (int ng : {2, 4})
                        if (const void* f8 = mak_gemm8_fn(rt, epi, staged, half, ng)) {
                            e = set(f8, bytes_n);
                            if (e != hipSuccess) return e;
                        }
            }
    for (int r : {1, 2, 4})
        for (int j : {1, 2, 3, 4, 6, 9, 11, 16})
            for (int ks : {1, 2})
                for (const void* f : {mak_gemv1_fn_store(r, j, ks), mak_gemv1_fn_residual(r, j, ks),
                                      mak_gemv1_fn_swiglu(r, j, ks), mak_gemv1_fn_logits(r, j, ks)}) {
                    hipError_t e = set(f, bytes);
                    if (e != hipSuccess) return e;
                }
    {
        hipError_t e = mak_gemv4_set_lds_limit(bytes_n);
        if (e != hipSuccess) return e;
        e = mak_gemv41_set_lds_limit(bytes_n);
        if (e != hipSuccess) return e;
    }
#define X(D)                                                                               \
    for (const void* f : {reinterpret_cast<const void*>(&k_attn<D>),                       \
                          reinterpret_cast<const void*>(&k_attn<D, true>)}) {              \
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,  \
                                           attn_bytes);                                    \
        if (e != hipSuccess) return e;                                                     \
    }
    MAK_ATTN_DIMS(X) X(0)
#undef X
    return hipSuccess;
}
