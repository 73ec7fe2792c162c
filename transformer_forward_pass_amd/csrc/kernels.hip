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
// GEMV input staging: hs[c*K + k], bf16, for c < NC (columns >= ncols zero)
// ---------------------------------------------------------------------------
template <int NC>
__device__ void stage_input(const GemvPhase& p, uint16_t* hs, double* red)
{
    const int K = p.geo.k;
    const int tid = threadIdx.x;
    for (int c = 0; c < NC; c++) {
        uint4* h4 = reinterpret_cast<uint4*>(hs + (size_t)c * K);
        const int col = p.col0 + c;
        if (c >= p.ncols) {
            for (int q = tid; q < (K >> 3); q += MAK_BLOCK) h4[q] = make_uint4(0, 0, 0, 0);
            continue;
        }
        if (p.in_kind == IN_RAW) {
            const uint4* src = reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
            for (int q = tid; q < (K >> 3); q += MAK_BLOCK) h4[q] = src[q];
            continue;
        }
        // RMSNorm of x (from the residual stream, or an embedding row)
        double ss = 0.0;
        if (p.in_kind == IN_NORM) {
            const uint4* src = reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
            for (int q = tid; q < (K >> 3); q += MAK_BLOCK) {
                uint4 v = src[q];
                h4[q] = v;
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    double a = bf_lo(u[e]), b = bf_hi(u[e]);
                    ss = fma(a, a, ss);
                    ss = fma(b, b, ss);
                }
            }
        } else {  // IN_GATHER_NORM
            const int tok = p.ctl->cols[col].token;
            const uint4* E = reinterpret_cast<const uint4*>(p.embed);
            uint4* xs = (blockIdx.x == 0)
                            ? reinterpret_cast<uint4*>(p.x_store + (size_t)col * p.x_ld)
                            : nullptr;
            for (int q = tid; q < (K >> 3); q += MAK_BLOCK) {
                uint4 v = E[packed_chunk(p.embed_geo, tok, q)];
                h4[q] = v;
                if (xs) xs[q] = v;
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    double a = bf_lo(u[e]), b = bf_hi(u[e]);
                    ss = fma(a, a, ss);
                    ss = fma(b, b, ss);
                }
            }
        }
        ss = block_sum(ss, red);
        const float r = rms_scale(ss, K, p.eps);
        const uint4* wn = reinterpret_cast<const uint4*>(p.norm_w);
        for (int q = tid; q < (K >> 3); q += MAK_BLOCK) {
            uint4 v = h4[q], w = wn[q];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                uint32_t lo = rms_apply(bf_lo(u[e]), r, bf_lo(ww[e]));
                uint32_t hi = rms_apply(bf_hi(u[e]), r, bf_hi(ww[e]));
                o[e] = lo | (hi << 16);
            }
            h4[q] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        __syncthreads();  // `red` is reused by the next column
    }
}

// ---------------------------------------------------------------------------
// GEMV phase
// ---------------------------------------------------------------------------
template <int R, int NC, int EPI>
__global__ __launch_bounds__(MAK_BLOCK) void k_gemv(GemvPhase p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ double red[4];
    __shared__ float bval[4][NC];
    __shared__ int bidx[4][NC];
    __shared__ int is_last;
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);

    stage_input<NC>(p, hs, red);
    __syncthreads();

    const int K = p.geo.k;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int J = (K >> 3) >> lrl;
    const uint4* W = reinterpret_cast<const uint4*>(p.w);
    const int n_waves = gridDim.x * (MAK_BLOCK / 64);
    const int N = p.geo.n_rows;

    float best_v[NC];
    int best_i[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        best_v[c] = -INFINITY;
        best_i[c] = 0x7fffffff;
    }

    for (int tile = blockIdx.x * (MAK_BLOCK / 64) + wave; tile < p.geo.n_tiles; tile += n_waves) {
        double acc[R][NC];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[r][c] = 0.0;

        const uint4* wt = W + (int64_t)tile * J * R * 64 + lane;
        uint4 cur[R];
#pragma unroll
        for (int r = 0; r < R; r++) cur[r] = wt[r * 64];
        for (int j = 0; j < J; j++) {
            uint4 nxt[R];
            if (j + 1 < J) {
#pragma unroll
                for (int r = 0; r < R; r++) nxt[r] = wt[((j + 1) * R + r) * 64];
            }
            const int chunk = (j << lrl) + s;
            uint4 hv[NC];
#pragma unroll
            for (int c = 0; c < NC; c++)
                hv[c] = reinterpret_cast<const uint4*>(hs + (size_t)c * K)[chunk];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                double hd[NC];
#pragma unroll
                for (int c = 0; c < NC; c++) {
                    const uint32_t hu = (e < 2) ? hv[c].x : (e < 4) ? hv[c].y : (e < 6) ? hv[c].z : hv[c].w;
                    hd[c] = (e & 1) ? bf_hi(hu) : bf_lo(hu);
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const uint32_t wu = (e < 2) ? cur[r].x : (e < 4) ? cur[r].y : (e < 6) ? cur[r].z : cur[r].w;
                    const double wd = (e & 1) ? bf_hi(wu) : bf_lo(wu);
#pragma unroll
                    for (int c = 0; c < NC; c++) acc[r][c] = fma(wd, hd[c], acc[r][c]);
                }
            }
            if (j + 1 < J) {
#pragma unroll
                for (int r = 0; r < R; r++) cur[r] = nxt[r];
            }
        }
        // reduce over the lr lanes of each row group (fixed xor tree)
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++)
                for (int o = lr >> 1; o > 0; o >>= 1) acc[r][c] += __shfl_xor(acc[r][c], o, 64);

        if (s == 0) {
            const int row0 = tile * G * R + grp * R;
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
                            uint16_t* xp = p.out + col * p.out_ld + row;
                            const float y = rbf((float)acc[r][c]);
                            *xp = f2bf(bf2f(*xp) + y);
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
    }

    if (EPI != EPI_LOGITS) return;

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
        for (int w = 1; w < 4; w++) {
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
    // lowest index), then feed the chosen tokens back as the next step's columns
    __shared__ int next_tok[MAK_MAX_COLS];
    for (int c = 0; c < p.ncols; c++) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        for (int b = threadIdx.x; b < p.n_blocks; b += MAK_BLOCK) {
            const float v2 = p.part_val[b * MAK_MAX_COLS + c];
            const int i2 = p.part_idx[b * MAK_MAX_COLS + c];
            if (v2 > v || (v2 == v && i2 < i)) {
                v = v2;
                i = i2;
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
        if (lane == 0) {
            bval[wave][0] = v;
            bidx[wave][0] = i;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < 4; w++) {
                if (bval[w][0] > v || (bval[w][0] == v && bidx[w][0] < i)) {
                    v = bval[w][0];
                    i = bidx[w][0];
                }
            }
            next_tok[c] = (i == 0x7fffffff) ? 0 : i;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        Ctl* ctl = p.ctl;
        ColState old[MAK_MAX_COLS];
        for (int c = 0; c < p.ncols; c++) old[c] = ctl->cols[p.col0 + c];
        const int step = ctl->step;
        for (int c = 0; c < p.ncols; c++) {
            if (p.out_tokens) p.out_tokens[step * p.ncols + c] = next_tok[c];
            ColState ns;
            ns.token = next_tok[c];
            ns.pos = old[c].pos + 1;
            ns.slot = old[c].slot;
            ns.first_pos = old[c].pos + 1;
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

// ---------------------------------------------------------------------------
// attention: one workgroup per (column, kv head)
// ---------------------------------------------------------------------------
// LDS layout (dynamic): qf[rep][d] f32 | kin[n_in][d] bf16 | vin[n_in][d] bf16 |
//                       S[rep][max_seq] bf16
__global__ __launch_bounds__(MAK_BLOCK) void k_attn(AttnPhase p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ double red[4];
    __shared__ float fred[4];
    __shared__ float mx[32];
    __shared__ float zs[32];

    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, d = p.head_dim, half = d >> 1;
    const int rep = Hq / Hkv;
    const int col = blockIdx.x / Hkv;
    const int g = blockIdx.x - col * Hkv;
    const ColState cs = p.ctl->cols[col];
    const int pos = cs.pos, fp = cs.first_pos, n = pos + 1, n_in = pos - fp + 1;
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    float* qf = reinterpret_cast<float*>(smem);
    uint16_t* kin = reinterpret_cast<uint16_t*>(qf + rep * d);
    uint16_t* vin = kin + MAK_MAX_COLS * d;
    uint16_t* S = vin + MAK_MAX_COLS * d;

    // stage A: raw q heads of this group, raw k/v of every in-step column of
    // this sequence up to this one
    for (int t = tid; t < rep * d; t += MAK_BLOCK) {
        const int h = t / d, i = t - h * d;
        qf[t] = bf2f(p.qkv[(size_t)col * p.qkv_ld + (g * rep + h) * d + i]);
    }
    for (int t = tid; t < n_in * d; t += MAK_BLOCK) {
        const int ci = t / d, i = t - ci * d;
        const size_t base = (size_t)(cs.first_col + ci) * p.qkv_ld;
        kin[t] = p.qkv[base + q_dim + g * d + i];
        vin[t] = p.qkv[base + q_dim + kv_dim + g * d + i];
    }
    __syncthreads();

    // stage B: per-head qk RMSNorm (one wave per vector)
    if (p.q_norm) {
        for (int vi = wave; vi < rep + n_in; vi += 4) {
            double ss = 0.0;
            for (int i = lane; i < d; i += 64) {
                const double x = (vi < rep) ? (double)qf[vi * d + i] : (double)bf2f(kin[(vi - rep) * d + i]);
                ss = fma(x, x, ss);
            }
            ss = wave_sum(ss);
            const float r = rms_scale(ss, d, p.eps);
            const uint16_t* wn = (vi < rep) ? p.q_norm : p.k_norm;
            for (int i = lane; i < d; i += 64) {
                if (vi < rep) {
                    qf[vi * d + i] = bf2f(rms_apply(qf[vi * d + i], r, bf2f(wn[i])));
                } else {
                    uint16_t* kp = &kin[(vi - rep) * d + i];
                    *kp = rms_apply(bf2f(*kp), r, bf2f(wn[i]));
                }
            }
        }
        __syncthreads();
    }

    // stage C: rope (pairs i, i + d/2), q at pos, in-step k at fp + ci
    for (int t = tid; t < (rep + n_in) * half; t += MAK_BLOCK) {
        const int vi = t / half, i = t - vi * half;
        const int at = (vi < rep) ? pos : fp + (vi - rep);
        const float c = bf2f(p.cos_t[(size_t)at * half + i]);
        const float sn = bf2f(p.sin_t[(size_t)at * half + i]);
        if (vi < rep) {
            const float a = qf[vi * d + i], b = qf[vi * d + i + half];
            qf[vi * d + i] = rbf(rbf(a * c) - rbf(b * sn));
            qf[vi * d + i + half] = rbf(rbf(b * c) + rbf(a * sn));
        } else {
            uint16_t* kp = &kin[(vi - rep) * d];
            const float a = bf2f(kp[i]), b = bf2f(kp[i + half]);
            kp[i] = f2bf(rbf(a * c) - rbf(b * sn));
            kp[i + half] = f2bf(rbf(b * c) + rbf(a * sn));
        }
    }
    __syncthreads();

    // stage D: append this column's k', v at pos
    const size_t head_base = ((size_t)cs.slot * Hkv + g) * p.max_seq;
    for (int i = tid; i < d; i += MAK_BLOCK) {
        p.kc[(head_base + pos) * d + i] = kin[(n_in - 1) * d + i];
        p.vc[(head_base + pos) * d + i] = vin[(n_in - 1) * d + i];
    }

    // stage E: scores sigma_j = bf16(bf16(q'.K_j) * scale), j <= pos
    for (int j = tid; j < n; j += MAK_BLOCK) {
        const uint16_t* kr = (j < fp) ? p.kc + (head_base + j) * d : kin + (j - fp) * d;
        for (int h = 0; h < rep; h++) {
            double acc = 0.0;
            for (int i = 0; i < d; i += 8) {
                const uint4 kv = *reinterpret_cast<const uint4*>(kr + i);
                const uint32_t u[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    acc = fma((double)qf[h * d + i + 2 * e], (double)bf_lo(u[e]), acc);
                    acc = fma((double)qf[h * d + i + 2 * e + 1], (double)bf_hi(u[e]), acc);
                }
            }
            S[h * p.max_seq + j] = f2bf(rbf((float)acc) * p.scale);
        }
    }
    // per-head max (each thread first scans the scores it wrote itself)
    for (int h = 0; h < rep; h++) {
        float v = -INFINITY;
        for (int j = tid; j < n; j += MAK_BLOCK) v = fmaxf(v, bf2f(S[h * p.max_seq + j]));
        v = block_max(v, fred);
        if (tid == 0) mx[h] = v;
    }
    __syncthreads();
    for (int h = 0; h < rep; h++) {
        const float m = mx[h];
        double z = 0.0;
        for (int j = tid; j < n; j += MAK_BLOCK)
            z += (double)(float)exp((double)bf2f(S[h * p.max_seq + j]) - (double)m);
        z = block_sum(z, red);
        if (tid == 0) zs[h] = (float)z;
    }
    __syncthreads();
    // probabilities P_j = bf16(fp32(e_j / Z)) replace the scores
    for (int h = 0; h < rep; h++) {
        const double m = mx[h], z = zs[h];
        for (int j = tid; j < n; j += MAK_BLOCK) {
            uint16_t* sp = &S[h * p.max_seq + j];
            const double e = (double)(float)exp((double)bf2f(*sp) - m);
            *sp = f2bf((float)(e / z));
        }
    }
    __syncthreads();

    // stage I: o_h[i] = bf16(sum_j P_j V_j[i])
    for (int t = tid; t < rep * d; t += MAK_BLOCK) {
        const int h = t / d, i = t - h * d;
        const uint16_t* Ph = S + h * p.max_seq;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        const int nc = (fp < n) ? fp : n;  // cached positions
        int j = 0;
        for (; j + 4 <= nc; j += 4) {
            a0 = fma((double)bf2f(Ph[j]), (double)bf2f(p.vc[(head_base + j) * d + i]), a0);
            a1 = fma((double)bf2f(Ph[j + 1]), (double)bf2f(p.vc[(head_base + j + 1) * d + i]), a1);
            a2 = fma((double)bf2f(Ph[j + 2]), (double)bf2f(p.vc[(head_base + j + 2) * d + i]), a2);
            a3 = fma((double)bf2f(Ph[j + 3]), (double)bf2f(p.vc[(head_base + j + 3) * d + i]), a3);
        }
        for (; j < nc; j++) a0 = fma((double)bf2f(Ph[j]), (double)bf2f(p.vc[(head_base + j) * d + i]), a0);
        for (; j < n; j++) a1 = fma((double)bf2f(Ph[j]), (double)bf2f(vin[(j - fp) * d + i]), a1);
        const double acc = (a0 + a1) + (a2 + a3);
        p.o[(size_t)col * q_dim + (g * rep + h) * d + i] = f2bf((float)acc);
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

template <int R, int NC>
static hipError_t launch_gemv_rn(const GemvPhase& p, int blocks, size_t lds, hipStream_t st)
{
    switch (p.epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemv<R, NC, EPI_STORE>), dim3(blocks), dim3(MAK_BLOCK), lds, st, p); break;
    case EPI_RESIDUAL: hipLaunchKernelGGL((k_gemv<R, NC, EPI_RESIDUAL>), dim3(blocks), dim3(MAK_BLOCK), lds, st, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemv<R, NC, EPI_SWIGLU>), dim3(blocks), dim3(MAK_BLOCK), lds, st, p); break;
    case EPI_LOGITS: hipLaunchKernelGGL((k_gemv<R, NC, EPI_LOGITS>), dim3(blocks), dim3(MAK_BLOCK), lds, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int R>
static hipError_t launch_gemv_r(const GemvPhase& p, int nc, int blocks, size_t lds, hipStream_t st)
{
    switch (nc) {
    case 1: return launch_gemv_rn<R, 1>(p, blocks, lds, st);
    case 2: return launch_gemv_rn<R, 2>(p, blocks, lds, st);
    case 4: return launch_gemv_rn<R, 4>(p, blocks, lds, st);
    case 8: return launch_gemv_rn<R, 8>(p, blocks, lds, st);
    }
    return hipErrorInvalidValue;
}

// Column capacity (template NC) for n active columns.
int mak_gemv_nc(int ncols) { return ncols <= 1 ? 1 : ncols <= 2 ? 2 : ncols <= 4 ? 4 : 8; }

hipError_t mak_launch_gemv(const GemvPhase& p, hipStream_t st)
{
    const int nc = mak_gemv_nc(p.ncols);
    const size_t lds = (size_t)nc * p.geo.k * sizeof(uint16_t);
    switch (p.geo.r) {
    case 1: return launch_gemv_r<1>(p, nc, p.n_blocks, lds, st);
    case 2: return launch_gemv_r<2>(p, nc, p.n_blocks, lds, st);
    case 4: return launch_gemv_r<4>(p, nc, p.n_blocks, lds, st);
    }
    return hipErrorInvalidValue;
}

size_t mak_attn_lds(const AttnPhase& p)
{
    const int rep = p.n_q_heads / p.n_kv_heads;
    return (size_t)rep * p.head_dim * 4 + 2 * (size_t)MAK_MAX_COLS * p.head_dim * 2 +
           (size_t)rep * p.max_seq * 2;
}

hipError_t mak_launch_attn(const AttnPhase& p, hipStream_t st)
{
    hipLaunchKernelGGL(k_attn, dim3(p.ncols * p.n_kv_heads), dim3(MAK_BLOCK), mak_attn_lds(p), st, p);
    return hipGetLastError();
}

hipError_t mak_launch_set_ctl(Ctl* ctl, const ColState* cols, int ncols, int step, hipStream_t st)
{
    CtlInit in = {};
    for (int c = 0; c < ncols && c < MAK_MAX_COLS; c++) in.cols[c] = cols[c];
    in.ncols = ncols;
    in.step = step;
    hipLaunchKernelGGL(k_set_ctl, dim3(1), dim3(64), 0, st, ctl, in);
    return hipGetLastError();
}

// Raise the dynamic-LDS ceiling of every kernel instantiation to `bytes`.
hipError_t mak_set_lds_limit(int bytes)
{
#define SETA(R, NC, E)                                                                          \
    do {                                                                                        \
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<R, NC, E>),    \
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);  \
        if (e != hipSuccess) return e;                                                          \
    } while (0)
#define SETE(R, NC) SETA(R, NC, EPI_STORE); SETA(R, NC, EPI_RESIDUAL); SETA(R, NC, EPI_SWIGLU); SETA(R, NC, EPI_LOGITS)
#define SETN(R) SETE(R, 1); SETE(R, 2); SETE(R, 4); SETE(R, 8)
    SETN(1);
    SETN(2);
    SETN(4);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
#undef SETA
#undef SETE
#undef SETN
}
