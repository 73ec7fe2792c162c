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
        // RMSNorm of x (the residual stream, or an embedding row): x and the
        // norm weight are loaded together and kept in registers (K <= 4096,
        // so at most 2 chunks per thread)
        const uint4* wn = reinterpret_cast<const uint4*>(p.norm_w);
        uint4 xv[2], wv[2];
        const uint4* src;
        if (p.in_kind == IN_NORM) {
            src = reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
        } else {  // IN_GATHER_NORM
            src = reinterpret_cast<const uint4*>(p.embed);
        }
        const int tok = (p.in_kind == IN_GATHER_NORM) ? p.ctl->cols[col].token : 0;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int q = tid + i * MAK_BLOCK;
            if (q < (K >> 3)) {
                xv[i] = (p.in_kind == IN_NORM) ? src[q] : src[packed_chunk(p.embed_geo, tok, q)];
                wv[i] = wn[q];
            }
        }
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int q = tid + i * MAK_BLOCK;
            if (q < (K >> 3)) {
                if (p.in_kind == IN_GATHER_NORM && blockIdx.x == 0)
                    reinterpret_cast<uint4*>(p.x_store + (size_t)col * p.x_ld)[q] = xv[i];
                const uint32_t u[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double a = bf_lo(u[e]), b = bf_hi(u[e]);
                    ss = fma(a, a, ss);
                    ss = fma(b, b, ss);
                }
            }
        }
        ss = block_sum(ss, red);
        const float r = rms_scale(ss, K, p.eps);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int q = tid + i * MAK_BLOCK;
            if (q < (K >> 3)) {
                const uint32_t u[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
                const uint32_t ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t lo = rms_apply(bf_lo(u[e]), r, bf_lo(ww[e]));
                    const uint32_t hi = rms_apply(bf_hi(u[e]), r, bf_hi(ww[e]));
                    o[e] = lo | (hi << 16);
                }
                h4[q] = make_uint4(o[0], o[1], o[2], o[3]);
            }
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

    const int K = p.geo.k;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int J = (K >> 3) >> lrl;
    const int Q = J * R;                      // 16-byte loads per lane per tile
    const uint4* W = reinterpret_cast<const uint4*>(p.w);
    const int n_waves = gridDim.x * (MAK_BLOCK / 64);
    const int N = p.geo.n_rows;
    constexpr int D = (NC >= 4) ? 8 : 16;     // loads in flight per lane (multiple of R)
    static_assert(D % R == 0, "ring depth must be a multiple of R");

    // The weights do not depend on this step's activations: start streaming
    // the first tile before the input (and its RMSNorm) is staged.
    int tile = blockIdx.x * (MAK_BLOCK / 64) + wave;
    uint4 buf[D];
    if (tile < p.geo.n_tiles) {
        const uint4* wt = W + (int64_t)tile * Q * 64 + lane;
#pragma unroll
        for (int i = 0; i < D; i++)
            if (i < Q) buf[i] = wt[i * 64];
    }

    // residual rows of the first tile (lane s == 0 owns rows row0 .. row0+R-1)
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
    if (tile < p.geo.n_tiles) load_res(tile);

    stage_input<NC>(p, hs, red);
    __syncthreads();

    float best_v[NC];
    int best_i[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        best_v[c] = -INFINITY;
        best_i[c] = 0x7fffffff;
    }

    for (; tile < p.geo.n_tiles; tile += n_waves) {
        double acc[R][NC];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[r][c] = 0.0;

        const uint4* wt = W + (int64_t)tile * Q * 64 + lane;
        uint4 hv[NC];
        constexpr bool kCacheH = NC <= 2;          // keep the input chunk as fp64
        double hdc[kCacheH ? NC : 1][8];
        // ring of D loads: slot i holds load q0 + i; load q = j*R + r
        for (int q0 = 0; q0 < Q; q0 += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                const int q = q0 + i;
                if (q < Q) {
                    const uint4 w = buf[i];
                    if (q + D < Q) buf[i] = wt[(q + D) * 64];
                    constexpr int RR = R;
                    const int r = i % RR;
                    if (r == 0) {
                        const int chunk = ((q / RR) << lrl) + s;
#pragma unroll
                        for (int c = 0; c < NC; c++)
                            hv[c] = reinterpret_cast<const uint4*>(hs + (size_t)c * K)[chunk];
                        if (kCacheH) {
#pragma unroll
                            for (int c = 0; c < (kCacheH ? NC : 1); c++) {
                                const uint32_t hu[4] = {hv[c].x, hv[c].y, hv[c].z, hv[c].w};
#pragma unroll
                                for (int e = 0; e < 8; e++)
                                    hdc[c][e] = (e & 1) ? bf_hi(hu[e >> 1]) : bf_lo(hu[e >> 1]);
                            }
                        }
                    }
                    const uint32_t wu[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const double wd = (e & 1) ? bf_hi(wu[e >> 1]) : bf_lo(wu[e >> 1]);
#pragma unroll
                        for (int c = 0; c < NC; c++) {
                            double hd;
                            if (kCacheH) {
                                hd = hdc[kCacheH ? c : 0][e];
                            } else {
                                const uint32_t hu = (e < 2) ? hv[c].x : (e < 4) ? hv[c].y : (e < 6) ? hv[c].z : hv[c].w;
                                hd = (e & 1) ? bf_hi(hu) : bf_lo(hu);
                            }
                            acc[r][c] = fma(wd, hd, acc[r][c]);
                        }
                    }
                }
            }
        }
        // start the next tile's weight stream before reducing this one
        const int next = tile + n_waves;
        if (next < p.geo.n_tiles) {
            const uint4* wn = W + (int64_t)next * Q * 64 + lane;
#pragma unroll
            for (int i = 0; i < D; i++)
                if (i < Q) buf[i] = wn[i * 64];
        }
        // reduce over the lr lanes of each row group (fixed tree)
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[r][c] = group_sum_rt(acc[r][c], lrl);

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
        if (EPI == EPI_RESIDUAL && tile + n_waves < p.geo.n_tiles) load_res(tile + n_waves);
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

// ---------------------------------------------------------------------------
// attention: one workgroup per (column, kv head)
// ---------------------------------------------------------------------------
// For the column's q heads of kv group g: per-head qk RMSNorm, rope at the
// column's position, append of this column's k', v at that position, then
// softmax(q'K^T * scale) V over positions 0..pos.  Positions before the first
// column of this sequence in the step come from the KV cache; the step's own
// earlier columns (a prefill chunk) come from LDS, so no workgroup reads a
// cache row another one writes in the same launch.
//
// Lanes split a K/V row into 16-byte chunks (LP = d/8 lanes per row); rows
// spread over lane groups and the 4 waves; each lane keeps U rows in flight.
// D_ / REP_ fix head_dim and q heads per kv head at compile time (0 = runtime).
//
// LDS (dynamic): pv[16][d] f64 | qf[rep][d] f32 | kin[8][d] bf16 |
//                vin[8][d] bf16 | S[rep][max_seq] f32
template <int D_, int REP_>
__global__ __launch_bounds__(MAK_BLOCK) void k_attn(AttnPhase p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int d = D_ > 0 ? D_ : p.head_dim;
    const int rep = REP_ > 0 ? REP_ : p.n_q_heads / p.n_kv_heads;
    constexpr int HG = (REP_ > 0 && REP_ < 4) ? REP_ : 4;   // heads per P.V pass
    const int Hq = p.n_q_heads, Hkv = p.n_kv_heads, half = d >> 1;
    const int col = blockIdx.x / Hkv;
    const int g = blockIdx.x - col * Hkv;
    const int q_dim = Hq * d, kv_dim = Hkv * d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    double* pv = reinterpret_cast<double*>(smem);
    float* qf = reinterpret_cast<float*>(pv + 16 * d);
    uint16_t* kin = reinterpret_cast<uint16_t*>(qf + rep * d);
    uint16_t* vin = kin + MAK_MAX_COLS * d;
    float* S = reinterpret_cast<float*>(vin + MAK_MAX_COLS * d);

    const int lp_log2 = __builtin_ctz(d >> 3);
    const int LP = 1 << lp_log2;
    const int rows_w = 64 >> lp_log2;
    const int rows_it = 4 * rows_w;
    const int sub = lane >> lp_log2, ch = lane & (LP - 1);
    const int my_row = wave * rows_w + sub;
    constexpr int U = 4;

    // ---- round trip 1: this column's state
    const ColState cs = p.ctl->cols[col];
    const int pos = cs.pos, fp = cs.first_pos, n = pos + 1, n_in = pos - fp + 1;
    const size_t head_base = ((size_t)cs.slot * Hkv + g) * p.max_seq;
    const uint16_t* kc_h = p.kc + head_base * d;
    const uint16_t* vc_h = p.vc + head_base * d;

    // ---- round trip 2: everything else at once.  First the leading cached
    // K and V rows (they do not depend on this step) ...
    uint4 kpre[U], vpre[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = u * rows_it + my_row;
        kpre[u] = make_uint4(0, 0, 0, 0);
        vpre[u] = make_uint4(0, 0, 0, 0);
        if (j < fp) {
            kpre[u] = *reinterpret_cast<const uint4*>(kc_h + (size_t)j * d + ch * 8);
            vpre[u] = *reinterpret_cast<const uint4*>(vc_h + (size_t)j * d + ch * 8);
        }
    }
    // ... then the raw q heads and the step's k/v rows of this sequence
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

    // per-head qk RMSNorm (one wave per vector)
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

    // rope (pairs i, i + d/2): q at pos, the step's k rows at fp + ci
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

    // append this column's k', v at pos (single owner: this workgroup)
    for (int i = tid; i < d; i += MAK_BLOCK) {
        p.kc[(head_base + pos) * d + i] = kin[(n_in - 1) * d + i];
        p.vc[(head_base + pos) * d + i] = vin[(n_in - 1) * d + i];
    }

    // scores sigma_j = bf16(bf16(q'.K_j) * scale)
    for (int j0 = 0; j0 < n; j0 += U * rows_it) {
        uint4 kv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + u * rows_it + my_row;
            if (j0 == 0) kv[u] = kpre[u];
            else kv[u] = (j < fp) ? *reinterpret_cast<const uint4*>(kc_h + (size_t)j * d + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
            if (j >= fp && j < n) kv[u] = *reinterpret_cast<const uint4*>(kin + (j - fp) * d + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + u * rows_it + my_row;
            const uint32_t ku[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
            double kd[8];
#pragma unroll
            for (int e = 0; e < 8; e++) kd[e] = (e & 1) ? bf_hi(ku[e >> 1]) : bf_lo(ku[e >> 1]);
#pragma unroll(REP_ > 0 ? REP_ : 1)
            for (int h = 0; h < rep; h++) {
                const float4 qa = *reinterpret_cast<const float4*>(qf + h * d + ch * 8);
                const float4 qb = *reinterpret_cast<const float4*>(qf + h * d + ch * 8 + 4);
                const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
                double part = 0.0;
#pragma unroll
                for (int e = 0; e < 8; e++) part = fma((double)qv[e], kd[e], part);
                part = (D_ > 0) ? group_sum<(D_ > 0 ? __builtin_ctz(D_ >> 3) : 0)>(part)
                                : group_sum_rt(part, lp_log2);
                if (ch == 0 && j < n) S[h * p.max_seq + j] = rbf(rbf((float)part) * p.scale);
            }
        }
    }
    __syncthreads();

    // softmax of each head inside one wave: max, e_j = fp32(exp(sigma_j - max)),
    // Z = fp32(sum e_j), P_j = bf16(fp32(e_j / Z)); a lane rewrites only the
    // entries it reads
    for (int h = wave; h < rep; h += 4) {
        float* Sh = S + h * p.max_seq;
        float m = -INFINITY;
        for (int j = lane; j < n; j += 64) m = fmaxf(m, Sh[j]);
        m = wave_max(m);
        double z = 0.0;
        for (int j = lane; j < n; j += 64) {
            const float e = (float)exp((double)Sh[j] - (double)m);
            Sh[j] = e;
            z += (double)e;
        }
        const double Z = (double)(float)wave_sum(z);
        for (int j = lane; j < n; j += 64) Sh[j] = rbf((float)((double)Sh[j] / Z));
    }
    __syncthreads();

    // o_h = bf16(sum_j P_j V_j): per-lane partial sums over its rows, folded
    // across lane groups, then across waves (in wave order) through LDS
    for (int h0 = 0; h0 < rep; h0 += HG) {
        double acc[HG][8];
#pragma unroll
        for (int hh = 0; hh < HG; hh++)
#pragma unroll
            for (int e = 0; e < 8; e++) acc[hh][e] = 0.0;
        for (int j0 = 0; j0 < n; j0 += U * rows_it) {
            uint4 vv[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = j0 + u * rows_it + my_row;
                if (j0 == 0) vv[u] = vpre[u];
                else vv[u] = (j < fp) ? *reinterpret_cast<const uint4*>(vc_h + (size_t)j * d + ch * 8)
                                      : make_uint4(0, 0, 0, 0);
                if (j >= fp && j < n) vv[u] = *reinterpret_cast<const uint4*>(vin + (j - fp) * d + ch * 8);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = j0 + u * rows_it + my_row;
                if (j >= n) continue;
                const uint32_t vu[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
                for (int hh = 0; hh < HG; hh++) {
                    if (h0 + hh >= rep) break;
                    const double pj = (double)S[(h0 + hh) * p.max_seq + j];
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        acc[hh][e] = fma(pj, (double)((e & 1) ? bf_hi(vu[e >> 1]) : bf_lo(vu[e >> 1])), acc[hh][e]);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < HG; hh++)
#pragma unroll
            for (int e = 0; e < 8; e++) {
                if (D_ > 0) {
                    acc[hh][e] = stride_sum<(D_ > 0 ? __builtin_ctz(D_ >> 3) : 1)>(acc[hh][e]);
                } else {
                    for (int o = LP; o < 64; o <<= 1) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);
                }
            }
        if (sub == 0) {
#pragma unroll
            for (int hh = 0; hh < HG; hh++)
#pragma unroll
                for (int e = 0; e < 8; e++) pv[(wave * 4 + hh) * d + ch * 8 + e] = acc[hh][e];
        }
        __syncthreads();
        for (int t = tid; t < HG * d; t += MAK_BLOCK) {
            const int hh = t / d, i = t - hh * d;
            if (h0 + hh < rep) {
                const double v = ((pv[(0 * 4 + hh) * d + i] + pv[(1 * 4 + hh) * d + i]) +
                                  pv[(2 * 4 + hh) * d + i]) + pv[(3 * 4 + hh) * d + i];
                p.o[(size_t)col * q_dim + (g * rep + h0 + hh) * d + i] = f2bf((float)v);
            }
        }
        __syncthreads();
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

// dynamic LDS of k_attn: pv[16][d] f64 | qf[rep][d] f32 | kin, vin [8][d] bf16 | S[rep][max_seq] f32
size_t mak_attn_lds_for(int rep, int d, int max_seq)
{
    return (size_t)16 * d * 8 + (size_t)rep * d * 4 + 2 * (size_t)MAK_MAX_COLS * d * 2 +
           (size_t)rep * max_seq * 4;
}

size_t mak_attn_lds(const AttnPhase& p)
{
    return mak_attn_lds_for(p.n_q_heads / p.n_kv_heads, p.head_dim, p.max_seq);
}

#define MAK_ATTN_SHAPES(X) X(32, 3) X(64, 2) X(64, 3) X(64, 4) X(64, 8) X(128, 2) X(128, 4)

hipError_t mak_launch_attn(const AttnPhase& p, hipStream_t st)
{
    const dim3 grid(p.ncols * p.n_kv_heads), block(MAK_BLOCK);
    const size_t lds = mak_attn_lds(p);
    const int rep = p.n_q_heads / p.n_kv_heads;
#define X(D, REP)                                                                  \
    if (p.head_dim == D && rep == REP) {                                           \
        hipLaunchKernelGGL((k_attn<D, REP>), grid, block, lds, st, p);           \
        return hipGetLastError();                                                  \
    }
    MAK_ATTN_SHAPES(X)
#undef X
    hipLaunchKernelGGL((k_attn<0, 0>), grid, block, lds, st, p);
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

// Raise the dynamic-LDS ceiling of the GEMV instantiations to `bytes` and of
// the attention kernel to `attn_bytes`.
hipError_t mak_set_lds_limit(int bytes, int attn_bytes)
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
#define X(D, REP)                                                                          \
    {                                                                                      \
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<D, REP>),  \
                                           hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                           attn_bytes);                                    \
        if (e != hipSuccess) return e;                                                     \
    }
    MAK_ATTN_SHAPES(X)
#undef X
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<0, 0>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, attn_bytes);
#undef SETA
#undef SETE
#undef SETN
}
