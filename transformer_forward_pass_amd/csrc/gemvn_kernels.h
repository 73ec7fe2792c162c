// gemvn_kernels.h -- the multi-column GEMV of prefill chunks and batched
// decode (gfx950): y[c] = W x[c] for up to 16 columns, the weights streamed
// once for all of them.
//
// Same packed weight layout and the same fp64 arithmetic as the batch-1
// kernel (every product exact, sums exact before the single rounding), so a
// column's result is bitwise what it would be alone.  What changes is the
// work split, sized for the extra arithmetic of NC columns per weight:
//
//  * a lane holds RR rows (RR/R consecutive tiles) for one 16-byte chunk of
//    the input at a time, so each converted input element serves RR rows and
//    each converted weight serves NC columns;
//  * a group of RR/R tiles can be shared by JW waves of the workgroup, each
//    taking every JW-th chunk iteration (a split of K); their row sums are
//    combined through LDS in wave order after a reduce-scatter over the
//    lanes of each row, which also spreads the epilogue over those lanes;
//  * the NC input rows (RMSNorm applied) are staged once per workgroup in
//    LDS with a single barrier for all columns' statistics.
#pragma once
#include "gemv_kernels.h"

namespace mak {

// a if keep, else zero (by value: a select between two lvalues would be made
// a select between their addresses and force them into memory)
__device__ __forceinline__ uint4 keep_or_zero(bool keep, uint4 a)
{
    return make_uint4(keep ? a.x : 0u, keep ? a.y : 0u, keep ? a.z : 0u, keep ? a.w : 0u);
}

// Input staging.  RMSNorm inputs (K <= 4096): wave w stages columns w,
// w + 8, ... (at most two), each lane holding chunks lane + 64*i, so a
// column's sum of squares is one wave reduction and no barrier separates
// the statistics from the normalisation.  Raw inputs: a plain copy spread
// over all threads.
constexpr int kStageChunks = 8;   // chunks per lane for RMSNorm inputs (K <= 64*8*8)
constexpr int kStageWaves = MAK_NBLOCK / 64;

template <int NC>
struct StagedN {
    static constexpr int CR = (NC + kStageWaves - 1) / kStageWaves;   // columns per wave
    uint4 v[CR][kStageChunks];
    uint4 w[kStageChunks];   // the norm weight, the same for every column
};

template <int NC>
__device__ __forceinline__ void issue_inputs_n(const GemvPhase& p, StagedN<NC>& st)
{
    if (p.in_kind == IN_RAW) return;
    const int C = p.geo.k >> 3;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave >= NC) return;
    const int n_i = (C + 63) >> 6;
    const bool gather = p.in_kind == IN_GATHER_NORM;
    const uint4* nw = reinterpret_cast<const uint4*>(p.norm_w);
#pragma unroll
    for (int r = 0; r < StagedN<NC>::CR; r++) {
        const int cw = wave + r * kStageWaves;
        if (cw >= NC) continue;   // wave-uniform
        const int col = p.col0 + min(cw, p.ncols - 1);
        const uint4* base = gather ? reinterpret_cast<const uint4*>(p.embed)
                                   : reinterpret_cast<const uint4*>(p.in + (size_t)col * p.in_ld);
        const int token = gather ? p.ctl->cols[col].token : 0;
#pragma unroll
        for (int i = 0; i < kStageChunks; i++) {
            if (i < n_i) {
                const int q = min(lane + 64 * i, C - 1);
                st.v[r][i] = base[gather ? packed_chunk(p.embed_geo, token, q) : (int64_t)q];
                if (r == 0) st.w[i] = nw[q];   // the norm weight, with the first column
            }
        }
    }
}

// hs[c*K + k] (bf16) for c < NC; columns >= ncols are zero.
template <int NC>
__device__ __forceinline__ void finish_inputs_n(const GemvPhase& p, const StagedN<NC>& st, uint16_t* hs)
{
    const int K = p.geo.k, C = K >> 3;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint4* hs4 = reinterpret_cast<uint4*>(hs);
    if (p.in_kind == IN_RAW) {
        // NC*C chunks over all threads, 8 loads in flight per thread
        const int total = NC * C;
        for (int base = 0; base < total; base += 8 * MAK_NBLOCK) {
            uint4 v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int q = min(base + i * MAK_NBLOCK + tid, total - 1);
                const int c = q / C, k = q - c * C;
                v[i] = reinterpret_cast<const uint4*>(p.in + (size_t)(p.col0 + min(c, p.ncols - 1)) * p.in_ld)[k];
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int q = base + i * MAK_NBLOCK + tid;
                if (q < total) hs4[q] = keep_or_zero(q / C < p.ncols, v[i]);
            }
        }
        return;
    }
    if (wave >= NC) return;
    const int n_i = (C + 63) >> 6;
#pragma unroll
    for (int r = 0; r < StagedN<NC>::CR; r++) {
        const int cw = wave + r * kStageWaves;   // this wave's r-th column
        if (cw >= NC) continue;                  // wave-uniform
        const bool active = cw < p.ncols;
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < kStageChunks; i++) {
            if (i < n_i && lane + 64 * i < C) {
                const uint32_t u[4] = {st.v[r][i].x, st.v[r][i].y, st.v[r][i].z, st.v[r][i].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double a = bf_lo(u[e]), b = bf_hi(u[e]);
                    ss = fma(a, a, ss);
                    ss = fma(b, b, ss);
                }
            }
        }
        ss = wave_sum(ss);
        const float rs = rms_scale(ss, K, p.eps);
        const bool store_x = active && p.in_kind == IN_GATHER_NORM && blockIdx.x == 0;
        uint4* xs = reinterpret_cast<uint4*>(p.x_store + (size_t)(p.col0 + cw) * p.x_ld);
#pragma unroll
        for (int i = 0; i < kStageChunks; i++) {
            const int q = lane + 64 * i;
            if (i < n_i && q < C) {
                if (store_x) xs[q] = st.v[r][i];
                const uint32_t u[4] = {st.v[r][i].x, st.v[r][i].y, st.v[r][i].z, st.v[r][i].w};
                const uint32_t ww[4] = {st.w[i].x, st.w[i].y, st.w[i].z, st.w[i].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    o[e] = rms_apply2(u[e], rs, ww[e]);
                }
                hs4[cw * C + q] = keep_or_zero(active, make_uint4(o[0], o[1], o[2], o[3]));
            }
        }
    }
}

// Order LDS accesses within one wave (a wave's LDS operations execute in
// order; this keeps the compiler from moving them across this point).
__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Values a lane keeps after the reduce-scatter of V = rr*nc row sums over
// 2^lr_log2 lanes (SwiGLU keeps gate/up pairs together: one halving fewer).
__host__ __device__ inline int gemvn_kept(int rr, int nc, int lr_log2, bool pairs)
{
    int logv = 0;
    while ((1 << logv) < rr * nc) logv++;
    const int h = lr_log2 < logv - (pairs ? 1 : 0) ? lr_log2 : logv - (pairs ? 1 : 0);
    return (rr * nc) >> h;
}

// Dynamic LDS of k_gemvn: staged inputs, then (waves sharing a group only)
// every wave's kept sums [wave][kept][lane].
__host__ __device__ inline size_t gemvn_part_offset(int nc, int k) { return ((size_t)nc * k * 2 + 15) & ~(size_t)15; }
__host__ __device__ inline size_t gemvn_lds(int nc, int k, int rr, int jw, int lr_log2, bool pairs)
{
    return gemvn_part_offset(nc, k) +
           (jw > 1 ? (size_t)(MAK_NBLOCK / 64) * gemvn_kept(rr, nc, lr_log2, pairs) * 64 * sizeof(double) : 0);
}

// xor-lane exchange of a double at distance 2^K (inside 64 lanes)
template <int K>
__device__ __forceinline__ double xor_lanes(double v)
{
    if (K == 0) return dpp_d<DPP_XOR1>(v);
    if (K == 1) return dpp_d<DPP_XOR2>(v);
    if (K == 3) return dpp_d<DPP_ROR8>(v);   // rotating a 16-lane row by 8 is xor 8
    if (K == 2) {
        const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), 0x101F);   // xor 4 within 32 lanes
        const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), 0x101F);
        return __hiloint2double(hi, lo);
    }
    if (K == 4) return get_xor<16>(v);
    return get_xor<32>(v);
}

// Reduce-scatter of a[0..V) over the 2^lrl lanes of each row group, lane
// bits from the lowest up: at level k a lane keeps the half of its list
// selected by its bit k and adds the partner's copy of that half.  After
// min(lrl, HM) halvings (HM = log2 V, one less to keep pairs) the lane holds
// the full sums of a[0..V >> that) at list positions
// i + sum_k bit_k(lane) * (V >> (k + 1)); further levels (lrl > HM) add the
// remaining values over the rest of the group.  Every sum uses the same tree
// in every group; sums are exact in fp64, so the tree does not matter.
template <int V, int HM, int K>
__device__ __forceinline__ void rs_level(double (&a)[V], int lrl, int lane)
{
    if (K >= lrl) return;
    if (K < HM) {
        constexpr int n = V >> K, half = n >> 1;
        const bool up = (lane >> K) & 1;
#pragma unroll
        for (int i = 0; i < half; i++) {
            const double lo = a[i], hi = a[i + half];
            const double send = up ? lo : hi;
            const double keep = up ? hi : lo;
            a[i] = keep + xor_lanes<K>(send);
        }
    } else {
        constexpr int n = V >> HM;
#pragma unroll
        for (int i = 0; i < n; i++) a[i] += xor_lanes<K>(a[i]);
    }
}

template <int V, int HM>
__device__ __forceinline__ void reduce_scatter(double (&a)[V], int lrl, int lane)
{
    rs_level<V, HM, 0>(a, lrl, lane);
    rs_level<V, HM, 1>(a, lrl, lane);
    rs_level<V, HM, 2>(a, lrl, lane);
    rs_level<V, HM, 3>(a, lrl, lane);
    rs_level<V, HM, 4>(a, lrl, lane);
    rs_level<V, HM, 5>(a, lrl, lane);
}

// Work split.  A group is RR/R consecutive tiles; unit (group, j) is the RR
// 1-KiB loads of chunk iteration j of those tiles.  Wave w of a workgroup
// takes group slot w / JW of each round and the iterations j = w % JW + i*JW;
// rounds stride over the groups by gridDim.x * (waves / JW).
template <int RR, int NC, int EPI>
__global__ __launch_bounds__(MAK_NBLOCK) void k_gemvn(GemvPhase p)
{
    constexpr int NW = MAK_NBLOCK / 64;
    constexpr int V = RR * NC;
    constexpr int LOGV = (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
    constexpr int HM = (EPI == EPI_SWIGLU) ? LOGV - 1 : LOGV;   // halvings at most
    constexpr int QB = (NC <= 2) ? 16 : (NC <= 4) ? 8 : 4;   // 16-byte loads per lane per batch
    static_assert(RR * NC <= 32, "the reduce-scatter handles at most 32 values per lane");
    constexpr int UB = (QB / RR) > 0 ? QB / RR : 1;        // units per batch
    static_assert(UB * RR == QB, "batch must hold whole units");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float bval[NW][NC];
    __shared__ int bidx[NW][NC];
    __shared__ int is_last;
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
    const int K = p.geo.k, C = K >> 3;
    double* part = reinterpret_cast<double*>(smem + gemvn_part_offset(NC, K));
    const uint4* hs4 = reinterpret_cast<const uint4*>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrl = p.geo.lr_log2;
    const int lr = 1 << lrl;
    const int grp = lane >> lrl;
    const int s = lane & (lr - 1);
    const int G = 64 >> lrl;
    const int R = p.geo.r;
    const int rl = (R == 4) ? 2 : (R == 2) ? 1 : 0;
    const int J = C >> lrl;
    const int n_tiles = p.geo.n_tiles;
    const int N = p.geo.n_rows;
    const int TU = RR >> rl;                               // tiles per group
    const int NG = (n_tiles + TU - 1) / TU;
    const int JW = p.jw;                                   // power of two, <= min(J, NW)
    const int jwl = (JW == 8) ? 3 : (JW == 4) ? 2 : (JW == 2) ? 1 : 0;
    const int GPR = NW >> jwl;                             // groups per workgroup per round
    const int wj = wave & (JW - 1);
    const int wg = wave >> jwl;
    const int UW = (J - wj + JW - 1) >> jwl;               // this wave's units per group
    const int per_round = gridDim.x * GPR;
    const int rounds = (NG + per_round - 1) / per_round;   // the same in every workgroup
    const int total = rounds * UW;
    const uint4* W = reinterpret_cast<const uint4*>(p.w);

    auto group_at = [&](int round) __attribute__((always_inline)) { return (round * (int)gridDim.x + (int)blockIdx.x) * GPR + wg; };

    // issue the next UB units (past the end: repeat the last unit, unused)
    int ir = 0, ij = 0;
    auto issue = [&](uint4 (&buf)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int ub = 0; ub < UB; ub++) {
            int r_ = ir, j_ = ij;
            if (r_ >= rounds) {
                r_ = rounds - 1;
                j_ = UW - 1;
            }
            const int g = min(group_at(r_), NG - 1);
            const int64_t j = wj + j_ * JW;
#pragma unroll
            for (int u = 0; u < RR; u++) {
                const int64_t t = min((int64_t)g * TU + (u >> rl), (int64_t)n_tiles - 1);
                const int ri = u & (R - 1);
                buf[ub * RR + u] = ld_stream16(&W[((t * J + j) * R + ri) * 64 + lane]);
            }
            if (++ij == UW) {
                ij = 0;
                ir++;
            }
        }
    };

    // 1. input loads, the first weight batch, then the staged (normalised) inputs
    StagedN<NC> st;
    issue_inputs_n<NC>(p, st);
    uint4 bufA[QB], bufB[QB];
    const int n_batches = (total + UB - 1) / UB;
    if (n_batches > 0) issue(bufA);
    finish_inputs_n<NC>(p, st, hs);
    __syncthreads();

    double acc[RR][NC];
#pragma unroll
    for (int u = 0; u < RR; u++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[u][c] = 0.0;
    float best_v[NC];
    int best_i[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        best_v[c] = -INFINITY;
        best_i[c] = 0x7fffffff;
    }

    // 2. one unit: RR rows x 8 inputs x NC columns
    auto fold_unit = [&](const uint4* b, int j) __attribute__((always_inline)) {
        uint4 hv[NC];
        const int chunk = (j << lrl) + s;
#pragma unroll
        for (int c = 0; c < NC; c++) hv[c] = hs4[c * C + chunk];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            double xd[NC];
#pragma unroll
            for (int c = 0; c < NC; c++) {
                const uint32_t hu = (e < 2) ? hv[c].x : (e < 4) ? hv[c].y : (e < 6) ? hv[c].z : hv[c].w;
                xd[c] = (e & 1) ? bf_hi(hu) : bf_lo(hu);
            }
#pragma unroll
            for (int u = 0; u < RR; u++) {
                const uint32_t wu = (e < 2) ? b[u].x : (e < 4) ? b[u].y : (e < 6) ? b[u].z : b[u].w;
                const double wd = (e & 1) ? bf_hi(wu) : bf_lo(wu);
#pragma unroll
                for (int c = 0; c < NC; c++) acc[u][c] = fma(wd, xd[c], acc[u][c]);
            }
        }
    };

    // 3. a finished group: a reduce-scatter over each row's lanes leaves
    //    every lane the full sums of its share of the V values; with JW > 1
    //    waves on the group, the first wave adds the others' shares (same
    //    lane, same values) in wave order through LDS; then each lane
    //    applies the epilogue to its values (SwiGLU: gate/up pairs).
    auto epilogue_value = [&](int g, int u, int c, double y, double y_up) __attribute__((always_inline)) {
        const int64_t t = (int64_t)g * TU + (u >> rl);
        const int64_t row = t * G * R + grp * R + (u & (R - 1));
        if (t >= n_tiles || row >= N || c >= p.ncols) return;
        const size_t col = (size_t)(p.col0 + c);
        if (EPI == EPI_SWIGLU) {
            const float gv = rbf((float)y);
            const float uv = rbf((float)y_up);
            const double gd = (double)gv;
            const float z = rbf((float)(gd / (1.0 + exp(-gd))));
            p.out[col * p.out_ld + (row >> 1)] = f2bf(z * uv);
        } else if (EPI == EPI_STORE) {
            p.out[col * p.out_ld + row] = f2bf((float)y);
        } else if (EPI == EPI_RESIDUAL) {
            const float xr = bf2f(p.out[col * p.out_ld + row]);
            p.out[col * p.out_ld + row] = f2bf(xr + rbf((float)y));
        } else {  // EPI_LOGITS
            const float v = (float)y;
            p.logits[(size_t)c * p.logits_ld + row] = v;
#pragma unroll
            for (int cc = 0; cc < NC; cc++) {   // (selects, not an indexed update)
                const bool take = cc == c && (v > best_v[cc] || (v == best_v[cc] && (int)row < best_i[cc]));
                best_v[cc] = take ? v : best_v[cc];
                best_i[cc] = take ? (int)row : best_i[cc];
            }
        }
    };
    auto finish_group = [&](int round) __attribute__((always_inline)) {
        const int g = group_at(round);
        // list order c*RR + u keeps each gate/up pair (u, u+1) adjacent
        double a[V];
#pragma unroll
        for (int u = 0; u < RR; u++)
#pragma unroll
            for (int c = 0; c < NC; c++) a[c * RR + u] = acc[u][c];
        reduce_scatter<V, HM>(a, lrl, lane);
        const int hk = lrl < HM ? lrl : HM;
        const int nk = V >> hk;                           // values this lane keeps
        int off = 0;
        for (int k = 0; k < hk; k++) off += ((s >> k) & 1) * (V >> (k + 1));
        // only the first lane of each residue class past the halvings applies them
        const bool lead = (s >> hk) == 0;
        if (JW > 1) {
#pragma unroll
            for (int i = 0; i < V; i++)
                if (i < nk) part[((size_t)wave * nk + i) * 64 + lane] = a[i];
            __syncthreads();
            if (wj == 0) {
#pragma unroll
                for (int i = 0; i < V; i++) {
                    if (i >= nk) continue;
                    double y = 0.0;
                    for (int w2 = 0; w2 < JW; w2++) y += part[((size_t)(wave + w2) * nk + i) * 64 + lane];
                    a[i] = y;
                }
            }
        }
        if (wj == 0 && g < NG && lead) {
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int i = 0; i + 1 < V; i += 2) {
                    if (i >= nk) continue;
                    const int idx = off + i;                  // even: gate row u, up row u + 1
                    epilogue_value(g, idx % RR, idx / RR, a[i], a[i + 1]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < V; i++) {
                    if (i >= nk) continue;
                    const int idx = off + i;
                    epilogue_value(g, idx % RR, idx / RR, a[i], 0.0);
                }
            }
        }
        if (JW > 1) __syncthreads();   // `part` is rewritten by the next round
#pragma unroll
        for (int u = 0; u < RR; u++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[u][c] = 0.0;
    };

    int cr = 0, cj = 0;   // next unit to fold (round, iteration)
    auto compute = [&](const uint4 (&buf)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int ub = 0; ub < UB; ub++) {
            if (cr < rounds) {
                fold_unit(buf + ub * RR, wj + cj * JW);
                if (++cj == UW) {
                    finish_group(cr);
                    cj = 0;
                    cr++;
                }
            }
        }
    };

    // 4. batches ping-pong between two buffers: once one has landed, the
    //    next is issued and only then is the landed one folded (a third
    //    buffer, two batches in flight, was measured slower)
    for (int b = 0; b < n_batches; b += 2) {
        batch_ready<QB>(bufA, QB);
        if (b + 1 < n_batches) issue(bufB);
        compute(bufA);
        if (b + 1 >= n_batches) break;
        batch_ready<QB>(bufB, QB);
        if (b + 2 < n_batches) issue(bufA);
        compute(bufB);
    }

    if (EPI == EPI_LOGITS) argmax_tail<NC>(p, best_v, best_i, bval, bidx, is_last, lane, wave, NW);
}

}  // namespace mak

// rows per lane (RR) x column capacity (NC) instantiated for the multi-column GEMV
#define MAK_GEMVN_SHAPES(X) \
    X(1, 2) X(2, 2) X(4, 2) X(1, 4) X(2, 4) X(4, 4) X(1, 8) X(2, 8) X(4, 8) X(1, 16) X(2, 16)
#define MAK_GEMVN_PAIR_SHAPES(X) X(2, 2) X(4, 2) X(2, 4) X(4, 4) X(2, 8) X(4, 8) X(2, 16)

// defined in gemvn_*.hip: the kernel for (rr, nc), or nullptr
const void* mak_gemvn_fn_store(int rr, int nc);
const void* mak_gemvn_fn_residual(int rr, int nc);
const void* mak_gemvn_fn_swiglu(int rr, int nc);
const void* mak_gemvn_fn_logits(int rr, int nc);
