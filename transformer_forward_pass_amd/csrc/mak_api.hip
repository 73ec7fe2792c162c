// mak_api.hip -- host side of libmak.so: validation, weight packing, arena
// layout, rope tables, and the sequencing of the decode program's phases.
//
// "model-as-a-kernel" (Method section): model load packs the weights and
// compiles the architecture into a program of phases; every phase is run by
// all resident workgroups; prompts are consumed in chunks of at most eight
// tokens; the model owns its buffers for its lifetime ("Requirements and
// limits" section).  Here each phase is one kernel launch on the model's
// stream (stream order is the barrier between phases).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/mak.h"
#include "mak_internal.h"

// kernels.hip
hipError_t mak_launch_gemv(const GemvPhase& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
hipError_t mak_launch_attn(const AttnPhase& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
hipError_t mak_launch_attn_split(const AttnPhase& p, int stage, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
// attn_block.hip
hipError_t mak_launch_attn_block(const AttnPhase& p, int stage, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
hipError_t mak_launch_set_ctl(Ctl* ctl, const ColState* cols, int ncols, int step, hipStream_t st, hipEvent_t e0,
                              hipEvent_t e1);
hipError_t mak_set_lds_limit(int bytes, int bytes_n, int attn_bytes);
size_t mak_attn_lds_for(int rep, int d, int max_seq);
size_t mak_attn_lds(const AttnPhase& p);
int mak_gemv_nc(int ncols);
int mak_gemv_blocks(GemvPhase& p, int cap, size_t lds_budget_n);
size_t mak_gemv_lds(const GemvPhase& p);
int mak_gemm16_plan(const GemvPhase& p, int ncols, size_t lds_budget);
int mak_gemm8_plan(const GemvPhase& p, int ncols, size_t lds_budget);
int mak_check_launch(const void* fn, dim3 grid, dim3 block, size_t lds);
const char* mak_launch_check_msg();

// ---------------------------------------------------------------------------
// Static scratch of mak_decode_step_static: the step's scratch buffers
// (argmax partials, split-KV scores, chunk maxima and partial outputs of one
// column) in a fixed device array instead of the arena, for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses the array's name as an address:
// the device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail(MAK_EDEVICE, "%s failed: %s", #expr, hipGetErrorString(e_));         \
    } while (0)

constexpr size_t kAlign = 256;
constexpr int kMaxGemvBlocks = 1024;      // grid cap of a GEMV phase (waves loop over tiles)
constexpr int kLdsBudget = 96 * 1024;      // batch-1 GEMV dynamic LDS per workgroup (fp32 input row; static < 4 KiB)
constexpr int kLdsBudgetN = 144 * 1024;    // multi-column GEMV: staged inputs (<= 128 KiB) + partial sums
constexpr int kLdsInputsN = 128 * 1024;    // multi-column GEMV: NC input rows of K bf16
constexpr int kAttnLdsBudget = 150 * 1024; // attention dynamic LDS (gfx950: 160 KiB per workgroup)
constexpr int kAttnSinglePassMax = 4096;   // most positions of the single-pass attention (LDS score row)
// default split-KV threshold (pos + 1 above it): 48K / head_dim positions,
// about where the three split launches overtake the single pass (measured:
// ~300 positions at head_dim 128, ~750 at 64)
constexpr int kAttnSplitWork = 48 * 1024;
// prompt chunks (the consecutive positions of one sequence) stay single-pass
// longer: 128K / head_dim positions (measured: a 2040-token prompt in chunks
// of 16 at head_dim 64 takes 213 ms with the decode threshold, 202 ms all
// single-pass; a 512-token prompt in chunks of 8 at head_dim 128 95 -> 88 ms)
constexpr int kAttnPromptSplitWork = 128 * 1024;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int ilog2(int v)
{
    int l = 0;
    while ((1 << (l + 1)) <= v) l++;
    return l;
}

int gcd(int a, int b)
{
    while (b) {
        int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Geometry of a packed [n, k] matrix.  r = rows per lane group: the largest
// of {4, 2, 1} that still leaves >= 2048 tiles (one per resident wave), and
// even when the rows are interleaved gate/up pairs.
PackGeom make_geom(int64_t n, int k, bool pairs)
{
    PackGeom g{};
    g.n_rows = (int32_t)n;
    g.k = k;
    const int C = k / 8;
    const int lr = gcd(C, 64);
    g.lr_log2 = ilog2(lr);
    const int G = 64 / lr;
    // two rows per lane group once that still leaves >= 2048 tiles: more,
    // smaller tiles keep each wave's batches flowing (measured faster than
    // four rows on the 1B-class shapes, e.g. gate/up 20.4 -> 18.2 us)
    int r = pairs ? 2 : 1;
    if ((n + (int64_t)G * 2 - 1) / ((int64_t)G * 2) >= 2048) r = 2;
    g.r = r;
    const int64_t rows_per_tile = (int64_t)G * r;
    g.n_tiles = (int32_t)((n + rows_per_tile - 1) / rows_per_tile);
    g.bytes = (int64_t)g.n_tiles * rows_per_tile * k * 2;
    return g;
}

// Row source of a packed matrix: up to 3 stacked [rows_i, k] blocks, or
// interleaved pairs (row 2i = a[i], row 2i+1 = b[i]).
struct RowSrc {
    const uint16_t* part[3];
    int64_t rows[3];
    bool interleave;
    const uint16_t* row(int64_t n, int k) const
    {
        if (interleave) return (n & 1 ? part[1] : part[0]) + (n >> 1) * (int64_t)k;
        for (int i = 0; i < 3; i++) {
            if (n < rows[i]) return part[i] + n * (int64_t)k;
            n -= rows[i];
        }
        return nullptr;
    }
};

void pack(const PackGeom& g, const RowSrc& src, std::vector<uint16_t>& out)
{
    const int k = g.k, C = k / 8;
    const int lr = 1 << g.lr_log2, G = 64 / lr, J = C / lr;
    out.assign((size_t)(g.bytes / 2), 0);
    const int64_t rows_per_tile = (int64_t)G * g.r;
    for (int64_t n = 0; n < g.n_rows; n++) {
        const uint16_t* s = src.row(n, k);
        const int64_t tile = n / rows_per_tile;
        const int rr = (int)(n - tile * rows_per_tile);
        const int grp = rr / g.r, ri = rr % g.r;
        for (int c = 0; c < C; c++) {
            const int j = c / lr, sl = c % lr;
            const int64_t slot = ((tile * J + j) * g.r + ri) * 64 + grp * lr + sl;
            std::memcpy(&out[(size_t)slot * 8], s + (size_t)c * 8, 16);
        }
    }
}

}  // namespace

extern "C" int mak_quantize_mxfp4(const uint16_t* w, int64_t rows, int32_t k, uint8_t* codes, uint8_t* scales);

namespace {

// Quantize each row (mak_quantize_mxfp4) and place its 16-byte code chunks
// and scale bytes in slot order; padding rows are zero codes.
int pack4(const PackGeom& g, const RowSrc& src, std::vector<uint8_t>& out)
{
    const int k = g.k, C = k / MAK_MX_BLOCK;
    const int lr = 1 << g.lr_log2, G = 64 / lr, J = C / lr;
    out.assign((size_t)g.bytes, 0);
    std::vector<uint8_t> codes((size_t)k / 2), sc((size_t)C);
    const int64_t rows_per_tile = (int64_t)G * g.r;
    for (int64_t n = 0; n < g.n_rows; n++) {
        const int rc = mak_quantize_mxfp4(src.row(n, k), 1, k, codes.data(), sc.data());
        if (rc) return rc;
        const int64_t tile = n / rows_per_tile;
        const int rr = (int)(n - tile * rows_per_tile);
        const int grp = rr / g.r, ri = rr % g.r;
        for (int c = 0; c < C; c++) {
            const int j = c / lr, sl = c % lr;
            const int64_t slot = ((tile * J + j) * g.r + ri) * 64 + grp * lr + sl;
            std::memcpy(&out[(size_t)slot * 16], &codes[(size_t)c * 16], 16);
            out[(size_t)(g.scale_off + slot)] = sc[(size_t)c];
        }
    }
    return MAK_OK;
}

// ---------------------------------------------------------------------------
// 4-bit weights: OCP MXFP4 (Microscaling Formats specification v1.0).  A
// block of 32 consecutive weights of a row shares the scale 2^e, stored as
// the E8M0 byte e + 127, with e = floor(log2(block max |w|)) - 2 (2 being the
// exponent of E2M1's largest value 6) clamped to [-127, 127] (-127 for an
// all-zero block); each weight becomes the E2M1 code of w / 2^e rounded to
// nearest, ties to the even code, saturating at 6; zero keeps a clear sign.
// ---------------------------------------------------------------------------

// floor(log2 |v|) of a nonzero finite bf16 magnitude (bits without the sign)
int bf16_floor_log2(uint32_t mag)
{
    const uint32_t ef = mag >> 7;
    if (ef) return (int)ef - 127;
    return (31 - __builtin_clz(mag)) - 133;   // subnormal: mag * 2^-133
}

// E2M1 magnitude index (0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6) of |v| / 2^e.
// With |v| = M * 2^E exactly (M the integer significand), 4|v|/2^e =
// M * 2^(E - e + 2) is compared with the midpoints between neighbouring
// magnitudes, times 4: 1, 3, 5, 7, 10, 14, 20.  At a midpoint the result is
// the even index (mantissa bit 0): below at 1, 5, 10, 20, above at 3, 7, 14.
uint32_t e2m1_index(uint32_t mag, int e)
{
    if (mag == 0) return 0;
    const uint32_t ef = mag >> 7;
    const uint64_t M = ef ? (0x80u | (mag & 0x7fu)) : mag;
    const int E = (ef ? (int)ef : 1) - 134;
    const int sh = E - e + 2;
    static const uint64_t T[7] = {1, 3, 5, 7, 10, 14, 20};
    uint32_t idx = 0;
    for (int i = 0; i < 7; i++) {
        int cmp;
        if (sh >= 0) {
            const uint64_t a = sh > 40 ? UINT64_MAX : (M << sh);
            cmp = a > T[i] ? 1 : (a < T[i] ? -1 : 0);
        } else if (-sh > 40) {
            cmp = -1;
        } else {
            const uint64_t t = T[i] << (-sh);
            cmp = M > t ? 1 : (M < t ? -1 : 0);
        }
        if (cmp > 0 || (cmp == 0 && (i & 1))) idx = (uint32_t)i + 1;
        else break;
    }
    return idx;
}

// Lanes sharing one row of a 4-bit matrix.  A 4-bit chunk holds 32 inputs,
// so lanes per row trade tiles against work per tile: at 64 lanes a K = 2048
// row is one load per lane (many small tiles, each ending in a 64-lane
// reduction), at 16 lanes four.  The layout takes the most lanes (<= 64,
// dividing K/32) that leave at most 2048 tiles -- eight waves per CU on 256
// CUs, all resident at once -- and otherwise the fewest.  Measured on the 1B
// shape (us per launch, lanes 64/32/16): QKV 6.8/6.5/6.8, O 4.4/4.8/5.6,
// gate/up 20.5/14.7/12.3, down 6.9/7.6/12.5 -- the rule picks 32, 64, 16, 64.
// MAK_MXFP4_LANES (a power of two, 1..64) caps the lanes per row.
int mxfp4_max_lanes()
{
    static int v = 0;
    if (!v) {
        const char* e = getenv("MAK_MXFP4_LANES");
        const int x = e ? atoi(e) : 0;
        v = (x >= 1 && x <= 64 && !(x & (x - 1))) ? x : 64;
    }
    return v;
}

// most tiles of a 4-bit matrix layout (MAK_MXFP4_MAX_TILES overrides)
int64_t mxfp4_max_tiles()
{
    static int64_t v = 0;
    if (!v) {
        const char* e = getenv("MAK_MXFP4_MAX_TILES");
        const long x = e ? atol(e) : 0;
        v = (x >= 64 && x <= (1 << 20)) ? x : 2048;
    }
    return v;
}

// rows per lane group of an [n, k] matrix with G groups per wave (make_geom's rule)
int rows_per_group(int64_t n, int G, bool pairs)
{
    int r = pairs ? 2 : 1;
    if ((n + (int64_t)G * 2 - 1) / ((int64_t)G * 2) >= 2048) r = 2;
    return r;
}

// Geometry of a packed 4-bit [n, k] matrix (mak_internal.h): 16-byte chunks
// of 32 codes, the row-group rule of make_geom.
PackGeom make_geom4(int64_t n, int k, bool pairs)
{
    PackGeom g{};
    g.n_rows = (int32_t)n;
    g.k = k;
    g.fmt = MAK_FMT_MXFP4;
    const int C = k / MAK_MX_BLOCK;
    int lr = gcd(C, mxfp4_max_lanes());
    while (lr > 1) {
        const int G = 64 / lr;
        const int64_t rows_per_tile = (int64_t)G * rows_per_group(n, G, pairs);
        if ((n + rows_per_tile - 1) / rows_per_tile <= mxfp4_max_tiles()) break;
        lr >>= 1;
    }
    g.lr_log2 = ilog2(lr);
    const int G = 64 / lr;
    g.r = rows_per_group(n, G, pairs);
    const int64_t rows_per_tile = (int64_t)G * g.r;
    g.n_tiles = (int32_t)((n + rows_per_tile - 1) / rows_per_tile);
    const int64_t slots = (int64_t)g.n_tiles * rows_per_tile * C;
    g.scale_off = slots * 16;
    g.bytes = (int64_t)align_up((size_t)(g.scale_off + slots));
    return g;
}

struct LayerDev {
    size_t attn_norm, mlp_norm, q_norm, k_norm;
    size_t w_qkv, w_o, w_gu, w_down;
    size_t k_cache, v_cache;
};

struct Layout {
    PackGeom g_embed, g_lm, g_qkv, g_o, g_gu, g_down;
    size_t ctl, out_tokens, x, qkv, o, m, logits, part_val, part_idx;
    size_t att_sc, att_cmax, att_opart;   // split-KV attention scratch
    int n_chunks, s_cap;
    size_t cos_t, sin_t, embed, lm_head, final_norm;
    std::vector<LayerDev> layers;
    size_t total;
    int qkv_ld;
};

int validate_cfg(const mak_config* c)
{
    if (!c) return fail(MAK_EINVAL, "cfg is NULL");
    if (c->n_layers < 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0 || c->max_seq <= 0 ||
        c->max_batch <= 0)
        return fail(MAK_EINVAL, "non-positive dimension in cfg");
    if (c->hidden % 8 || c->intermediate % 8 || (c->n_q_heads * c->head_dim) % 8)
        return fail(MAK_EINVAL, "hidden, intermediate and q_dim must be multiples of 8");
    if (c->head_dim < 16 || c->head_dim > 128 || (c->head_dim & (c->head_dim - 1)))
        return fail(MAK_EINVAL, "head_dim must be a power of two in [16, 128]");
    if (c->n_q_heads % c->n_kv_heads)
        return fail(MAK_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
    if (c->n_q_heads / c->n_kv_heads > 32)
        return fail(MAK_EINVAL, "more than 32 query heads per kv head");
    if (c->max_batch > MAK_MAX_BATCH) return fail(MAK_EINVAL, "max_batch > %d", MAK_MAX_BATCH);
    if (c->hidden > 4096) return fail(MAK_EINVAL, "hidden > 4096 is not supported");
    if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0f))
        return fail(MAK_EINVAL, "rms_eps must be >= 0 and rope_theta > 0");
    if (c->max_seq > (1 << 20)) return fail(MAK_EINVAL, "max_seq too large");
    if (c->weight_format != MAK_WEIGHTS_BF16 && c->weight_format != MAK_WEIGHTS_MXFP4)
        return fail(MAK_EINVAL, "weight_format must be MAK_WEIGHTS_BF16 or MAK_WEIGHTS_MXFP4");
    if (c->weight_format == MAK_WEIGHTS_MXFP4 &&
        (c->hidden % MAK_MX_BLOCK || c->intermediate % MAK_MX_BLOCK || (c->n_q_heads * c->head_dim) % MAK_MX_BLOCK))
        return fail(MAK_EINVAL, "4-bit weights need hidden, intermediate and q_dim multiples of 32");
    const size_t attn_lds = mak_attn_lds_for(c->n_q_heads / c->n_kv_heads, c->head_dim,
                                             std::min(c->max_seq, kAttnSinglePassMax));
    if (attn_lds > (size_t)kAttnLdsBudget)
        return fail(MAK_EINVAL, "attention workspace (%zu B of LDS) exceeds %d B: lower max_seq",
                    attn_lds, kAttnLdsBudget);
    return MAK_OK;
}

Layout make_layout(const mak_config* c)
{
    Layout L{};
    const int H = c->hidden, d = c->head_dim, I = c->intermediate, V = c->vocab;
    const int q_dim = c->n_q_heads * d, kv_dim = c->n_kv_heads * d;
    L.g_embed = make_geom(V, H, false);
    L.g_lm = L.g_embed;
    auto geom = (c->weight_format == MAK_WEIGHTS_MXFP4) ? make_geom4 : make_geom;
    L.g_qkv = geom(q_dim + 2 * kv_dim, H, false);
    L.g_o = geom(H, q_dim, false);
    L.g_gu = geom(2 * (int64_t)I, H, true);
    L.g_down = geom(H, I, false);
    L.qkv_ld = q_dim + 2 * kv_dim;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.ctl = take(sizeof(Ctl));
    L.out_tokens = take((size_t)c->max_seq * MAK_MAX_COLS * 4);
    L.x = take((size_t)MAK_MAX_COLS * H * 2);
    L.qkv = take((size_t)MAK_MAX_COLS * L.qkv_ld * 2);
    L.o = take((size_t)MAK_MAX_COLS * q_dim * 2);
    L.m = take((size_t)MAK_MAX_COLS * I * 2);
    L.logits = take((size_t)MAK_MAX_COLS * V * 4);
    L.part_val = take((size_t)kMaxGemvBlocks * MAK_MAX_COLS * 4);
    L.part_idx = take((size_t)kMaxGemvBlocks * MAK_MAX_COLS * 4);
    L.n_chunks = (c->max_seq + MAK_ATTN_CHUNK - 1) / MAK_ATTN_CHUNK;
    L.s_cap = std::min(c->max_seq, kAttnSinglePassMax);
    L.att_sc = take((size_t)MAK_MAX_COLS * c->n_q_heads * c->max_seq * 4);
    L.att_cmax = take((size_t)MAK_MAX_COLS * c->n_q_heads * L.n_chunks * 4);
    L.att_opart = take((size_t)MAK_MAX_COLS * c->n_q_heads * L.n_chunks * d * 8);
    L.cos_t = take((size_t)c->max_seq * (d / 2) * 2);
    L.sin_t = take((size_t)c->max_seq * (d / 2) * 2);
    L.embed = take((size_t)L.g_embed.bytes);
    L.lm_head = c->tie_embeddings ? L.embed : take((size_t)L.g_lm.bytes);
    L.final_norm = take((size_t)H * 2);
    const size_t cache_bytes = (size_t)c->max_batch * c->n_kv_heads * c->max_seq * d * 2;
    L.layers.resize(c->n_layers);
    for (int l = 0; l < c->n_layers; l++) {
        LayerDev& ld = L.layers[l];
        ld.attn_norm = take((size_t)H * 2);
        ld.mlp_norm = take((size_t)H * 2);
        ld.q_norm = c->qk_norm ? take((size_t)d * 2) : 0;
        ld.k_norm = c->qk_norm ? take((size_t)d * 2) : 0;
        ld.w_qkv = take((size_t)L.g_qkv.bytes);
        ld.w_o = take((size_t)L.g_o.bytes);
        ld.w_gu = take((size_t)L.g_gu.bytes);
        ld.w_down = take((size_t)L.g_down.bytes);
        ld.k_cache = take(cache_bytes);
        ld.v_cache = take(cache_bytes);
    }
    L.total = off;
    return L;
}

uint16_t host_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

// Scratch of one step: the LM head's per-workgroup argmax partials
// ([kMaxGemvBlocks][MAK_MAX_COLS] value and index) and the split-KV
// attention's scores, chunk maxima and partial outputs.
struct StepScratch {
    float* part_val;
    int32_t* part_idx;
    float* att_sc;
    float* att_cmax;
    double* att_opart;
};

struct PhaseTiming {
    bool on = false;
    struct Pending {
        hipEvent_t a, b;
        int kind;
    };
    std::vector<hipEvent_t> pool;
    std::vector<Pending> pending;
    double ms[MAK_PHASE_COUNT] = {};
    int64_t launches[MAK_PHASE_COUNT] = {};
};

// Attention kernel of a step: the single pass over an LDS score row (up to
// 4096 positions), split-KV, or blockwise split-KV (a prompt chunk: every
// column of one sequence, each chunk of K and V rows read once for all of
// them).
enum AttnMode { ATTN_SINGLE = 1, ATTN_SPLIT = 2, ATTN_BLOCK = 3 };

// A captured step: (ncols, lm_begin, lm_count, attention mode) -> executable graph.
struct StepGraph {
    int ncols, lm_begin, lm_count, attn;
    hipGraphExec_t exec;
};

struct mak_model {
    mak_config cfg;
    PhaseTiming tm;
    hipStream_t cur = nullptr;       // stream the phase launches go to (capture or model stream)
    hipStream_t capture = nullptr;   // private stream used only to capture step graphs
    bool use_graphs = true;
    int prefill_chunk = MAK_PREFILL_CHUNK;   // prompt tokens per prefill step (<= MAK_MAX_COLS)
    int split_above = 0;                 // split-KV attention once pos + 1 exceeds this
    int prompt_split_above = 0;          // the same for prompt chunks (blockwise)
    bool block_attn = true;              // prompt chunks past split_above run blockwise
    std::vector<StepGraph> graphs;
    Layout L;
    char* arena;
    size_t arena_bytes;
    hipStream_t stream;
    std::vector<int32_t> slot_len;   // cached positions per slot
    int device = 0;                  // the GPU current at mak_load
    bool untimed = false;            // launches carry no timing events (the static-scratch step)
    template <class T>
    T* at(size_t off) const { return reinterpret_cast<T*>(arena + off); }
};

namespace {

hipEvent_t take_event(mak_model* m)
{
    if (!m->tm.pool.empty()) {
        hipEvent_t e = m->tm.pool.back();
        m->tm.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch through `fn(e0, e1)` (returns hipError_t).  With phase timing on,
// e0/e1 are events that HIP stamps at the kernel's own start and end.
template <class F>
int launch(mak_model* m, int kind, F&& fn)
{
    hipEvent_t a = nullptr, b = nullptr;
    const bool timed = m->tm.on && !m->untimed;
    if (timed) {
        a = take_event(m);
        b = take_event(m);
        if (!a || !b) return fail(MAK_EDEVICE, "hipEventCreate failed");
    }
    const hipError_t e = fn(a, b);
    if (e == hipErrorInvalidConfiguration) return fail(MAK_EINVAL, "%s", mak_launch_check_msg());
    if (e != hipSuccess) return fail(MAK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    if (timed) m->tm.pending.push_back({a, b, kind});
    return MAK_OK;
}

// After the stream has drained: fold pending event pairs into the totals.
int collect_timing(mak_model* m)
{
    for (auto& p : m->tm.pending) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, p.a, p.b));
        m->tm.ms[p.kind] += ms;
        m->tm.launches[p.kind] += 1;
        m->tm.pool.push_back(p.a);
        m->tm.pool.push_back(p.b);
    }
    m->tm.pending.clear();
    return MAK_OK;
}

// Largest column group whose fp32 inputs, staged in padded 32-input blocks
// (36 floats each), fit the LDS budget of the 4-bit GEMV (at most 8).
int max_cols_for_k4(int k)
{
    const int n = kLdsInputsN / ((k / MAK_MX_BLOCK) * 36 * 4);
    return n >= 8 ? 8 : n >= 4 ? 4 : n >= 2 ? 2 : 1;
}

// Largest column group whose bf16 input rows fit the LDS budget.
int max_cols_for_k(int k)
{
    int n = kLdsInputsN / (k * 2);
    if (n >= 16) return 16;
    if (n >= 8) return 8;
    if (n >= 4) return 4;
    if (n >= 2) return 2;
    return 1;
}

int run_gemv(mak_model* m, int kind, GemvPhase p, int ncols, int col0)
{
    // split the columns into groups whose inputs fit in LDS (the matrix-core
    // kernel stages at most 16 RMSNorm inputs of K <= 4096 and reads raw
    // inputs from memory: one launch)
    const bool q4 = p.geo.fmt == MAK_FMT_MXFP4;
    const bool mfma = !q4 && (mak_gemm16_plan(p, ncols, kLdsBudgetN) != 0 || mak_gemm8_plan(p, ncols, kLdsBudgetN) != 0);
    const int step = q4 ? max_cols_for_k4(p.geo.k)
                        : (p.epi == EPI_LOGITS || mfma) ? ncols : max_cols_for_k(p.geo.k);
    if (q4 && p.epi == EPI_LOGITS) return fail(MAK_EINVAL, "internal: 4-bit LM head");
    if (p.epi == EPI_LOGITS && !mfma && max_cols_for_k(p.geo.k) < ncols)
        return fail(MAK_EINVAL, "LM head input too wide for %d columns", ncols);
    for (int c0 = 0; c0 < ncols; c0 += step) {
        GemvPhase q = p;
        q.col0 = col0 + c0;
        q.ncols = std::min(step, ncols - c0);
        q.n_blocks = mak_gemv_blocks(q, kMaxGemvBlocks, kLdsBudgetN);
        if (q.epi == EPI_LOGITS && q.col0 != col0)
            return fail(MAK_EINVAL, "internal: LM head split");
        // host-side shape checks of what the kernel assumes
        if (q.geo.k % (q4 ? MAK_MX_BLOCK : 8) || q.ncols < 1 || q.ncols > MAK_MAX_COLS ||
            q.col0 + q.ncols > MAK_MAX_COLS || (q4 && q.ncols > 8) ||
            mak_gemv_lds(q) > (size_t)(q4 ? kLdsInputsN : q.multi ? kLdsBudgetN : kLdsBudget) || q.n_blocks < 1 ||
            (q.epi == EPI_SWIGLU && (q.geo.r % 2)) ||
            (q.multi && q.in_kind != IN_RAW && (q.geo.k >> 3) > MAK_NBLOCK))
            return fail(MAK_EINVAL, "internal: bad GEMV phase");
        int rc = launch(m, kind, [&](hipEvent_t e0, hipEvent_t e1) { return mak_launch_gemv(q, m->cur, e0, e1); });
        if (rc) return rc;
    }
    return MAK_OK;
}

// Launch one step of the program on m->cur for the columns currently in the
// control block: ncols columns; LM head (with argmax feedback) for
// [lm_begin, lm_begin + lm_count).  `sc` holds the step's scratch buffers.
int record_step(mak_model* m, int ncols, int lm_begin, int lm_count, int32_t* d_out_tokens, int attn,
                const StepScratch& sc)
{
    const mak_config& c = m->cfg;
    const Layout& L = m->L;
    const int H = c.hidden, d = c.head_dim, q_dim = c.n_q_heads * d;
    Ctl* ctl = m->at<Ctl>(L.ctl);
    uint16_t* x = m->at<uint16_t>(L.x);
    uint16_t* qkv = m->at<uint16_t>(L.qkv);
    uint16_t* o = m->at<uint16_t>(L.o);
    uint16_t* mm = m->at<uint16_t>(L.m);

    for (int l = 0; l < c.n_layers; l++) {
        const LayerDev& ld = L.layers[l];
        int rc;
        // RMSNorm + QKV
        GemvPhase p{};
        p.w = m->at<void>(ld.w_qkv);
        p.geo = L.g_qkv;
        p.in_kind = (l == 0) ? IN_GATHER_NORM : IN_NORM;
        p.epi = EPI_STORE;
        p.in = x;
        p.in_ld = H;
        p.eps = c.rms_eps;
        p.norm_w = m->at<uint16_t>(ld.attn_norm);
        p.embed = m->at<void>(L.embed);
        p.embed_geo = L.g_embed;
        p.x_store = x;
        p.x_ld = H;
        p.out = qkv;
        p.out_ld = L.qkv_ld;
        p.ctl = ctl;
        if ((rc = run_gemv(m, MAK_PHASE_QKV, p, ncols, 0))) return rc;

        // attention
        AttnPhase a{};
        a.qkv = qkv;
        a.qkv_ld = L.qkv_ld;
        a.kc = m->at<uint16_t>(ld.k_cache);
        a.vc = m->at<uint16_t>(ld.v_cache);
        a.cos_t = m->at<uint16_t>(L.cos_t);
        a.sin_t = m->at<uint16_t>(L.sin_t);
        a.q_norm = c.qk_norm ? m->at<uint16_t>(ld.q_norm) : nullptr;
        a.k_norm = c.qk_norm ? m->at<uint16_t>(ld.k_norm) : nullptr;
        a.o = o;
        a.ctl = ctl;
        a.ncols = ncols;
        a.n_q_heads = c.n_q_heads;
        a.n_kv_heads = c.n_kv_heads;
        a.head_dim = d;
        a.max_seq = c.max_seq;
        a.eps = c.rms_eps;
        a.scale = (float)(1.0 / std::sqrt((double)d));
        a.sc = sc.att_sc;
        a.cmax = sc.att_cmax;
        a.opart = sc.att_opart;
        a.n_chunks = L.n_chunks;
        a.s_cap = L.s_cap;
        if (mak_attn_lds(a) > (size_t)kAttnLdsBudget) return fail(MAK_EINVAL, "internal: attention LDS");
        if (attn == ATTN_BLOCK) {
            for (int stage = 0; stage < 4; stage++)
                if ((rc = launch(m, MAK_PHASE_ATTN, [&](hipEvent_t e0, hipEvent_t e1) {
                         return stage < 3 ? mak_launch_attn_block(a, stage, m->cur, e0, e1)
                                          : mak_launch_attn_split(a, 2, m->cur, e0, e1);
                     })))
                    return rc;
        } else if (attn == ATTN_SPLIT) {
            for (int stage = 0; stage < 3; stage++)
                if ((rc = launch(m, MAK_PHASE_ATTN, [&](hipEvent_t e0, hipEvent_t e1) {
                         return mak_launch_attn_split(a, stage, m->cur, e0, e1);
                     })))
                    return rc;
        } else if ((rc = launch(m, MAK_PHASE_ATTN, [&](hipEvent_t e0, hipEvent_t e1) {
                        return mak_launch_attn(a, m->cur, e0, e1);
                    }))) {
            return rc;
        }

        // O + residual
        GemvPhase po{};
        po.w = m->at<void>(ld.w_o);
        po.geo = L.g_o;
        po.in_kind = IN_RAW;
        po.epi = EPI_RESIDUAL;
        po.in = o;
        po.in_ld = q_dim;
        po.out = x;
        po.out_ld = H;
        po.ctl = ctl;
        if ((rc = run_gemv(m, MAK_PHASE_O, po, ncols, 0))) return rc;

        // RMSNorm + gate/up + SwiGLU
        GemvPhase pg{};
        pg.w = m->at<void>(ld.w_gu);
        pg.geo = L.g_gu;
        pg.in_kind = IN_NORM;
        pg.epi = EPI_SWIGLU;
        pg.in = x;
        pg.in_ld = H;
        pg.eps = c.rms_eps;
        pg.norm_w = m->at<uint16_t>(ld.mlp_norm);
        pg.out = mm;
        pg.out_ld = c.intermediate;
        pg.ctl = ctl;
        if ((rc = run_gemv(m, MAK_PHASE_GATEUP, pg, ncols, 0))) return rc;

        // down + residual
        GemvPhase pd{};
        pd.w = m->at<void>(ld.w_down);
        pd.geo = L.g_down;
        pd.in_kind = IN_RAW;
        pd.epi = EPI_RESIDUAL;
        pd.in = mm;
        pd.in_ld = c.intermediate;
        pd.out = x;
        pd.out_ld = H;
        pd.ctl = ctl;
        if ((rc = run_gemv(m, MAK_PHASE_DOWN, pd, ncols, 0))) return rc;
    }
    if (lm_count > 0) {
        GemvPhase p{};
        p.w = m->at<void>(L.lm_head);
        p.geo = L.g_lm;
        p.in_kind = (c.n_layers == 0) ? IN_GATHER_NORM : IN_NORM;
        p.epi = EPI_LOGITS;
        p.in = x;
        p.in_ld = H;
        p.eps = c.rms_eps;
        p.norm_w = m->at<uint16_t>(L.final_norm);
        p.embed = m->at<void>(L.embed);
        p.embed_geo = L.g_embed;
        p.x_store = x;
        p.x_ld = H;
        p.logits = m->at<float>(L.logits);
        p.logits_ld = c.vocab;
        p.part_val = sc.part_val;
        p.part_idx = sc.part_idx;
        p.out_tokens = d_out_tokens;
        p.ctl = ctl;
        int rc = run_gemv(m, MAK_PHASE_LMHEAD, p, lm_count, lm_begin);
        if (rc) return rc;
    }
    return MAK_OK;
}

// Every kernel node of a captured step graph must satisfy the launch rules
// its launch was checked against (grid, workgroup bound, LDS ceilings).
int check_graph(hipGraph_t graph)
{
    size_t n = 0;
    HIP_TRY(hipGraphGetNodes(graph, nullptr, &n));
    std::vector<hipGraphNode_t> nodes(n);
    if (n) HIP_TRY(hipGraphGetNodes(graph, nodes.data(), &n));
    for (size_t i = 0; i < n; i++) {
        hipGraphNodeType t;
        HIP_TRY(hipGraphNodeGetType(nodes[i], &t));
        if (t != hipGraphNodeTypeKernel) continue;
        hipKernelNodeParams kp{};
        HIP_TRY(hipGraphKernelNodeGetParams(nodes[i], &kp));
        if (mak_check_launch(kp.func, kp.gridDim, kp.blockDim, kp.sharedMemBytes))
            return fail(MAK_EINVAL, "captured node %zu: %s", i, mak_launch_check_msg());
    }
    return MAK_OK;
}

// Run one step: replay (capturing on first use) the step's graph on the
// model's stream, or launch the phases one by one when graphs are off or
// phase timing is on.  The step reads its per-call state (tokens, positions,
// slots) from the control block, so one graph serves every step of a shape.
// max_n = the largest pos + 1 among the step's columns: above the model's
// threshold (or past the single-pass capacity) attention runs split-KV,
// blockwise when the step is a prompt chunk (one_seq: columns are the
// consecutive positions of one sequence).
StepScratch arena_scratch(const mak_model* m)
{
    const Layout& L = m->L;
    return StepScratch{m->at<float>(L.part_val), m->at<int32_t>(L.part_idx), m->at<float>(L.att_sc),
                       m->at<float>(L.att_cmax), m->at<double>(L.att_opart)};
}

// Attention kernel for a step whose longest context is max_n positions:
// split-KV above the model's threshold or past the single-pass capacity,
// blockwise for a prompt chunk of two or more columns.
int attn_mode(const mak_model* m, int max_n, int ncols = 1, bool one_seq = false)
{
    const int above = (one_seq && ncols >= 2) ? m->prompt_split_above : m->split_above;
    if (max_n <= above && max_n <= m->L.s_cap) return ATTN_SINGLE;
    return (one_seq && ncols >= 2 && m->block_attn) ? ATTN_BLOCK : ATTN_SPLIT;
}

int run_step(mak_model* m, int ncols, int lm_begin, int lm_count, int32_t* d_out_tokens, int max_n,
             bool one_seq = false)
{
    const int attn = attn_mode(m, max_n, ncols, one_seq);
    const StepScratch sc = arena_scratch(m);
    if (!m->use_graphs || m->tm.on) {
        m->cur = m->stream;
        return record_step(m, ncols, lm_begin, lm_count, d_out_tokens, attn, sc);
    }
    for (const StepGraph& g : m->graphs)
        if (g.ncols == ncols && g.lm_begin == lm_begin && g.lm_count == lm_count && g.attn == attn) {
            HIP_TRY(hipGraphLaunch(g.exec, m->stream));
            return MAK_OK;
        }
    hipGraph_t graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(m->capture, hipStreamCaptureModeThreadLocal));
    m->cur = m->capture;
    int rc = record_step(m, ncols, lm_begin, lm_count, d_out_tokens, attn, sc);
    hipError_t e = hipStreamEndCapture(m->capture, &graph);
    m->cur = m->stream;
    if (rc) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (e != hipSuccess) return fail(MAK_EDEVICE, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
    if ((rc = check_graph(graph))) {
        (void)hipGraphDestroy(graph);
        return rc;
    }
    StepGraph sg{ncols, lm_begin, lm_count, attn, nullptr};
    e = hipGraphInstantiate(&sg.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(MAK_EDEVICE, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
    m->graphs.push_back(sg);
    HIP_TRY(hipGraphLaunch(sg.exec, m->stream));
    return MAK_OK;
}

int set_cols(mak_model* m, const ColState* cols, int ncols, int step)
{
    m->cur = m->stream;
    return launch(m, MAK_PHASE_CTL,
                  [&](hipEvent_t e0, hipEvent_t e1) {
                      return mak_launch_set_ctl(m->at<Ctl>(m->L.ctl), cols, ncols, step, m->stream, e0, e1);
                  });
}

// Consume ids[0..n) of `slot` from start_pos; LM head on the last token when
// want_lm.  Leaves the control block holding the next decode column.
int prefill_chunks(mak_model* m, int slot, const int32_t* ids, int n, int start_pos, bool want_lm,
                   int step0)
{
    for (int c0 = 0; c0 < n; c0 += m->prefill_chunk) {
        const int T = std::min(m->prefill_chunk, n - c0);
        ColState cols[MAK_MAX_COLS] = {};
        for (int t = 0; t < T; t++) {
            cols[t].token = ids[c0 + t];
            cols[t].pos = start_pos + c0 + t;
            cols[t].slot = slot;
            cols[t].first_pos = start_pos + c0;
            cols[t].first_col = 0;
        }
        int rc = set_cols(m, cols, T, step0);
        if (rc) return rc;
        const bool last = c0 + T >= n;
        rc = run_step(m, T, T - 1, (last && want_lm) ? 1 : 0, m->at<int32_t>(m->L.out_tokens), start_pos + c0 + T,
                      true);
        if (rc) return rc;
    }
    return MAK_OK;
}

int check_model(const mak_model* m)
{
    if (!m) return fail(MAK_EINVAL, "model is NULL");
    return MAK_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the
// first call for that device).
int static_scratch_ptr(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return fail(MAK_EDEVICE, "device %d beyond the static scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MAK_EDEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MAK_OK;
}

// Carve one column's step scratch out of the static array; MAK_EINVAL if
// this model's shape needs more than the array holds.
int static_step_scratch(const mak_model* m, StepScratch* out)
{
    void* base = nullptr;
    int rc = static_scratch_ptr(m->device, &base);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    const size_t part = (size_t)kMaxGemvBlocks * MAK_MAX_COLS * 4;
    const size_t sc = (size_t)c.n_q_heads * c.max_seq * 4;
    const size_t cm = (size_t)c.n_q_heads * m->L.n_chunks * 4;
    const size_t op = (size_t)c.n_q_heads * m->L.n_chunks * c.head_dim * 8;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const size_t o_pv = take(part), o_pi = take(part), o_sc = take(sc), o_cm = take(cm), o_op = take(op);
    if (off > kStaticScratchBytes)
        return fail(MAK_EINVAL,
                    "this model needs %zu bytes of step scratch (n_q_heads %d, max_seq %d, head_dim %d); "
                    "the static scratch holds %zu",
                    off, c.n_q_heads, c.max_seq, c.head_dim, kStaticScratchBytes);
    char* b = static_cast<char*>(base);
    *out = StepScratch{reinterpret_cast<float*>(b + o_pv), reinterpret_cast<int32_t*>(b + o_pi),
                       reinterpret_cast<float*>(b + o_sc), reinterpret_cast<float*>(b + o_cm),
                       reinterpret_cast<double*>(b + o_op)};
    return MAK_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* mak_last_error(void) { return g_err.c_str(); }

int mak_quantize_mxfp4(const uint16_t* w, int64_t rows, int32_t k, uint8_t* codes, uint8_t* scales)
{
    if (!w || !codes || !scales) return fail(MAK_EINVAL, "null pointer");
    if (rows < 0 || k <= 0 || k % MAK_MX_BLOCK) return fail(MAK_EINVAL, "rows >= 0 and k a positive multiple of 32");
    const int nb = k / MAK_MX_BLOCK;
    // validate every weight first, so a failing call writes nothing
    for (int64_t i = 0; i < rows * (int64_t)k; i++)
        if (((w[i] >> 7) & 0xffu) == 0xffu)
            return fail(MAK_EINVAL, "weight %lld (row %lld) is not finite", (long long)i, (long long)(i / k));
    for (int64_t r = 0; r < rows; r++) {
        for (int b = 0; b < nb; b++) {
            const uint16_t* v = w + r * k + (int64_t)b * MAK_MX_BLOCK;
            uint32_t amax = 0;
            for (int i = 0; i < MAK_MX_BLOCK; i++) amax = std::max<uint32_t>(amax, v[i] & 0x7fffu);
            int e = amax ? bf16_floor_log2(amax) - 2 : -127;
            e = std::min(127, std::max(-127, e));
            scales[r * nb + b] = (uint8_t)(e + 127);
            uint8_t* out = codes + r * (k / 2) + (int64_t)b * (MAK_MX_BLOCK / 2);
            for (int i = 0; i < MAK_MX_BLOCK; i += 2) {
                uint32_t q[2];
                for (int h = 0; h < 2; h++) {
                    const uint32_t idx = e2m1_index(v[i + h] & 0x7fffu, e);
                    q[h] = idx | ((idx && (v[i + h] & 0x8000u)) ? 8u : 0u);
                }
                out[i / 2] = (uint8_t)(q[0] | (q[1] << 4));
            }
        }
    }
    return MAK_OK;
}

int mak_plan(const mak_config* cfg, size_t* arena_bytes)
{
    int rc = validate_cfg(cfg);
    if (rc) return rc;
    if (!arena_bytes) return fail(MAK_EINVAL, "arena_bytes is NULL");
    *arena_bytes = make_layout(cfg).total;
    return MAK_OK;
}

int mak_load(const mak_config* cfg, const mak_weights* w, void* d_arena, size_t arena_bytes,
             void* hip_stream, mak_model** out)
{
    int rc = validate_cfg(cfg);
    if (rc) return rc;
    if (!w || !out || !d_arena) return fail(MAK_EINVAL, "NULL weights, arena or out pointer");
    if (reinterpret_cast<uintptr_t>(d_arena) % kAlign)
        return fail(MAK_EINVAL, "arena must be %zu-byte aligned", kAlign);
    const mak_config& c = *cfg;
    if (!w->embed || !w->final_norm || (c.n_layers > 0 && !w->layers))
        return fail(MAK_EINVAL, "missing embed, final_norm or layers");
    if (!c.tie_embeddings && !w->lm_head) return fail(MAK_EINVAL, "untied model needs lm_head");
    for (int l = 0; l < c.n_layers; l++) {
        const mak_layer_weights& lw = w->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.mlp_norm || !lw.w_gate ||
            !lw.w_up || !lw.w_down)
            return fail(MAK_EINVAL, "layer %d: missing weight", l);
        if (c.qk_norm ? (!lw.q_norm || !lw.k_norm) : (lw.q_norm || lw.k_norm))
            return fail(MAK_EINVAL, "layer %d: q_norm/k_norm must be given iff qk_norm", l);
    }
    Layout L = make_layout(cfg);
    if (arena_bytes < L.total)
        return fail(MAK_ENOMEM, "arena has %zu bytes, needs %zu", arena_bytes, L.total);

    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    HIP_TRY(mak_set_lds_limit(kLdsBudget, kLdsBudgetN, kAttnLdsBudget));
    char* A = reinterpret_cast<char*>(d_arena);
    const int H = c.hidden, d = c.head_dim, I = c.intermediate;
    const int q_dim = c.n_q_heads * d, kv_dim = c.n_kv_heads * d;

    std::vector<uint16_t> buf;
    auto put = [&](size_t off, const void* src, size_t bytes) -> int {
        HIP_TRY(hipMemcpyAsync(A + off, src, bytes, hipMemcpyHostToDevice, st));
        HIP_TRY(hipStreamSynchronize(st));
        return MAK_OK;
    };
    std::vector<uint8_t> buf4;
    auto put_packed = [&](size_t off, const PackGeom& g, const RowSrc& s) -> int {
        if (g.fmt == MAK_FMT_MXFP4) {
            if (const int e = pack4(g, s, buf4)) return e;
            return put(off, buf4.data(), buf4.size());
        }
        pack(g, s, buf);
        return put(off, buf.data(), buf.size() * 2);
    };
    HIP_TRY(hipMemsetAsync(A, 0, L.total, st));
    if ((rc = put_packed(L.embed, L.g_embed, RowSrc{{w->embed, nullptr, nullptr}, {c.vocab, 0, 0}, false})))
        return rc;
    if (!c.tie_embeddings &&
        (rc = put_packed(L.lm_head, L.g_lm, RowSrc{{w->lm_head, nullptr, nullptr}, {c.vocab, 0, 0}, false})))
        return rc;
    if ((rc = put(L.final_norm, w->final_norm, (size_t)H * 2))) return rc;
    for (int l = 0; l < c.n_layers; l++) {
        const mak_layer_weights& lw = w->layers[l];
        const LayerDev& ld = L.layers[l];
        if ((rc = put(ld.attn_norm, lw.attn_norm, (size_t)H * 2))) return rc;
        if ((rc = put(ld.mlp_norm, lw.mlp_norm, (size_t)H * 2))) return rc;
        if (c.qk_norm) {
            if ((rc = put(ld.q_norm, lw.q_norm, (size_t)d * 2))) return rc;
            if ((rc = put(ld.k_norm, lw.k_norm, (size_t)d * 2))) return rc;
        }
        if ((rc = put_packed(ld.w_qkv, L.g_qkv, RowSrc{{lw.wq, lw.wk, lw.wv}, {q_dim, kv_dim, kv_dim}, false})))
            return rc;
        if ((rc = put_packed(ld.w_o, L.g_o, RowSrc{{lw.wo, nullptr, nullptr}, {H, 0, 0}, false}))) return rc;
        if ((rc = put_packed(ld.w_gu, L.g_gu, RowSrc{{lw.w_gate, lw.w_up, nullptr}, {I, I, 0}, true})))
            return rc;
        if ((rc = put_packed(ld.w_down, L.g_down, RowSrc{{lw.w_down, nullptr, nullptr}, {H, 0, 0}, false})))
            return rc;
    }
    // rope tables: inv_i = fp32(theta^(-2i/d)), a = fp32(pos * inv_i), bf16(cos a), bf16(sin a)
    {
        const int half = d / 2;
        std::vector<uint16_t> ct((size_t)c.max_seq * half), stb((size_t)c.max_seq * half);
        for (int i = 0; i < half; i++) {
            const float inv = (float)std::pow((double)c.rope_theta, -2.0 * i / (double)d);
            for (int p = 0; p < c.max_seq; p++) {
                const float a = (float)p * inv;
                ct[(size_t)p * half + i] = host_bf16((float)std::cos((double)a));
                stb[(size_t)p * half + i] = host_bf16((float)std::sin((double)a));
            }
        }
        if ((rc = put(L.cos_t, ct.data(), ct.size() * 2))) return rc;
        if ((rc = put(L.sin_t, stb.data(), stb.size() * 2))) return rc;
    }
    HIP_TRY(hipStreamSynchronize(st));

    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    {
        void* unused = nullptr;   // once per device, with that device current
        if ((rc = static_scratch_ptr(dev, &unused))) return rc;
    }
    mak_model* m = new (std::nothrow) mak_model();
    if (!m) return fail(MAK_ENOMEM, "host allocation failed");
    m->device = dev;
    m->cfg = c;
    m->L = std::move(L);
    m->arena = A;
    m->arena_bytes = arena_bytes;
    m->stream = st;
    m->slot_len.assign(c.max_batch, 0);
    m->split_above = kAttnSplitWork / c.head_dim;
    m->prompt_split_above = kAttnPromptSplitWork / c.head_dim;
    m->cur = st;
    if (hipStreamCreateWithFlags(&m->capture, hipStreamNonBlocking) != hipSuccess) {
        delete m;
        return fail(MAK_EDEVICE, "hipStreamCreateWithFlags failed");
    }
    *out = m;
    g_err.clear();
    return MAK_OK;
}

int mak_batch_max(const mak_model* m) { return m ? m->cfg.max_batch : MAK_EINVAL; }

int mak_slot_length(const mak_model* m, int32_t slot)
{
    if (!m) return fail(MAK_EINVAL, "model is NULL");
    if (slot < 0 || slot >= m->cfg.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    return m->slot_len[slot];
}

int mak_read_kv(const mak_model* m, int32_t layer, int32_t slot, int32_t pos0, int32_t n,
                uint16_t* k_out, uint16_t* v_out)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (!k_out || !v_out || n < 0) return fail(MAK_EINVAL, "NULL output or n < 0");
    if (layer < 0 || layer >= c.n_layers) return fail(MAK_ERANGE, "layer %d out of range", layer);
    if (slot < 0 || slot >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    if (pos0 < 0 || (int64_t)pos0 + n > m->slot_len[slot])
        return fail(MAK_ERANGE, "positions beyond the cached length %d", m->slot_len[slot]);
    const int d = c.head_dim;
    const LayerDev& ld = m->L.layers[layer];
    for (int g = 0; g < c.n_kv_heads; g++) {
        const size_t src = (((size_t)slot * c.n_kv_heads + g) * c.max_seq + pos0) * d * 2;
        const size_t dst = (size_t)g * n * d;
        HIP_TRY(hipMemcpyAsync(k_out + dst, m->arena + ld.k_cache + src, (size_t)n * d * 2,
                               hipMemcpyDeviceToHost, m->stream));
        HIP_TRY(hipMemcpyAsync(v_out + dst, m->arena + ld.v_cache + src, (size_t)n * d * 2,
                               hipMemcpyDeviceToHost, m->stream));
    }
    HIP_TRY(hipStreamSynchronize(m->stream));
    return MAK_OK;
}

int mak_set_executor(mak_model* m, int executor)
{
    int rc = check_model(m);
    if (rc) return rc;
    if (executor != MAK_EXEC_GRAPH && executor != MAK_EXEC_PHASED)
        return fail(MAK_EINVAL, "unknown executor %d", executor);
    m->use_graphs = executor == MAK_EXEC_GRAPH;
    return MAK_OK;
}

int mak_set_attention_split(mak_model* m, int32_t above)
{
    int rc = check_model(m);
    if (rc) return rc;
    if (above < 0) return fail(MAK_EINVAL, "split threshold %d < 0", above);
    m->split_above = above;
    m->prompt_split_above = above;
    return MAK_OK;
}

int mak_set_block_attention(mak_model* m, int32_t on)
{
    int rc = check_model(m);
    if (rc) return rc;
    if (on != 0 && on != 1) return fail(MAK_EINVAL, "block attention switch %d is not 0 or 1", on);
    m->block_attn = on != 0;
    return MAK_OK;
}

int mak_set_prefill_chunk(mak_model* m, int32_t tokens)
{
    int rc = check_model(m);
    if (rc) return rc;
    if (tokens < 1 || tokens > MAK_MAX_COLS) return fail(MAK_EINVAL, "prefill chunk %d not in [1, %d]", tokens, MAK_MAX_COLS);
    m->prefill_chunk = tokens;
    return MAK_OK;
}

int mak_set_phase_timing(mak_model* m, int enable)
{
    int rc = check_model(m);
    if (rc) return rc;
    HIP_TRY(hipStreamSynchronize(m->stream));
    if ((rc = collect_timing(m))) return rc;
    m->tm.on = enable != 0;
    if (m->tm.on) {
        for (int k = 0; k < MAK_PHASE_COUNT; k++) {
            m->tm.ms[k] = 0.0;
            m->tm.launches[k] = 0;
        }
    }
    return MAK_OK;
}

int mak_phase_times(const mak_model* m, double* ms, int64_t* launches)
{
    int rc = check_model(m);
    if (rc) return rc;
    for (int k = 0; k < MAK_PHASE_COUNT; k++) {
        if (ms) ms[k] = m->tm.ms[k];
        if (launches) launches[k] = m->tm.launches[k];
    }
    return MAK_OK;
}

void mak_free(mak_model* m)
{
    if (!m) return;
    if (hipStreamSynchronize(m->stream) == hipSuccess) collect_timing(m);
    for (hipEvent_t e : m->tm.pool) (void)hipEventDestroy(e);
    for (StepGraph& g : m->graphs) (void)hipGraphExecDestroy(g.exec);
    if (m->capture) (void)hipStreamDestroy(m->capture);
    delete m;
}

int mak_prefill(mak_model* m, int32_t slot, const int32_t* ids, int32_t n, int32_t start_pos,
                float* d_logits)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (!ids || n < 1) return fail(MAK_EINVAL, "ids NULL or n < 1");
    if (slot < 0 || slot >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    if (start_pos < 0 || start_pos > m->slot_len[slot])
        return fail(MAK_ERANGE, "start_pos %d beyond cached length %d", start_pos, m->slot_len[slot]);
    if ((int64_t)start_pos + n > c.max_seq)
        return fail(MAK_ERANGE, "start_pos + n = %lld exceeds max_seq %d", (long long)start_pos + n, c.max_seq);
    for (int i = 0; i < n; i++)
        if (ids[i] < 0 || ids[i] >= c.vocab) return fail(MAK_ERANGE, "token %d out of range", ids[i]);
    if ((rc = prefill_chunks(m, slot, ids, n, start_pos, d_logits != nullptr, 0))) return rc;
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->at<float>(m->L.logits), (size_t)c.vocab * 4,
                               hipMemcpyDeviceToDevice, m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    if ((rc = collect_timing(m))) return rc;
    m->slot_len[slot] = start_pos + n;
    return MAK_OK;
}

int mak_decode_step(mak_model* m, int32_t slot, int32_t token, int32_t pos, float* d_logits,
                    int32_t* next_token)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (slot < 0 || slot >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    if (token < 0 || token >= c.vocab) return fail(MAK_ERANGE, "token %d out of range", token);
    if (pos < 0 || pos >= c.max_seq) return fail(MAK_ERANGE, "pos %d out of range", pos);
    if (pos > m->slot_len[slot])
        return fail(MAK_ERANGE, "pos %d beyond cached length %d", pos, m->slot_len[slot]);
    ColState cs{};
    cs.token = token;
    cs.pos = pos;
    cs.slot = slot;
    cs.first_pos = pos;
    cs.first_col = 0;
    if ((rc = set_cols(m, &cs, 1, 0))) return rc;
    if ((rc = run_step(m, 1, 0, 1, m->at<int32_t>(m->L.out_tokens), pos + 1))) return rc;
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->at<float>(m->L.logits), (size_t)c.vocab * 4,
                               hipMemcpyDeviceToDevice, m->stream));
    if (next_token)
        HIP_TRY(hipMemcpyAsync(next_token, m->at<int32_t>(m->L.out_tokens), 4, hipMemcpyDeviceToHost,
                               m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    if ((rc = collect_timing(m))) return rc;
    m->slot_len[slot] = pos + 1;
    return MAK_OK;
}

int mak_decode_step_static(mak_model* m, int32_t slot, int32_t token, int32_t pos, float* d_logits,
                           int32_t* d_next_token)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (slot < 0 || slot >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    if (token < 0 || token >= c.vocab) return fail(MAK_ERANGE, "token %d out of range", token);
    if (pos < 0 || pos >= c.max_seq) return fail(MAK_ERANGE, "pos %d out of range", pos);
    if (pos > m->slot_len[slot])
        return fail(MAK_ERANGE, "pos %d beyond cached length %d", pos, m->slot_len[slot]);
    StepScratch sc{};
    if ((rc = static_step_scratch(m, &sc))) return rc;
    ColState cs{};
    cs.token = token;
    cs.pos = pos;
    cs.slot = slot;
    cs.first_pos = pos;
    cs.first_col = 0;
    // one launch per phase on the model's stream: no graph, no events
    m->untimed = true;
    rc = set_cols(m, &cs, 1, 0);
    if (!rc) {
        m->cur = m->stream;
        rc = record_step(m, 1, 0, 1, m->at<int32_t>(m->L.out_tokens), attn_mode(m, pos + 1), sc);
    }
    m->untimed = false;
    if (rc) return rc;
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->at<float>(m->L.logits), (size_t)c.vocab * 4, hipMemcpyDeviceToDevice,
                               m->stream));
    if (d_next_token)
        HIP_TRY(hipMemcpyAsync(d_next_token, m->at<int32_t>(m->L.out_tokens), 4, hipMemcpyDeviceToDevice,
                               m->stream));
    m->slot_len[slot] = pos + 1;
    return MAK_OK;
}

int mak_generate(mak_model* m, int32_t slot, const int32_t* prompt, int32_t n, int32_t max_new,
                 int32_t* out_tokens)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (!prompt || !out_tokens || n < 1 || max_new < 1)
        return fail(MAK_EINVAL, "NULL prompt/out_tokens, n < 1 or max_new < 1");
    if (slot < 0 || slot >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slot);
    if ((int64_t)n + max_new - 1 > c.max_seq)
        return fail(MAK_ERANGE, "n + max_new - 1 exceeds max_seq %d", c.max_seq);
    for (int i = 0; i < n; i++)
        if (prompt[i] < 0 || prompt[i] >= c.vocab) return fail(MAK_ERANGE, "token %d out of range", prompt[i]);
    m->slot_len[slot] = 0;
    if ((rc = prefill_chunks(m, slot, prompt, n, 0, true, 0))) return rc;
    int32_t* d_out = m->at<int32_t>(m->L.out_tokens);
    for (int s = 1; s < max_new; s++)   // the token at position n + s - 1
        if ((rc = run_step(m, 1, 0, 1, d_out, n + s))) return rc;
    HIP_TRY(hipMemcpyAsync(out_tokens, d_out, (size_t)max_new * 4, hipMemcpyDeviceToHost, m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    if ((rc = collect_timing(m))) return rc;
    m->slot_len[slot] = n + max_new - 1;
    return MAK_OK;
}

int mak_decode_batch(mak_model* m, int32_t B, const int32_t* slots, const int32_t* tokens,
                     const int32_t* positions, int32_t steps, int32_t* out_tokens, float* d_logits)
{
    int rc = check_model(m);
    if (rc) return rc;
    const mak_config& c = m->cfg;
    if (!slots || !tokens || !positions || !out_tokens || steps < 1)
        return fail(MAK_EINVAL, "NULL argument or steps < 1");
    if (B < 1 || B > c.max_batch || B > MAK_MAX_COLS)
        return fail(MAK_ERANGE, "batch %d out of range (max %d)", B, c.max_batch);
    if (steps > c.max_seq) return fail(MAK_ERANGE, "steps > max_seq");
    ColState cols[MAK_MAX_COLS] = {};
    for (int b = 0; b < B; b++) {
        if (slots[b] < 0 || slots[b] >= c.max_batch) return fail(MAK_ERANGE, "slot %d out of range", slots[b]);
        for (int b2 = 0; b2 < b; b2++)
            if (slots[b2] == slots[b]) return fail(MAK_EINVAL, "slot %d repeated in batch", slots[b]);
        if (tokens[b] < 0 || tokens[b] >= c.vocab) return fail(MAK_ERANGE, "token %d out of range", tokens[b]);
        if (positions[b] < 0 || positions[b] > m->slot_len[slots[b]])
            return fail(MAK_ERANGE, "position %d beyond cached length of slot %d", positions[b], slots[b]);
        if ((int64_t)positions[b] + steps > c.max_seq)
            return fail(MAK_ERANGE, "position + steps exceeds max_seq for slot %d", slots[b]);
        cols[b].token = tokens[b];
        cols[b].pos = positions[b];
        cols[b].slot = slots[b];
        cols[b].first_pos = positions[b];
        cols[b].first_col = b;
    }
    if ((rc = set_cols(m, cols, B, 0))) return rc;
    int32_t* d_out = m->at<int32_t>(m->L.out_tokens);
    int max_pos = 0;
    for (int b = 0; b < B; b++) max_pos = std::max(max_pos, (int)positions[b]);
    for (int s = 0; s < steps; s++)
        if ((rc = run_step(m, B, 0, B, d_out, max_pos + s + 1))) return rc;
    HIP_TRY(hipMemcpyAsync(out_tokens, d_out, (size_t)steps * B * 4, hipMemcpyDeviceToHost, m->stream));
    if (d_logits)
        HIP_TRY(hipMemcpyAsync(d_logits, m->at<float>(m->L.logits), (size_t)B * c.vocab * 4,
                               hipMemcpyDeviceToDevice, m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    if ((rc = collect_timing(m))) return rc;
    for (int b = 0; b < B; b++) m->slot_len[slots[b]] = positions[b] + steps;
    return MAK_OK;
}

}  // extern "C"
