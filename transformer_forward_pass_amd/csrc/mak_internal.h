// mak_internal.h -- plain-old-data shared by the host runtime and the gfx950
// kernels: the packed-GEMV geometry, the per-column decode state and the
// phase descriptors of the device program.
#pragma once
#include <stdint.h>

#define MAK_WAVE 64
#define MAK_BLOCK 256               // threads per workgroup (4 waves)
#define MAK_GBLOCK 512              // threads per workgroup of the batch-1 GEMV (8 waves, one workgroup per CU)
#define MAK_NBLOCK 512              // threads per workgroup of the multi-column GEMV (8 waves)
#define MAK_MAX_COLS 16             // columns per step (batch rows; prefill chunks use <= 8)
#define MAK_ATTN_CHUNK 128          // positions per chunk of the split-KV attention

// ---------------------------------------------------------------------------
// Packed weight geometry.
//
// A [N, K] bf16 matrix (K a multiple of 8) is cut into 16-byte chunks of 8
// consecutive inputs, C = K/8 chunks per row.  `lr` = gcd(C, 64) lanes of a
// wave share one row; a wave therefore covers g = 64/lr row groups, each of
// `r` rows.  One wave's tile is g*r rows.  Inside a tile, the 16-byte slots
// are stored in the order [j][ri][lane] with j = chunk iteration (C/lr of
// them), ri = row within the group and lane = group*lr + s, where slot
// (j, ri, lane) holds chunk j*lr + s of row tile*g*r + group*r + ri.
// Every wave load is therefore 64 lanes x 16 B = 1 KiB contiguous.  Rows past
// N are zero padding.
//
// 4-bit matrices (fmt MAK_FMT_MXFP4, OCP MXFP4: K a multiple of 32): a 16-byte
// chunk holds 32 consecutive inputs' E2M1 codes (two per byte, the lower
// index in the low nibble), which are exactly one 32-weight block sharing one
// E8M0 scale; C = K/32 chunks per row and the same slot order.  The scale
// bytes follow the codes at byte offset scale_off, one per slot, in slot
// order, so scale(slot) = base[scale_off + slot].
// ---------------------------------------------------------------------------
#define MAK_FMT_BF16 0
#define MAK_FMT_MXFP4 1
#define MAK_MX_BLOCK 32

struct PackGeom {
    int32_t n_rows;    // N
    int32_t k;         // K
    int32_t lr_log2;   // log2(lanes per row)
    int32_t r;         // rows per lane group (1, 2 or 4)
    int32_t n_tiles;   // ceil(N / (g*r))
    int32_t fmt;       // MAK_FMT_BF16 or MAK_FMT_MXFP4
    int64_t bytes;     // packed size in bytes (bf16: n_tiles*g*r*K*2; 4-bit: codes + scales)
    int64_t scale_off; // 4-bit: byte offset of the scale bytes (= n_tiles*g*r*K/2)
};

// State of one column (one token being processed) of a step.
struct ColState {
    int32_t token;      // input token id
    int32_t pos;        // position of this token in its sequence
    int32_t slot;       // KV slot of the sequence
    int32_t first_pos;  // position of the first column of this sequence in the step
    int32_t first_col;  // index of that column
    int32_t pad_[3];
};

// Device control block (lives in the arena).
struct Ctl {
    ColState cols[MAK_MAX_COLS];
    int32_t ncols;       // columns in the current step
    int32_t lm_begin;    // first column whose logits are computed
    int32_t lm_count;    // number of such columns
    int32_t step;        // tokens emitted so far by the current call
    uint32_t ticket;     // arrival counter of the LM-head argmax reduction
    int32_t err;         // device-side error flag
    int32_t pad_[2];
};

enum InKind : int32_t {
    IN_RAW = 0,          // bf16 vectors in[col*in_ld + k]
    IN_NORM = 1,         // RMSNorm(x[col]) with norm_w
    IN_GATHER_NORM = 2,  // RMSNorm(embedding row of cols[col].token); block 0 also stores x
};

enum EpiKind : int32_t {
    EPI_STORE = 0,       // out[col*out_ld + row] = bf16(acc)
    EPI_RESIDUAL = 1,    // x[col*out_ld + row] = bf16(x + bf16(acc))
    EPI_SWIGLU = 2,      // rows (2i, 2i+1) = (gate_i, up_i) -> out[col*out_ld + i]
    EPI_LOGITS = 3,      // logits[col*logits_ld + row] = fp32(acc); argmax + feedback
};

struct GemvPhase {
    const void* w;            // packed weights (PackGeom layout)
    PackGeom geo;
    int32_t in_kind;
    int32_t epi;
    int32_t ncols;            // active columns
    int32_t col0;             // first column (of Ctl.cols) this phase works on
    const uint16_t* in;       // IN_RAW / IN_NORM source, [col][in_ld]
    int32_t in_ld;
    float eps;
    const uint16_t* norm_w;   // [K] for IN_NORM / IN_GATHER_NORM
    const void* embed;        // packed embedding (IN_GATHER_NORM)
    PackGeom embed_geo;
    uint16_t* x_store;        // IN_GATHER_NORM: block 0 writes gathered rows here
    int32_t x_ld;
    int32_t out_ld;
    uint16_t* out;            // EPI_STORE / EPI_RESIDUAL / EPI_SWIGLU destination
    float* logits;            // EPI_LOGITS destination [col][logits_ld]
    int32_t logits_ld;
    int32_t n_blocks;         // grid size (EPI_LOGITS ticket count)
    int32_t rr;               // multi-column kernel: rows per lane (a multiple of geo.r)
    int32_t jw;               // multi-column kernel: waves sharing one tile group (split of K)
    int32_t threads;          // workgroup size of the launch
    int32_t multi;            // 1: the multi-column kernel (k_gemvn) runs the launch
    int32_t ks;               // batch-1 kernel: waves per tile (1, or 2 = chunks split over a wave pair)
    float* part_val;          // EPI_LOGITS per-block partial maxima [n_blocks][MAK_MAX_COLS]
    int32_t* part_idx;
    int32_t* out_tokens;      // EPI_LOGITS: emitted tokens [step][lm_count] (device)
    Ctl* ctl;
};

struct AttnPhase {
    const uint16_t* qkv;      // raw projections [col][qkv_ld]: q | k | v
    int32_t qkv_ld;
    uint16_t* kc;             // this layer's K cache  [slot][Hkv][max_seq][d]
    uint16_t* vc;             // this layer's V cache
    const uint16_t* cos_t;    // rope tables [max_seq][d/2] (bf16)
    const uint16_t* sin_t;
    const uint16_t* q_norm;   // [d] or null
    const uint16_t* k_norm;
    uint16_t* o;              // attention output [col][Hq*d]
    Ctl* ctl;
    int32_t ncols;
    int32_t n_q_heads, n_kv_heads, head_dim, max_seq;
    float eps;
    float scale;              // fp32(1/sqrt(head_dim))
    // split-KV attention (long contexts) scratch
    float* sc;                // scores [col][Hq][max_seq]
    float* cmax;              // chunk maxima [col][Hq][n_chunks]
    double* opart;            // partial outputs [col][Hq][n_chunks][head_dim]
    int32_t n_chunks;         // ceil(max_seq / MAK_ATTN_CHUNK)
    int32_t s_cap;            // single-pass kernel: most positions its LDS score row holds
};

// ---------------------------------------------------------------------------
// Launch-configuration check, applied to every launch before it is issued
// and to every kernel node of a captured step graph: a grid of at least one
// workgroup in each dimension, a workgroup no larger than the kernel's
// compiled bound (its __launch_bounds__), dynamic LDS within the kernel's
// dynamic-LDS ceiling, and static plus dynamic LDS within the device's LDS
// per workgroup (160 KiB on gfx950).  Returns 0 when the launch is valid,
// else the number of the first violated rule (1 grid, 2 workgroup size,
// 3 dynamic-LDS ceiling, 4 total LDS).
// ---------------------------------------------------------------------------
static inline int mak_launch_check(uint32_t gx, uint32_t gy, uint32_t gz, uint32_t bx, uint32_t by, uint32_t bz,
                                   int64_t max_threads, int64_t static_lds, int64_t dyn_lds,
                                   int64_t max_dyn_lds, int64_t lds_per_block)
{
    if (gx < 1 || gy < 1 || gz < 1) return 1;
    const int64_t threads = (int64_t)bx * by * bz;
    if (threads < 1 || threads > max_threads) return 2;
    if (dyn_lds < 0 || dyn_lds > max_dyn_lds) return 3;
    if (static_lds + dyn_lds > lds_per_block) return 4;
    return 0;
}
