/*
 * mak.h -- C ABI of libmak.so: greedy decoding of a llama-family decoder on
 * one MI355X (gfx950) GPU.
 *
 * The operations are the ones the "model-as-a-kernel" page lists in its
 * Usage and API sections: pack a model's weights into a device program, run
 * one decode step returning live fp32 logits, consume a prompt in chunks of
 * at most eight tokens, generate greedily, and decode several sequences as a
 * batch.  The model is a stack of RMSNorm decoder blocks with rotary
 * attention (GQA, optional per-head qk RMSNorm), a SwiGLU MLP, plain unscaled
 * rope, an LM head and greedy argmax (API section, "Supported" paragraph).
 * Sampling is greedy only ("Requirements and limits" section).
 *
 * Conventions shared by every entry point
 *   - Weights are bf16 bit patterns (uint16_t) in the [out, in] row-major
 *     layout of a linear layer.  Host arrays are read during mak_load only.
 *   - Positions are 0-based; prompt token i sits at position i.
 *   - "d_" pointers are device memory on the model's GPU; all work is queued
 *     on the stream given to mak_load and every call returns after that
 *     stream has finished the call's work, unless stated otherwise.
 *   - Return value: MAK_OK (0) or a negative MAK_E* code.  A failing call
 *     performs all validation before any device work, so it leaves the
 *     model and its KV cache unchanged.  mak_last_error() describes the last
 *     failure of the calling thread.
 *   - A model is not thread-safe; calls on one model must be serialised.
 *
 * Arithmetic: bf16 storage, fp64 accumulation of every dot product and fp64
 * evaluation of exp/sqrt, with bf16 rounding at the op boundaries of eager
 * bf16 execution ("model-as-a-kernel", Method section: every operation rounds
 * as an eager bf16 run does; reductions use fixed trees and no floating-point
 * atomics, so the output is bitwise deterministic).
 */
#ifndef MAK_H
#define MAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAK_OK 0
#define MAK_EINVAL (-1)   /* null pointer, shape mismatch or unsupported shape      */
#define MAK_ERANGE (-2)   /* token, position, slot, batch or length out of range    */
#define MAK_ENOMEM (-3)   /* arena smaller than mak_plan's figure                   */
#define MAK_EDEVICE (-4)  /* HIP runtime error (message kept for mak_last_error)     */

#define MAK_MAX_BATCH 16    /* columns of one decode batch                          */
#define MAK_PREFILL_CHUNK 16 /* prompts are consumed in chunks of at most 16 tokens */

/* Weight formats of the per-layer linear matrices (q, k, v, o, gate, up,
 * down).  The embedding, the LM head and the norm weights stay bf16.
 *   MAK_WEIGHTS_BF16   bf16, as given.
 *   MAK_WEIGHTS_MXFP4  4-bit: mak_load quantizes each matrix with
 *                      mak_quantize_mxfp4 and decoding streams the codes
 *                      ("model-as-a-kernel", API section, "Supported"
 *                      paragraph: 4-bit weights; the page's nf4 format is not
 *                      specified there, so the 4-bit format is OCP MXFP4). */
#define MAK_WEIGHTS_BF16 0
#define MAK_WEIGHTS_MXFP4 1

/* Model shape.  head_dim a power of two in [16, 128]; hidden, intermediate and
 * n_q_heads*head_dim multiples of 8 (of 32 with MAK_WEIGHTS_MXFP4);
 * n_q_heads a multiple of n_kv_heads; 1 <= max_batch <= MAK_MAX_BATCH;
 * max_seq >= 1. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
    float rms_eps, rope_theta;
    int32_t tie_embeddings; /* 1: the LM head is the embedding matrix           */
    int32_t qk_norm;        /* 1: per-head RMSNorm of q and k before rope        */
    int32_t max_seq;        /* positions per KV slot                             */
    int32_t max_batch;      /* KV slots = sequences decodable at once            */
    int32_t weight_format;  /* MAK_WEIGHTS_BF16 (0) or MAK_WEIGHTS_MXFP4         */
} mak_config;

/* One decoder layer's weights (host bf16 bits). q_norm/k_norm are [head_dim]
 * and must be NULL unless cfg.qk_norm. */
typedef struct {
    const uint16_t *attn_norm; /* [hidden]                          */
    const uint16_t *wq;        /* [n_q_heads*head_dim, hidden]      */
    const uint16_t *wk;        /* [n_kv_heads*head_dim, hidden]     */
    const uint16_t *wv;        /* [n_kv_heads*head_dim, hidden]     */
    const uint16_t *wo;        /* [hidden, n_q_heads*head_dim]      */
    const uint16_t *q_norm;    /* [head_dim] or NULL                */
    const uint16_t *k_norm;    /* [head_dim] or NULL                */
    const uint16_t *mlp_norm;  /* [hidden]                          */
    const uint16_t *w_gate;    /* [intermediate, hidden]            */
    const uint16_t *w_up;      /* [intermediate, hidden]            */
    const uint16_t *w_down;    /* [hidden, intermediate]            */
} mak_layer_weights;

typedef struct {
    const uint16_t *embed;            /* [vocab, hidden]                    */
    const uint16_t *lm_head;          /* [vocab, hidden], NULL when tied     */
    const uint16_t *final_norm;       /* [hidden]                           */
    const mak_layer_weights *layers;  /* [n_layers]                         */
} mak_weights;

typedef struct mak_model mak_model; /* opaque */

/* 4-bit quantization (host only, no device work) of a [rows, k] bf16 matrix
 * into OCP MXFP4 (Microscaling Formats specification v1.0), the format of
 * MAK_WEIGHTS_MXFP4.  Each block of 32 consecutive weights of a row shares
 * one scale 2^e with e = floor(log2(max |w| of the block)) - 2, clamped to
 * [-127, 127] (-127 for an all-zero block), written to scales[row][k/32] as
 * the E8M0 byte e + 127.  Each weight becomes the FP4 E2M1 code (sign, 2
 * exponent bits, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) of
 * w / 2^e rounded to nearest, ties to the even code, magnitudes above 6
 * saturating to 6, zero with a clear sign bit; codes[row][k/2] holds two per
 * byte, the lower-indexed weight in the low nibble.  Every dequantized value
 * code * 2^e is exactly a bf16 value.  k must be a positive multiple of 32 and
 * every weight finite (MAK_EINVAL otherwise, nothing written). */
int mak_quantize_mxfp4(const uint16_t *w, int64_t rows, int32_t k, uint8_t *codes, uint8_t *scales);

/* Device bytes mak_load needs for this shape: packed weights, rope tables,
 * max_batch KV slots of max_seq positions, and scratch.  No device work. */
int mak_plan(const mak_config *cfg, size_t *arena_bytes);

/* Pack the weights into the caller's device arena and build the phase
 * program ("model-as-a-kernel", Method section: model load packs the weights
 * and compiles the architecture into a program).  d_arena must stay valid
 * until mak_free; the model owns its contents.  hip_stream is a hipStream_t
 * (NULL = the default stream).  Synchronises the stream before returning,
 * so the host weight arrays may be freed afterwards. */
int mak_load(const mak_config *cfg, const mak_weights *w, void *d_arena, size_t arena_bytes,
             void *hip_stream, mak_model **out);

/* Consume n prompt tokens of sequence `slot` at positions start_pos ..
 * start_pos+n-1, in chunks of at most MAK_PREFILL_CHUNK tokens, or the size
 * set by mak_set_prefill_chunk ("model-as-a-kernel", Usage: chunked prompt
 * consumption).  start_pos may not exceed the slot's
 * cached length.  If d_logits is not NULL it receives the fp32 logits [vocab]
 * of the last prompt token.  n >= 1. */
int mak_prefill(mak_model *m, int32_t slot, const int32_t *ids, int32_t n, int32_t start_pos,
                float *d_logits);

/* One decode step ("model-as-a-kernel", API: decode_step returns live fp32
 * logits [V]): token at position pos of `slot` (pos <= cached length; a
 * smaller pos rewinds).  d_logits (may be NULL) receives fp32 logits
 * [vocab]; next_token (host, may be NULL) receives the greedy argmax (lowest
 * index among equal maxima). */
int mak_decode_step(mak_model *m, int32_t slot, int32_t token, int32_t pos, float *d_logits,
                    int32_t *next_token);

/* mak_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The call allocates nothing (no hipMalloc/hipFree, no graph
 * instantiation, no events): it launches the step's phases one by one on the
 * model's stream and takes the step's scratch (the LM head's argmax partials
 * and the split-KV attention's scores, chunk maxima and partial outputs)
 * from a static device array of 4 MiB that each GPU holds until the process
 * ends, instead of the arena.  d_logits (device, [vocab] fp32, may be NULL)
 * and d_next_token (device, one int32, may be NULL) receive the results by
 * device-to-device copies.  The call returns once the work is queued; it
 * does not synchronise the stream.  Results are bitwise those of
 * mak_decode_step.  Returns MAK_EINVAL if the model's shape needs more step
 * scratch than the static array holds (n_q_heads * max_seq * 4 +
 * n_q_heads * ceil(max_seq/128) * (head_dim * 8 + 4) + 128 KiB, 256-byte
 * aligned parts).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (two models, or two streams) race and must be
 * serialised by the caller. */
int mak_decode_step_static(mak_model *m, int32_t slot, int32_t token, int32_t pos, float *d_logits,
                           int32_t *d_next_token);

/* Greedy generation ("model-as-a-kernel", Usage: generate): reset `slot`,
 * prefill the n-token prompt from position 0, then emit exactly max_new tokens
 * into out_tokens (host, [max_new]); the first is the argmax of the prefill
 * logits and each later token is fed back on the device without a host
 * round trip.  Requires n + max_new - 1 <= max_seq. */
int mak_generate(mak_model *m, int32_t slot, const int32_t *prompt, int32_t n, int32_t max_new,
                 int32_t *out_tokens);

/* Batched greedy decode ("model-as-a-kernel", API: decode_batch(tokens,
 * positions, steps)): B sequences (distinct slots) advance together for
 * `steps` steps; step 0 consumes tokens[b] at positions[b], each later step
 * consumes the previous step's argmax at the next position.  out_tokens
 * (host, [steps][B]) receives every argmax; d_logits (may be NULL) receives
 * the fp32 logits [B][vocab] of the last step.  Each sequence's results do
 * not depend on the others in the batch. */
int mak_decode_batch(mak_model *m, int32_t B, const int32_t *slots, const int32_t *tokens,
                     const int32_t *positions, int32_t steps, int32_t *out_tokens,
                     float *d_logits);

/* Copy the cached K (after qk-norm and rope) and V of `layer`, `slot`,
 * positions [pos0, pos0+n) into host arrays k_out and v_out, each
 * [n_kv_heads][n][head_dim] bf16 bits ("model-as-a-kernel", Correctness
 * section: the layer KV cache is compared bitwise against the reference).
 * Requires pos0 + n <= the slot's cached length. */
int mak_read_kv(const mak_model *m, int32_t layer, int32_t slot, int32_t pos0, int32_t n,
                uint16_t *k_out, uint16_t *v_out);

/* Executor.  MAK_EXEC_GRAPH (the default) replays one captured hipGraph of
 * the step's phase launches per step shape; MAK_EXEC_PHASED launches every
 * phase as its own kernel from the host -- the page's phase-per-launch mode
 * ("model-as-a-kernel", API: decode_step(..., phased=True); Method: bitwise
 * identical to the fused mode). */
#define MAK_EXEC_GRAPH 0
#define MAK_EXEC_PHASED 1
int mak_set_executor(mak_model *m, int executor);

/* Attention work split ("model-as-a-kernel", Method section: split-KV with
 * a deterministic combine).  While a step's largest context pos + 1 is at
 * most `above` (default 49152 / head_dim: 384 at head_dim 128, 768 at 64,
 * where the split form starts to pay; for prompt chunks 131072 / head_dim,
 * where their blockwise form does; a call sets both to `above`), each query
 * head's attention runs in one workgroup over all positions; beyond it, or
 * past the single-pass capacity of 4096 positions, attention runs split-KV:
 * scores and a maximum per chunk of 128 positions, then the exact global
 * softmax and P.V per chunk, then the chunk sums in chunk order.  Both forms give bitwise-identical results;
 * 0 always splits.  Returns MAK_EINVAL for a negative threshold. */
int mak_set_attention_split(mak_model *m, int32_t above);

/* Prompt-chunk attention past the split threshold.  A prefill step's
 * columns are consecutive positions of one sequence, so with on = 1 (the
 * default) its split-KV attention runs blockwise: one workgroup per (query
 * head, chunk of 128 positions) reads that chunk's K rows, then its V rows,
 * once for all columns of the step and applies each column's causal limit;
 * each (column, head) softmax row is computed once ("CuTeDSL at Perplexity",
 * section on prefill and decode specialization: a prefill variant with its
 * own grid and block assignment).  With
 * on = 0 each column runs the per-column split-KV kernels.  Both give
 * bitwise-identical results; decode and batched steps are unaffected.
 * Returns MAK_EINVAL unless on is 0 or 1. */
int mak_set_block_attention(mak_model *m, int32_t on);

/* Prompt tokens per prefill step, 1..16 (default MAK_PREFILL_CHUNK = 16).  The
 * "model-as-a-kernel" page consumes prompts in chunks of up to eight tokens,
 * bitwise identical to token-by-token consumption (Method section).  Larger
 * chunks stream each layer's weights once for more tokens and stay bitwise
 * identical, since every dot product is exact before its single rounding.
 * Steps of 9..16 tokens run on the fp64 matrix cores and take about as long
 * as a step of 8 on the vector units, hence the default.
 * Returns MAK_EINVAL outside 1..16. */
int mak_set_prefill_chunk(mak_model *m, int32_t tokens);

/* Per-phase timing ("model-as-a-kernel", API: decode_step_timed runs the
 * phases one launch each and reports per-phase milliseconds).  While
 * enabled, the phases run one launch each and every kernel carries a pair of
 * hipEvents on the model's stream that HIP stamps at the kernel's own start
 * and end; the duration is added to the total of its phase kind.  Enabling
 * resets the totals.  mak_phase_times fills ms[MAK_PHASE_COUNT] and
 * launches[MAK_PHASE_COUNT] (either may be NULL). */
#define MAK_PHASE_QKV 0    /* RMSNorm + Q/K/V GEMV                          */
#define MAK_PHASE_ATTN 1   /* qk-norm, rope, KV append, attention           */
#define MAK_PHASE_O 2      /* O GEMV + residual                             */
#define MAK_PHASE_GATEUP 3 /* RMSNorm + gate/up GEMV + SwiGLU               */
#define MAK_PHASE_DOWN 4   /* down GEMV + residual                          */
#define MAK_PHASE_LMHEAD 5 /* final RMSNorm + LM head + argmax + feedback   */
#define MAK_PHASE_CTL 6    /* control-block updates                         */
#define MAK_PHASE_COUNT 7
int mak_set_phase_timing(mak_model *m, int enable);
int mak_phase_times(const mak_model *m, double *ms, int64_t *launches);

/* Number of sequences one batch may hold (the model's KV slots). */
int mak_batch_max(const mak_model *m);

/* Cached length (next free position) of a slot, or a negative error code. */
int mak_slot_length(const mak_model *m, int32_t slot);

/* Release the model's host-side state (the arena stays the caller's). */
void mak_free(mak_model *m);

/* Message of the calling thread's last failure ("" if none). */
const char *mak_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MAK_H */
