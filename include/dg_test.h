/*
 * dg_test.h - entry points that run parts of the denoising step on given
 * inputs, so each stage can be compared with an independent implementation.
 * They use the same kernels as dg_denoise_step; conventions as in dg.h.
 */
#ifndef DG_TEST_H
#define DG_TEST_H

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Byte offsets of the buffers inside the workspace (for inspection).
 * rows = max_rows; E = n_experts; k = top_k.
 *   h        fp32 [rows][d]          residual stream
 *   u        bf16 [rows][d]          RMSNorm output (GEMM operand)
 *   q        bf16 [rows][Hq][dh]     rotated queries
 *   attn_o   bf16 [rows][Hq*dh]      attention output
 *   z        fp32 [rows][E]          router logits
 *   idx      int32 [rows][k]         selected experts (descending logit)
 *   w        fp32 [rows][k]          softmax over the selected logits
 *   wslot    int32 [rows*k]          t*k + j of each expert slot (index into w)
 *   cnt      int32 [E]; off int32 [E+1]
 *   items    int32 words             expert work list: per group (0 = shared
 *                                    expert, 1+e = routed expert e) the item
 *                                    and row-chunk offsets, the queue head,
 *                                    the spin-timeout counter (word
 *                                    DG_ITEMS_SPIN_TIMEOUTS) and per-chunk
 *                                    completion counters
 *   perm     int32 [rows*k]          token of each expert slot
 *   slot     int32 [rows][k]         slot of each (token, choice)
 *   hid      bf16 [rows*k][F]        routed expert SwiGLU activations
 *   hid_s    bf16 [rows][Fs]         shared expert SwiGLU activations
 *   y        bf16 [rows*k][d]        routed expert outputs (weighted), then
 *            fp32 [rows][d]          the shared expert's outputs
 *   lm_gpart float4 [rows][V/256]    sampled-candidate partials per
 *                                    vocabulary tile (key, id, logit, 0)
 *   stats    dg_row_stats [rows]     per-row LM-head statistics
 *   ss       fp32 [d/64][rows]       partial sums of squares of h per
 *                                    64-column tile (output projection)
 *   zpart    fp32 [8][rows16][E]     router logits per part of d: eight
 *                                    parts up to 512 rows, four above
 *                                    (rows16 = rows rounded up to 16)
 *   sync     int32 [256]             router row-block arrival counters
 *   prev     int32 [max_requests][canvas]  argmax of each slot's last
 *                                    denoising step */
/* Word of the items buffer that counts expert-kernel waits which ran out of
 * their poll budget instead of seeing their input published. A correct run
 * leaves it unchanged; the library never resets it. */
#define DG_ITEMS_SPIN_TIMEOUTS 409

/* Running routing statistics in the items buffer (uint64 at these word
 * indices, never reset by the library): the number of experts that received
 * at least one row, summed over permutation calls, and the number of calls.
 * Their ratio over an interval is the mean number of experts whose weights a
 * layer had to stream. */
#define DG_ITEMS_TOUCHED_TOTAL 410
#define DG_ITEMS_PERMUTE_CALLS 412

/* Self-conditioning buffers (size 0 without it; F = d_selfcond):
 *   sc_p     bf16 [rows][V]          exp(L - m) per 64-column quarter, then
 *                                    normalised in place to softmax(L)
 *   sc_qpart float2 [rows][V/64]     (m, sum of exp) per quarter
 *   sc_part  fp32 [splits][rows][d]  partial sums of the contraction with E
 *   sc_e     bf16 [rows][d]          expected embedding e = p E
 *   sc_g, sc_u fp32 [rows][F]        gate and up products
 *   sc_hid   bf16 [rows][F]          SwiGLU activations
 *   sc_out   fp32 [rows][d]          the signal of the step's rows
 *   sc_state fp32 [max_requests][canvas][d]  each slot's signal for its
 *                                    next step */
typedef struct dg_ws_layout {
  size_t h, u, q, attn_o, attn_part, attn_ml, rope, z, idx, w, wslot, cnt, off, items, perm,
      slot, hid, hid_s, y, lm_part, lm_gpart, stats, ids, ss, zpart, sync, prev, sc_p, sc_qpart, sc_part, sc_e,
      sc_g, sc_u, sc_hid, sc_out, sc_state, total;
} dg_ws_layout;

dg_status dg_workspace_layout(const dg_config *cfg, dg_ws_layout *out);

/* One layer over n rows of request slot req at positions len..len+n-1
 * (len = dg_cache_len). d_h: device fp32 [n][d], input and output. causal=0:
 * denoising attention (no mask inside the rows); causal=1: encoder attention.
 * K/V rows are written to cache rows [len, len+n); the length is unchanged.
 * Intermediates stay in the workspace (dg_workspace_layout). */
dg_status dg_test_layer(dg_ctx *ctx, void *stream, int32_t req, int32_t layer, float *d_h,
                        int32_t n, int32_t causal);

/* Router top-k and permutation from given router logits d_z fp32 [rows][E]
 * (device). Outputs (device, any may be NULL): idx [rows][k], w [rows][k],
 * cnt [E], off [E+1], perm [rows*k], slot [rows][k]. */
dg_status dg_test_route(dg_ctx *ctx, void *stream, const float *d_z, int32_t rows,
                        int32_t *d_idx, float *d_w, int32_t *d_cnt, int32_t *d_off,
                        int32_t *d_perm, int32_t *d_slot);

/* Final RMSNorm, LM head statistics and sampler from a given residual stream
 * d_h fp32 [n_req*canvas][d] (device), with the same arguments and effects on
 * canvas / committed / stats as dg_denoise_step. */
dg_status dg_test_head(dg_ctx *ctx, void *stream, const dg_step_args *a, const float *d_h);

/* The denoising step of dg_denoise_step, same arguments and effects, with
 * the residual stream copied out after the embedding and after every layer:
 * d_h_layers is device fp32 [n_layers + 1][n_req * canvas][d_model] (entry 0
 * the embedding rows, entry l + 1 the rows after layer l), and, when
 * d_idx_layers is not NULL, each layer's expert choices, device int32
 * [n_layers][n_req * canvas][top_k] (descending router logit). The copies
 * are extra work on the stream; the kernels and their order are those of
 * dg_denoise_step (explainer §3.2: the bidirectional decoder pass over the
 * canvas). DG_EINVAL if d_h_layers is NULL. */
dg_status dg_test_forward(dg_ctx *ctx, void *stream, const dg_step_args *a, float *d_h_layers,
                          int32_t *d_idx_layers);

/* The confidence sampler of dg_denoise_step (explainer §3.3) fed given
 * per-position statistics instead of the LM head's: d_in is device
 * dg_row_stats [n_req * canvas], of which max_logit, log_z, held_logit,
 * argmax, entropy, sample and sample_logit are read (as the LM head would
 * have written them). Canvas, committed mask, d_stats (conf, accepted) and
 * d_stop are updated exactly as by dg_denoise_step with the same arguments,
 * including the per-slot previous-argmax state of adaptive stopping. */
dg_status dg_test_sample(dg_ctx *ctx, void *stream, const dg_step_args *a, const dg_row_stats *d_in);

/* Canvas attention alone (explainer §3.2; aiboss88.com, "hybrid attention"):
 * the n query rows d_q (device bf16 [n][n_q_heads][head_dim], already
 * rotated) of request slot req at positions len..len+n-1 (len =
 * dg_cache_len) attend, per query head h with kv head h*Hkv/Hq, to the
 * cache rows [0, len + n) of layer `layer` (K rotated; V in the cache's
 * block order; rows [len, len+n) are the block's own rows, written by the
 * caller). causal = 0: no mask; causal = 1: query i sees keys < len + i + 1.
 * Scale 1/sqrt(head_dim). d_o: device bf16 [n][n_q_heads * head_dim].
 * Needs n <= max_rows and len + n <= max_ctx. */
dg_status dg_test_attention(dg_ctx *ctx, void *stream, int32_t req, int32_t layer, const void *d_q, int32_t n,
                            int32_t causal, void *d_o);

/* Per-stage timing. While enabled, every launch of a stage is bracketed by a
 * pair of hipEvents recorded on the call's stream; dg_timing_read waits for
 * the last recorded event, adds the elapsed times into ms[stage] and
 * launches[stage] (arrays of n_stages >= DG_STAGE_COUNT entries, overwritten)
 * and recycles the events. Stages: */
enum {
  DG_STAGE_EMBED = 0,   /* embedding gather (+ RoPE table) */
  DG_STAGE_NORM,        /* RMSNorm */
  DG_STAGE_QKV,         /* QKV projection + RoPE + KV write */
  DG_STAGE_ATTN,        /* canvas attention (split keys + merge) */
  DG_STAGE_OPROJ,       /* output projection + residual */
  DG_STAGE_ROUTER,      /* router logits + top-k + softmax (fused) */
  DG_STAGE_TOPK,        /* top-k from given logits (test entry point only) */
  DG_STAGE_PERMUTE,     /* token -> expert permutation */
  DG_STAGE_EXPERTS,     /* grouped experts: gate/up + SwiGLU, then down (routed + shared) */
  DG_STAGE_COMBINE,     /* weighted combine + residual */
  DG_STAGE_LMHEAD,      /* LM head with fused vocabulary statistics */
  DG_STAGE_MERGE,       /* vocabulary statistics merge */
  DG_STAGE_SAMPLER,     /* confidence sampler / initial canvas */
  DG_STAGE_SELFCOND,    /* self-conditioning signal for the next step */
  DG_STAGE_COUNT
};
dg_status dg_timing_enable(dg_ctx *ctx, int32_t enable);
dg_status dg_timing_read(dg_ctx *ctx, double *ms, int32_t *launches, int32_t n_stages);

#ifdef __cplusplus
}
#endif
#endif /* DG_TEST_H */
