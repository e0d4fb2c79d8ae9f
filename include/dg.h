/*
 * dg.h - one block-diffusion denoising step on MI355X (gfx950), C ABI.
 *
 * The model is the one the pages describe (codemajin.net DiffusionGemma
 * explainer §2.1-§3.3; aiboss88.com product page, "technical principles"):
 * a weight-shared MoE transformer used two ways.
 *   - As a causal encoder it turns the prompt, and every finished 256-token
 *     block, into K/V rows appended to a per-request KV cache (dg_prefill,
 *     dg_commit_block). Committed rows are never rewritten (explainer §3.2).
 *   - As a bidirectional decoder it denoises the current canvas: every canvas
 *     position attends to the cached prefix and to every other canvas
 *     position, the LM head gives a distribution per position, and the
 *     confidence sampler keeps the most confident tokens and re-noises the
 *     rest to uniform random ids (dg_denoise_step; explainer §3.3, aibars.net
 *     news item, "Uniform State Diffusion").
 *
 * Conventions (all calls):
 *   - Plain C types only. Device pointers are named d_*; everything else is
 *     host memory. A stream is a hipStream_t passed as void* (NULL = the
 *     null stream).
 *   - The caller owns all device memory: weights, KV cache, workspace, canvas,
 *     masks. The library never allocates device memory; it keeps the raw
 *     pointers given to dg_create, which must stay valid until dg_destroy.
 *     The dg_ctx itself is host memory owned by the library.
 *   - Weights are bf16 in the [out][in] convention (y = x W^T). Norm gains
 *     and the router are row-major; the streamed matrices (projections,
 *     experts, and the embedding, which is also the LM head) are in the
 *     fragment-major layout made by dg_pack_weight.
 *   - Every call validates its arguments and the cache capacity before it
 *     enqueues anything; on DG_EINVAL / DG_ECAPACITY nothing has been
 *     launched and no state changed. Work is enqueued asynchronously on the
 *     given stream. A HIP launch error returns DG_EHIP and makes the context
 *     sticky: every later call returns DG_ESTATE until dg_destroy.
 *     dg_last_error() gives a message. No C++ exception crosses the ABI.
 *   - One context per stream at a time; not thread-safe.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_EINVAL = -1,     /* bad argument or unsupported shape */
  DG_ECAPACITY = -2,  /* KV cache or workspace too small for the call */
  DG_EHIP = -3,       /* a HIP call failed; the context is now sticky */
  DG_ESTATE = -4      /* the context is sticky after an earlier failure */
} dg_status;

/* Model shape and sampler constants.
 * Supported shapes: head_dim in {64, 128}; d_model a multiple of 256, at most
 * 4096;
 * n_q_heads a multiple of n_kv_heads; (n_q_heads*head_dim) and
 * (n_kv_heads*head_dim) multiples of 128; n_experts <= 128 and a multiple
 * of 8; top_k <= 8; d_expert and d_shared multiples of 64; vocab a multiple
 * of 256; canvas a multiple of 16, at most 1024; canvas <= max_rows <=
 * 32*canvas (up to 32 requests of one block each per call).
 * tau_first / tau_last: temperature at the first / last step, falling
 * linearly (explainer §3.3: 0.8 -> 0.4). */
typedef struct dg_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, d_expert, d_shared, vocab;
  int32_t canvas;        /* C: tokens per block (explainer §3.2: 256) */
  int32_t max_ctx;       /* KV rows per request and layer (multiple of 32) */
  int32_t max_requests;  /* number of request slots in the KV cache */
  int32_t max_rows;      /* largest number of rows one call processes */
  float rms_eps, rope_theta, tau_first, tau_last;
  int32_t expert_format; /* dg_weight_format of the expert matrices (0 = bf16) */
  int32_t d_selfcond;    /* width of the self-conditioning feed-forward layer
                            (a multiple of 64); 0 = no self-conditioning */
  int32_t lmhead_format; /* dg_weight_format of the LM head's copy of the
                            embedding (0 = bf16: the embedding itself) */
} dg_config;

/* Storage of the routed and shared expert matrices (w_gate, w_up, w_down,
 * ws_gate, ws_up, ws_down):
 *   DG_WEIGHTS_BF16  bf16, fragment-major (dg_pack_weight);
 *   DG_WEIGHTS_FP8   OCP E4M3 codes with one power-of-two scale per weight
 *                    row, as made by dg_quantize_fp8; the s_* / ss_* fields
 *                    of dg_layer_weights point at the scales. The
 *                    explainer's step timings (§5.2) are measured at FP8
 *                    precision; the pages do not give the format. */
typedef enum { DG_WEIGHTS_BF16 = 0, DG_WEIGHTS_FP8 = 1 } dg_weight_format;

/* One layer's weights (device, bf16):
 *   attn_norm [d]        w_qkv [(Hq+2Hkv)*dh][d]   (q heads, then k, then v)
 *   w_o [d][Hq*dh]       moe_norm [d]              w_router [E][d]
 *   w_gate, w_up [E][F][d]   w_down [E][d][F]
 *   ws_gate, ws_up [Fs][d]   ws_down [d][Fs]       (shared expert)
 * attn_norm, moe_norm and w_router are row-major. w_qkv, w_o, w_gate, w_up,
 * w_down, ws_gate, ws_up and ws_down are fragment-major: the shapes above,
 * each converted with dg_pack_weight (an expert bank [E][N][K] is converted
 * as one [E*N][K] matrix). */
typedef struct dg_layer_weights {
  const void *attn_norm, *w_qkv, *w_o, *moe_norm, *w_router;
  const void *w_gate, *w_up, *w_down, *ws_gate, *ws_up, *ws_down;
  /* FP8 experts only (NULL otherwise): device fp32 row scales of
   * w_gate and w_up [E*F], w_down [E*d], ws_gate and ws_up [Fs], ws_down [d] */
  const float *s_gate, *s_up, *s_down, *ss_gate, *ss_up, *ss_down;
} dg_layer_weights;

/* embed [V][d] is also the LM head (tied), fragment-major (dg_pack_weight
 * of the row-major [V][d] matrix); final_norm [d];
 * layers: host array of n_layers entries (copied by dg_create).
 * Self-conditioning (explainer §3.2; only with d_selfcond > 0, else NULL):
 * the predicted clean-token distribution of a denoising step, p_i =
 * softmax(L_i) at temperature 1, goes through the tied embedding, e_i =
 * sum_v p_iv E_v, and the SwiGLU layer s_i = (silu(e_i W_g^T) * e_i W_u^T)
 * W_d^T, which is added to the input embedding of position i at the next
 * denoising step of the same block:
 *   sc_gate, sc_up [d_selfcond][d], sc_down [d][d_selfcond]: bf16,
 *     fragment-major (dg_pack_weight);
 *   embed_t: the embedding transposed, [d][V] (dg_pack_weight of the
 *     row-major [d][V] matrix), the operand of the contraction over the
 *     vocabulary (a second copy of the embedding, d * V * 2 bytes). */
typedef struct dg_weights {
  const void *embed, *final_norm;
  const dg_layer_weights *layers;
  const void *sc_gate, *sc_up, *sc_down, *embed_t;
  /* lmhead_format == DG_WEIGHTS_FP8 only (else NULL): the LM head reads
   * E4M3 codes of the embedding with one power-of-two scale per vocabulary
   * row, as made by dg_quantize_fp8_lmhead (embed_fp8 [V*d] bytes,
   * embed_scale [V] fp32); the input embedding stays the bf16 embed. */
  const void *embed_fp8;
  const float *embed_scale;
} dg_weights;

/* Per-position statistics of a denoising step (optional output). */
typedef struct dg_row_stats {
  float max_logit;   /* M_i = max_v L_iv */
  float log_z;       /* log sum_v exp((L_iv - M_i) / tau_s) */
  float held_logit;  /* L_i[x_i] for the token held before the step */
  float conf;        /* c_i = log p_tau(candidate) */
  int32_t argmax;    /* lowest v with L_iv = M_i */
  int32_t accepted;  /* 1 if position i is in the accepted set */
  float entropy;     /* H_i = -sum_v p_iv ln p_iv, p_i = softmax(L_i / tau_s), nats */
  int32_t sample;    /* sampled candidate (DG_CAND_SAMPLE only, else unspecified) */
  float sample_logit;/* L_i[sample] */
  int32_t pad;
} dg_row_stats;

/* The candidate of a position that is not committed:
 *   DG_CAND_ARGMAX  the most likely token (lowest id on ties);
 *   DG_CAND_SAMPLE  a draw from softmax(L_i / tau_s) by the Gumbel-max
 *                   identity: argmax_v (L_iv / tau_s - ln(-ln u_iv)), lowest
 *                   id on ties. u_iv is word ((v >> 4) & 3) of Philox4x32-10
 *                   with key = seed and counter = (v & ~0x30, i,
 *                   (block << 16) | step, 0x80000000 | req), as
 *                   ((word >> 9) + 1/2) * 2^-23. The pages accept the most
 *                   likely tokens (explainer §3.3); sampling is a variant. */
typedef enum { DG_CAND_ARGMAX = 0, DG_CAND_SAMPLE = 1 } dg_candidate;

/* How the sampler ranks canvas positions (explainer §3.3):
 *   DG_CONF_PROB     c_i = log p_tau(y_i), the candidate's log-probability;
 *   DG_CONF_ENTROPY  c_i = -H_i, low-entropy positions first. */
typedef enum { DG_CONF_PROB = 0, DG_CONF_ENTROPY = 1 } dg_confidence;

/* Arguments of dg_init_canvas / dg_denoise_step.
 *   n_req        number of requests in the batch (rows = n_req * canvas)
 *   req          host [n_req]: KV-cache slot of each request (distinct)
 *   d_canvas     device int32 [n_req][canvas], read and updated in place
 *   d_committed  device uint8 [n_req][canvas], read and updated in place
 *   step, n_steps  1 <= step <= n_steps (dg_init_canvas ignores them)
 *   seed         host uint64 [n_req]: Philox key per request
 *   block        host int32 [n_req]: block index (Philox counter word 2)
 *   d_stats      optional device dg_row_stats [n_req][canvas] (NULL = none)
 *   confidence   dg_confidence (0 = DG_CONF_PROB; another value: DG_EINVAL)
 *   stop_entropy adaptive stopping threshold in nats (explainer §3.3);
 *                <= 0 disables it (NaN: DG_EINVAL). A request's block stops at this step when
 *                the mean of H_i over its canvas is below the threshold and
 *                every position's argmax equals its argmax at the previous
 *                step of the block; the step then accepts every position.
 *   d_stop       optional device int32 [n_req]: 1 where the block stopped at
 *                this step, else 0 (NULL = not reported)
 *   candidate    dg_candidate (0 = DG_CAND_ARGMAX; another value: DG_EINVAL);
 *                needs block < 2^15 and n_steps < 2^16 for DG_CAND_SAMPLE
 * The library keeps each request slot's argmax of its last step in the
 * workspace. It counts as the previous step only for steps of the same block:
 * after dg_create, dg_init_canvas, dg_commit_block or dg_reset of a slot, the
 * slot's next step never stops.
 * Re-noise ids come from Philox4x32-10 (Salmon et al., SC'11) with
 * key = (low, high 32 bits of seed[r]) and counter = (i, step, block[r],
 * req[r]) for canvas position i of request r; id = (word0 * vocab) >> 32.
 * dg_init_canvas uses step 0. */
typedef struct dg_step_args {
  int32_t n_req;
  const int32_t *req;
  int32_t *d_canvas;
  uint8_t *d_committed;
  int32_t step, n_steps;
  const uint64_t *seed;
  const int32_t *block;
  dg_row_stats *d_stats;
  int32_t confidence;
  float stop_entropy;
  int32_t *d_stop;
  int32_t candidate;
} dg_step_args;

typedef struct dg_ctx dg_ctx;

/* Convert a row-major bf16 matrix W [n][k] into the fragment-major layout of
 * the streamed projection weights: element W[i][j] moves to index
 *   (i/16)*16*k + (j/64)*1024 + ((j%64)/32)*512 + (((j%32)/8)*16 + i%16)*8 + j%8.
 * Each 16-row block is then contiguous, and every 64-wide step of it lists,
 * for each half q, the eight consecutive elements lane L of a wavefront
 * feeds the bf16 matrix core (row i%16 = L%16, elements 32q + 8(L/16) ..)
 * in lane order, so the kernels load weights in whole 1 KB runs.
 * d_src and d_dst are device buffers of n*k elements that must not overlap;
 * the copy is enqueued on stream. DG_EINVAL if a pointer is NULL, the
 * buffers overlap, or n % 16 != 0 or k % 64 != 0. A launch failure returns
 * DG_EHIP. Needs no context. */
dg_status dg_pack_weight(void *stream, const void *d_src, void *d_dst, int64_t n, int32_t k);

/* FP8 copy of a row-major bf16 matrix W [n][k] (device pointers), for
 * DG_WEIGHTS_FP8 experts. For each row, d_scale[row] = 2^e with the smallest
 * integer e such that max_k |W[row][k]| <= 448 * 2^e (1 for a zero row), and
 * d_dst holds the OCP E4M3 code of W * 2^-e (round to nearest, ties to
 * even) in the FP8 fragment-major layout: rows in blocks of 16, each block's
 * K-steps of 64 as 1024 bytes [lane][q][8] with lane = 16*((k%32)/8) + n%16,
 * q = (k%64)/32, byte k%8. An expert bank [E][N][K] is one [E*N][K] matrix.
 * Needs n % 16 == 0, k % 64 == 0, finite weights, and d_dst [n*k bytes] not
 * overlapping d_src; else DG_EINVAL, nothing launched. Asynchronous on
 * stream; the caller owns all three buffers. */
dg_status dg_quantize_fp8(void *stream, const void *d_src, void *d_dst, float *d_scale, int64_t n,
                          int32_t k);

/* FP8 copy of a row-major bf16 matrix W [n][k] for the LM head
 * (lmhead_format = DG_WEIGHTS_FP8; the explainer's step timings, §5.2, are
 * at FP8 precision): the same codes and row scales as dg_quantize_fp8, in
 * the LM head's step-major layout: byte (k/32)*n*32 + (row/16)*512 +
 * (16*((k%32)/8) + row%16)*8 + k%8, so that every 32-wide K-step of 256
 * consecutive rows is 8 KB of consecutive bytes. Needs n % 16 == 0,
 * k % 64 == 0, finite weights and non-overlapping buffers, else DG_EINVAL
 * with nothing launched. Asynchronous on stream; the caller owns all three
 * buffers. */
dg_status dg_quantize_fp8_lmhead(void *stream, const void *d_src, void *d_dst, float *d_scale, int64_t n,
                                 int32_t k);

/* Bytes of KV cache for ONE request slot:
 * n_layers * 2 * n_kv_heads * max_ctx * head_dim * 2.
 * Layout of the whole cache: [req][layer][K|V][kv_head] planes of
 * max_ctx * head_dim bf16 each. A K plane is row-major [max_ctx][head_dim],
 * K stored after RoPE. A V plane is cut into blocks of 32 positions
 * (max_ctx % 32 == 0); inside block b, position 32b + o (o = 16*h + 4*g + r,
 * h < 2, g < 4, r < 4) and dim c sit at element
 *   32*head_dim*b + (g*head_dim + c)*8 + 4*h + r,
 * so the eight values one matrix-core lane multiplies (positions
 * {4g..4g+3, 16+4g..16+4g+3} of the block, one dim) are contiguous. */
size_t dg_kv_cache_bytes(const dg_config *cfg);

/* Bytes of device workspace needed for calls of up to cfg->max_rows rows. */
size_t dg_workspace_bytes(const dg_config *cfg);

/* Validate cfg, copy the weight pointer table and bind the caller's KV cache
 * (max_requests * dg_kv_cache_bytes) and workspace (dg_workspace_bytes).
 * The workspace must be zero-filled when the context is created (the
 * kernels' arrival counters and the wait-timeout counter read by dg_sync
 * start from it). Every request slot starts empty (cache length 0). */
dg_status dg_create(const dg_config *cfg, const dg_weights *w, void *d_kv_cache,
                    void *d_workspace, size_t workspace_bytes, dg_ctx **out);
void dg_destroy(dg_ctx *ctx);

/* Causal prefill (aiboss88.com, "hybrid attention": prefill is causal and
 * writes the KV cache): runs the encoder over d_ids[0..n) (device int32) at
 * positions len..len+n-1 of slot req and appends their K/V rows.
 * Needs len + n <= max_ctx (else DG_ECAPACITY). Processes the
 * prompt in chunks of at most max_rows rows; the result equals one causal
 * pass over the whole prompt. */
dg_status dg_prefill(dg_ctx *ctx, void *stream, int32_t req, const int32_t *d_ids,
                     int32_t n);

/* Fill each canvas with uniform random ids (Philox step 0) and clear its
 * committed mask (aiboss88.com: the canvas starts as random placeholders). */
dg_status dg_init_canvas(dg_ctx *ctx, void *stream, const dg_step_args *a);

/* One denoising step over n_req canvases (explainer §3.1-§3.3):
 *   embed the canvas (plus, with self-conditioning, the signal of the
 *   slot's previous step of the same block); for each layer: RMSNorm, QKV projection, RoPE at
 *   positions len..len+C-1, attention of every canvas position over
 *   [cached prefix ; canvas] with no mask, output projection + residual,
 *   RMSNorm, router top-k softmax, token->expert permutation, grouped SwiGLU
 *   experts plus the shared expert, weighted combine + residual;
 *   final RMSNorm; tied LM head reduced per row to (max, argmax, log-sum-exp,
 *   entropy, held-token logit) without materialising the logits; sampler:
 *     tau_s = tau_first + (tau_last - tau_first) * (step-1)/(n_steps-1),
 *     k_s   = floor(step * canvas / n_steps),
 *     candidate y_i = x_i if committed else argmax_i (or a sample, see
 *     dg_candidate),
 *     c_i = (L_i[y_i] - M_i)/tau_s - log Z_i  (or -H_i, see dg_confidence),
 *     k_s = canvas instead when the block stops early (stop_entropy),
 *     the k_s positions of highest c_i (ties: lower i) take y_i and are marked
 *     committed; all others get a fresh uniform id and are cleared.
 *   with self-conditioning, the step's own signal s_i (see dg_weights) is
 *   kept per request slot for its next step; dg_init_canvas,
 *   dg_commit_block and dg_reset of a slot forget it (the first step of a
 *   block adds nothing).
 * The canvas K/V rows are written to cache rows [len, len+C) as scratch; the
 * cache length does not change and rows [0, len) are only read.
 * Needs len + C <= max_ctx for every request (else DG_ECAPACITY). */
dg_status dg_denoise_step(dg_ctx *ctx, void *stream, const dg_step_args *a);

/* Append finished blocks (explainer §3.2: each finished block is appended to
 * the KV cache before the next block starts): the causal encoder pass over
 * d_canvas [n_req][canvas] writes K/V rows [len, len+C) of each request's
 * slot, then len += C. Needs len + C <= max_ctx (else DG_ECAPACITY). */
dg_status dg_commit_block(dg_ctx *ctx, void *stream, int32_t n_req, const int32_t *req,
                          const int32_t *d_canvas);

/* One autoregressive decode step per request (AR mode; the explainer's §5.2
 * compares a denoising step with one such step): the causal encoder pass over
 * d_tokens[r] (device int32 [n_req]) at position len of slot req[r] appends
 * that token's K/V rows (len += 1), and the LM head over its row gives
 * d_next[r] (device int32 [n_req]) = the greedy argmax, lowest id on ties.
 * Needs 1 <= n_req <= min(32, max_rows), distinct slots and len + 1 <=
 * max_ctx (else DG_EINVAL / DG_ECAPACITY, nothing launched). The workspace's
 * first n_req LM-head statistics rows are overwritten. */
dg_status dg_ar_step(dg_ctx *ctx, void *stream, int32_t n_req, const int32_t *req, const int32_t *d_tokens,
                     int32_t *d_next);

/* Committed KV length of a request slot (host-side bookkeeping), or -1. */
int32_t dg_cache_len(const dg_ctx *ctx, int32_t req);

/* Forget a slot's cache (length 0). Does not touch device memory. */
dg_status dg_reset(dg_ctx *ctx, int32_t req);

/* Set a slot's committed length without running the encoder, for callers that
 * fill the cache rows themselves (e.g. a restored snapshot of the cache). */
dg_status dg_set_cache_len(dg_ctx *ctx, int32_t req, int32_t len);

/* Wait for the work enqueued on stream, then check the kernels' own error
 * report. The grouped-expert kernel is one persistent grid whose down-
 * projection items wait, with a bounded poll, for the gate/up items of
 * their row chunk (all of which are dequeued earlier, so in a correct run
 * every wait ends). If any such wait ran out since the previous dg_sync (or
 * since dg_create), the outputs of the steps in between are unspecified:
 * the context becomes sticky and DG_EHIP is returned with a message. A HIP
 * error while waiting is also DG_EHIP. Blocks the calling thread. */
dg_status dg_sync(dg_ctx *ctx, void *stream);

/* Last error message of the context ("" if none). */
const char *dg_last_error(const dg_ctx *ctx);

/* MoE routing without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid allocation). The same kernels as the router and permutation of
 * a denoising step (explainer §2.1: 8 of 128 experts per token), run on
 * given router logits, with no context and no workspace:
 *   d_z     device fp32 [rows][n_experts] router logits (read);
 *   d_idx   device int32 [rows][top_k]: the top_k experts of each row in
 *           descending logit, ties to the lower expert id;
 *   d_w     device fp32 [rows][top_k]: softmax over the selected logits;
 *   d_cnt   device int32 [n_experts]: rows per expert;
 *   d_off   device int32 [n_experts + 1]: exclusive prefix sum of d_cnt;
 *   d_perm  device int32 [rows * top_k]: token of each expert slot, grouped
 *           by expert, tokens ascending inside an expert;
 *   d_slot  device int32 [rows][top_k]: slot in d_perm of each choice.
 * The caller owns and passes every input and output. The kernels' other
 * buffers (the permutation's work-list words and slot index, about 80 KB)
 * live in a static device array that the library holds on each GPU it runs
 * on until the process ends; this call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine). Nothing in that array needs
 * clearing between calls. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and give unspecified results. Needs 1 <= rows <=
 * DG_ROUTE_NOALLOC_MAX_ROWS, n_experts a multiple of 8 at most 128 and
 * 1 <= top_k <= min(8, n_experts), else DG_EINVAL (bad argument) or
 * DG_ECAPACITY (more rows than the static array holds), with nothing
 * launched. A launch failure returns DG_EHIP. Asynchronous on stream. */
#define DG_ROUTE_NOALLOC_MAX_ROWS 2368
dg_status dg_route_noalloc(void *stream, const float *d_z, int32_t rows, int32_t n_experts, int32_t top_k,
                           int32_t *d_idx, float *d_w, int32_t *d_cnt, int32_t *d_off, int32_t *d_perm,
                           int32_t *d_slot);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
