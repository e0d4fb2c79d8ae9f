// Host-side launchers of the gfx950 kernels (internal to libdg).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"
#include "philox.h"

// k_elem.hip
// Self-conditioning signal added to the input embeddings: state
// [slots][rows_per_req][d] fp32, read for request r when bit r of valid is set.
struct SelfCondIn {
  const float* state;
  ReqTable rt;
  uint32_t valid;
};
void launch_embed(hipStream_t s, const int32_t* ids, int rows, const bf16_t* embed, int d, int V,
                  float* h, const bf16_t* gain, float eps, bf16_t* u, const SelfCondIn* sc);
void launch_rmsnorm(hipStream_t s, const float* h, const bf16_t* gain, int rows, int d, float eps,
                    bf16_t* u);
void launch_rope_table(hipStream_t s, const ReqTable& rt, int dh, float theta, float2* cs);
void launch_init_canvas(hipStream_t s, int n_req, int C, int V, int32_t* canvas, uint8_t* committed,
                        const uint64_t* seeds_host, const int32_t* blocks_host,
                        const int32_t* slots_host);
void launch_pack(hipStream_t s, const bf16_t* src, bf16_t* dst, int64_t n, int k);
// FP8 codes in the expert layout (pack8_index) or, with lmhead, the LM head's
// step-major layout (lm8_index).
void launch_quant_fp8(hipStream_t s, const bf16_t* src, uint8_t* dst, float* scale, int64_t n, int k, bool lmhead);

// k_dense.hip (weight-streaming dense projections)
// launch_qkv also zeroes the n_sync arrival counters of the layer's router
// and attention kernels
void launch_qkv(hipStream_t s, const bf16_t* u, int rows, int d, const bf16_t* w, bf16_t* q,
                const KvGeom& kv, int layer, int Hq, int Hkv, int dh, const float2* rope,
                const ReqTable& rt, int32_t* sync, int n_sync);
// h += a W^T; ss (optional) receives per-64-column partial sums of squares
// of the updated rows, [N/64][rows]
void launch_resid(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* w, int N, float* h, float* ss);

// k_lmhead.hip (LM head with fused vocabulary statistics; embed fragment-major)
// Sampled candidates drawn in the LM-head epilogue (Gumbel-max): the
// requests' Philox keys, blocks and slots, canvas rows per request, the step,
// 1 / tau, and the per-tile partials [rows][V/256] (key, column, logit, 0).
struct GumbelDraw {
  SampleTable st;
  int C, step;
  float k1;
  float4* gpart;
};
// Self-conditioning outputs of the LM head: p [rows][V] bf16 exp(L - m) per
// 64-column quarter, qpart [rows][V/64] (m, sum of exp) per quarter.
struct SelfCondOut {
  bf16_t* p;
  float2* qpart;
};
// FP8 LM-head weights: codes in the lm8_index layout and per-row scales
// (embed8 == nullptr: the bf16 fragment-major embed).
struct LmFp8 {
  const uint8_t* codes;
  const float* scale;
};
void launch_lmhead(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* embed, int V,
                   const int32_t* held, float tau, float4* part, float* held_logit, int held_stride,
                   const GumbelDraw* gumbel, const SelfCondOut* sc, const LmFp8* fp8);
int lmhead_parts(int V);
// Self-conditioning: part[split][rows][d] = P[:, split range] ET[:, split range]^T
// (P bf16 [rows][V] normalised, ET fragment-major [d][V]); sc_gemm_splits(V) splits.
int sc_gemm_splits(int V);
void launch_sc_gemm(hipStream_t s, const bf16_t* p, int rows, int V, const bf16_t* et, int d, float* part);

// k_selfcond.hip
// p[row][v] *= exp(m_q - M) / Z1 (q = v / 64) with M = max_q m_q and
// Z1 = sum_q exp(m_q - M) z_q from qpart: the normalised softmax(L) in bf16.
void launch_sc_norm(hipStream_t s, bf16_t* p, const float2* qpart, int rows, int V);
// e[row][c] = bf16(sum over splits of part[split][row][c]) (split order).
void launch_sc_merge(hipStream_t s, const float* part, int nsplit, int rows, int d, bf16_t* e);
// x[i] = 0 for i < n (fp32; a fill kernel, no memset node under capture).
void launch_zero_f32(hipStream_t s, float* x, int64_t n);
// hid[i] = bf16(silu(g[i]) * u[i]) for i < n.
void launch_swiglu_act(hipStream_t s, const float* g, const float* u, bf16_t* hid, int64_t n);
// state[slot[r]][i][c] = out[r * C + i][c] for the requests of the table.
void launch_sc_store(hipStream_t s, const float* out, const ReqTable& rt, int d, float* state);

// k_attn.hip
int attn_splits(const ReqTable& rt, int Hq, int Hkv, int max_rows);
int attn_groups_bound(int max_rows, int Hq, int Hkv);
int attn_group_queries();  // query vectors per (request, kv head, query block) group
// V planes of the KV cache hold each 32-key block in matrix-core operand
// order: key o of the block, dim c at element ((o%16)/4 * dh + c) * 8 +
// (o/16)*4 + o%4 of the block (32*dh elements).
__host__ __device__ __forceinline__ int64_t v_index(int64_t pos, int c, int dh) {
  const int o = (int)(pos & 31);
  return (pos >> 5) * 32 * dh + ((int64_t)((o & 15) >> 2) * dh + c) * 8 + (o >> 4) * 4 + (o & 3);
}
void launch_attention(hipStream_t s, const bf16_t* q, const KvGeom& kv, int layer, const ReqTable& rt, int Hq,
                      int Hkv, int dh, int causal, int nsplit, float* opart, float2* ml, int32_t* sync, bf16_t* out);

// k_route.hip
void launch_topk(hipStream_t s, const float* z, int rows, int E, int k, int32_t* idx, float* w);
// Outputs of the token -> expert permutation and the expert kernel's work
// list (see k_route.hip).
struct RouterPermute {
  int ch, ft_routed, ft_shared, dt;  // chunk rows; gate/up tiles (routed, shared); down tiles
  int32_t *cnt, *off, *perm, *slot, *widx, *items;
};
// Router (MoE pre-norm, logits, top-k); with perm, the last row block to
// finish also runs the permutation (sync needs div_up(rows, 16) + 1 words).
// pf / pfn: three byte ranges of pfn bytes each (the shared expert's
// matrices) that work-groups leaving early prefetch (prefetch_stripe).
void launch_router(hipStream_t s, const float* h, const float* ss, const bf16_t* gain, int rows, int d, float eps,
                   const bf16_t* wr, int E, int k, bf16_t* u, float* z, float* zpart, int32_t* sync, int32_t* idx,
                   float* w, const RouterPermute* perm, const void* const* pf = nullptr, int64_t pfn = 0);
// The permutation as a launch of its own, from expert ids of an earlier launch.
void launch_permute(hipStream_t s, const int32_t* idx, int rows, int E, int k, const RouterPermute& p);
size_t permute_lds_bytes(int rows, int E, int k);

// k_moe.hip
int moe_rows_per_chunk(int rows, int E, int k);
int moe_chunk_bound(int rows, int E, int k);
// Row scales of FP8 expert weights: g / u [E*F], d [E*d] (routed banks),
// sg / su [Fs], sd [d] (shared expert).
struct ExpertScales {
  const float *g, *u, *d, *sg, *su, *sd;
};
// Expert weights are bf16 (fp8 == nullptr) or FP8 codes with the given row
// scales.
void launch_moe_experts(hipStream_t s, const bf16_t* u, int rows, int d, int F, int Fs, int E, int k,
                        const int32_t* perm, const int32_t* cnt, const int32_t* off, const float* wts,
                        const int32_t* widx, int32_t* items, const void* wg, const void* wu, const void* wd,
                        const void* sg, const void* su, const void* sd, const ExpertScales* fp8, bf16_t* hid,
                        bf16_t* hid_s, bf16_t* y, float* ys);
void launch_moe_combine(hipStream_t s, float* h, const float* ys, const bf16_t* y,
                        const int32_t* slot, int rows, int d, int k, const bf16_t* next_gain,
                        float eps, bf16_t* u);

// k_head.hip
// gpart: the sampled-candidate partials of launch_lmhead, or nullptr.
void launch_lm_merge(hipStream_t s, const float4* part, int n_parts, int rows, float tau,
                     void* stats, const float4* gpart);
// Sampler options: confidence (dg_confidence), adaptive stopping threshold
// (0 = off), the per-slot argmax of the previous step [slots][C] (read, then
// overwritten), which requests of the batch have one (bit r), and the
// optional per-request stop flags.
struct SamplerMode {
  int confidence;
  int candidate;  // dg_candidate
  float stop_entropy;
  int32_t* prev_argmax;
  uint32_t prev_valid;
  int32_t* stop;
};
void launch_sampler(hipStream_t s, void* stats, int n_req, int C, int V, int32_t* canvas,
                    uint8_t* committed, int step, int k_s, float tau, const uint64_t* seeds_host,
                    const int32_t* blocks_host, const int32_t* slots_host, void* stats_out,
                    const SamplerMode& mode);
