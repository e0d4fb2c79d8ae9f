// libdg: the C ABI of dg.h / dg_test.h. Host code only: validation, workspace
// carving, and the launch sequence of one denoising step / encoder pass.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "../../include/dg_test.h"
#include "common.h"
#include "kernels.h"

static_assert(MOE_SPIN_TIMEOUTS == DG_ITEMS_SPIN_TIMEOUTS && MOE_TOUCHED_TOTAL == DG_ITEMS_TOUCHED_TOTAL &&
                  MOE_PERMUTE_CALLS == DG_ITEMS_PERMUTE_CALLS,
              "test header and kernels disagree");

namespace {

// Arrival counters of the router: one per 16-row block, plus one for the
// permutation run by the last block to finish.
int router_sync_words(int max_rows) { return div_up(max_rows, 16) + 1; }

struct LayerW {
  const bf16_t *attn_norm, *w_qkv, *w_o, *moe_norm, *w_router;
  const void *w_gate, *w_up, *w_down, *ws_gate, *ws_up, *ws_down;  // bf16 or FP8 codes
  ExpertScales fp8;                                                // FP8 row scales
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace carving: every buffer sized for cfg.max_rows rows.
dg_ws_layout make_layout(const dg_config& c) {
  dg_ws_layout L;
  memset(&L, 0, sizeof(L));
  const size_t R = (size_t)c.max_rows, d = c.d_model, E = c.n_experts, k = c.top_k;
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.h = take(R * d * 4);
  L.u = take(R * d * 2);
  L.q = take(R * qd * 2);
  L.attn_o = take(R * qd * 2);
  L.attn_part = take((size_t)DG_ATTN_SPLITS * R * qd * 4);
  const size_t groups = attn_groups_bound(c.max_rows, c.n_q_heads, c.n_kv_heads);
  L.attn_ml = take((size_t)DG_ATTN_SPLITS * groups * attn_group_queries() * 8);
  L.rope = take(R * (c.head_dim / 2) * 8);
  L.z = take(R * E * 4);
  L.idx = take(R * k * 4);
  L.w = take(R * k * 4);
  L.wslot = take(R * k * 4);
  L.cnt = take(256 * 4);
  L.off = take(257 * 4);
  L.items = take(((size_t)MOE_DONE + moe_chunk_bound(c.max_rows, c.n_experts, c.top_k)) * 4);
  L.perm = take(R * k * 4);
  L.slot = take(R * k * 4);
  L.hid = take(R * k * c.d_expert * 2);
  L.hid_s = take(R * c.d_shared * 2);
  L.y = take(R * k * d * 2 + R * d * 4);  // routed outputs (bf16), then the shared expert's (fp32)
  L.lm_part = take(R * (size_t)lmhead_parts(c.vocab) * 16);
  L.lm_gpart = take(R * (size_t)lmhead_parts(c.vocab) * 16);
  L.stats = take(R * sizeof(dg_row_stats));
  L.ids = take(R * 4);
  L.ss = take(R * (d / 64) * 4);
  L.zpart = take(8 * (size_t)div_up((int)R, 16) * 16 * E * 4);
  L.sync = take((router_sync_words(c.max_rows) + groups) * 4);  // router row blocks, then attention groups
  L.prev = take((size_t)c.max_requests * c.canvas * 4);
  const size_t Fsc = c.d_selfcond > 0 ? (size_t)c.d_selfcond : 0, on = Fsc > 0 ? 1 : 0;
  L.sc_p = take(on * R * c.vocab * 2);
  L.sc_qpart = take(on * R * (c.vocab / 64) * 8);
  L.sc_part = take(on * (size_t)sc_gemm_splits(c.vocab) * R * d * 4);
  L.sc_e = take(on * R * d * 2);
  L.sc_g = take(R * Fsc * 4);
  L.sc_u = take(R * Fsc * 4);
  L.sc_hid = take(R * Fsc * 2);
  L.sc_out = take(on * R * d * 4);
  L.sc_state = take(on * (size_t)c.max_requests * c.canvas * d * 4);
  L.total = o;
  return L;
}

const char* check_config(const dg_config& c) {
  if (c.n_layers < 0 || c.d_model <= 0 || c.d_model % 256 || c.d_model > 4096)
    return "d_model must be a positive multiple of 256, at most 4096";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  if (c.n_kv_heads <= 0 || c.n_q_heads <= 0 || c.n_q_heads % c.n_kv_heads)
    return "n_q_heads must be a positive multiple of n_kv_heads";
  if ((c.n_q_heads * c.head_dim) % 128 || (c.n_kv_heads * c.head_dim) % 128)
    return "n_q_heads*head_dim and n_kv_heads*head_dim must be multiples of 128";
  if (c.n_experts <= 0 || c.n_experts > 128 || c.n_experts % 8) return "n_experts must be a multiple of 8, at most 128";
  if (c.top_k <= 0 || c.top_k > 8 || c.top_k > c.n_experts) return "top_k must be in 1..min(8, n_experts)";
  if (c.d_expert <= 0 || c.d_expert % 64 || c.d_shared <= 0 || c.d_shared % 64)
    return "d_expert and d_shared must be positive multiples of 64";
  if (c.vocab <= 0 || c.vocab % 256) return "vocab must be a positive multiple of 256";
  if (c.canvas <= 0 || c.canvas % 16 || c.canvas > 1024) return "canvas must be a multiple of 16, at most 1024";
  if (c.max_requests <= 0) return "max_requests must be positive";
  if (c.max_rows < c.canvas || c.max_rows > DG_MAX_REQ * c.canvas)
    return "max_rows must lie in [canvas, 32*canvas]";
  if (c.max_ctx < 2 * c.canvas || c.max_ctx % 32) return "max_ctx must be a multiple of 32 holding at least two blocks";
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f) || !(c.tau_first > 0.f) || !(c.tau_last > 0.f))
    return "rms_eps >= 0, rope_theta > 0 and temperatures > 0 required";
  if (c.expert_format != DG_WEIGHTS_BF16 && c.expert_format != DG_WEIGHTS_FP8)
    return "expert_format must be DG_WEIGHTS_BF16 or DG_WEIGHTS_FP8";
  if (c.d_selfcond < 0 || c.d_selfcond % 64) return "d_selfcond must be 0 or a positive multiple of 64";
  if (c.lmhead_format != DG_WEIGHTS_BF16 && c.lmhead_format != DG_WEIGHTS_FP8)
    return "lmhead_format must be DG_WEIGHTS_BF16 or DG_WEIGHTS_FP8";
  return nullptr;
}

}  // namespace

struct dg_ctx {
  dg_config cfg;
  std::vector<LayerW> layers;
  const bf16_t* embed;
  const bf16_t* final_norm;
  const bf16_t *sc_gate = nullptr, *sc_up = nullptr, *sc_down = nullptr, *embed_t = nullptr;
  LmFp8 lm8{nullptr, nullptr};  // FP8 LM-head weights (lmhead_format == DG_WEIGHTS_FP8)
  const LmFp8* lm_fp8() const { return lm8.codes ? &lm8 : nullptr; }
  KvGeom kv;
  char* ws;
  dg_ws_layout lay;
  std::vector<int32_t> len;
  // per slot: 1 once a denoising step of the current block has left its
  // argmax in the workspace (adaptive stopping compares against it)
  std::vector<uint8_t> prev_valid;
  // per slot: 1 once a denoising step of the current block has left its
  // self-conditioning signal in the workspace
  std::vector<uint8_t> sc_valid;
  // expert-kernel waits that ran out, as last read by dg_sync (the counter
  // starts at zero in the zero-filled workspace)
  int32_t timeouts_seen = 0;
  bool sticky = false;
  std::string err;

  // per-stage event timing (dg_timing_enable)
  bool timing = false;
  std::vector<hipEvent_t> free_events;
  struct Pending {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  hipStream_t cur_stream = nullptr;
  int cur_stage = -1;
  hipEvent_t cur_a = nullptr;

  hipEvent_t take_event() {
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void stage_begin(hipStream_t s, int stage) {
    if (!timing) return;
    cur_stream = s;
    cur_stage = stage;
    cur_a = take_event();
    if (cur_a) (void)hipEventRecord(cur_a, s);
  }
  void stage_end() {
    if (!timing || !cur_a) return;
    hipEvent_t b = take_event();
    if (!b) return;
    (void)hipEventRecord(b, cur_stream);
    pending.push_back({cur_stage, cur_a, b});
    cur_a = nullptr;
  }
  ~dg_ctx() {
    for (auto& p : pending) {
      (void)hipEventDestroy(p.a);
      (void)hipEventDestroy(p.b);
    }
    for (auto e : free_events) (void)hipEventDestroy(e);
  }

  template <class T>
  T* buf(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
  dg_status fail(dg_status st, const std::string& msg) {
    err = msg;
    if (st == DG_EHIP) sticky = true;
    return st;
  }
  dg_status check_hip(const char* where) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DG_EHIP, std::string(where) + ": " + hipGetErrorString(e));
    return DG_OK;
  }
};

namespace {

#define STAGE(stage, ...)          \
  do {                             \
    c->stage_begin(s, stage);      \
    __VA_ARGS__;                   \
    c->stage_end();                \
  } while (0)

// One layer over the rows of every request in the table. On entry u holds
// the layer's attention pre-norm of h; on exit (unless kv_only) h is updated
// and, when next_gain is given, u holds RMSNorm(h) * next_gain for whatever
// consumes the rows next (the following layer or the LM head).
RouterPermute permute_outputs(dg_ctx* c, int rows) {
  const dg_config& g = c->cfg;
  const dg_ws_layout& L = c->lay;
  return RouterPermute{moe_rows_per_chunk(rows, g.n_experts, g.top_k), g.d_expert / 64, g.d_shared / 64,
                       g.d_model / 128, c->buf<int32_t>(L.cnt), c->buf<int32_t>(L.off), c->buf<int32_t>(L.perm),
                       c->buf<int32_t>(L.slot), c->buf<int32_t>(L.wslot), c->buf<int32_t>(L.items)};
}

void run_layer(dg_ctx* c, hipStream_t s, int l, const ReqTable& rt, int causal, bool kv_only,
               const bf16_t* next_gain) {
  const dg_config& g = c->cfg;
  const LayerW& w = c->layers[l];
  const dg_ws_layout& L = c->lay;
  const int rows = rt.n_req * rt.rows_per_req;
  const int d = g.d_model;
  float* h = c->buf<float>(L.h);
  bf16_t* u = c->buf<bf16_t>(L.u);

  const int rsync = router_sync_words(g.max_rows);
  STAGE(DG_STAGE_QKV, launch_qkv(s, u, rows, d, w.w_qkv, c->buf<bf16_t>(L.q), c->kv, l, g.n_q_heads,
                                 g.n_kv_heads, g.head_dim, c->buf<float2>(L.rope), rt, c->buf<int32_t>(L.sync),
                                 rsync + attn_groups_bound(g.max_rows, g.n_q_heads, g.n_kv_heads)));
  if (kv_only) return;
  const int ns = attn_splits(rt, g.n_q_heads, g.n_kv_heads, g.max_rows);
  STAGE(DG_STAGE_ATTN, launch_attention(s, c->buf<bf16_t>(L.q), c->kv, l, rt, g.n_q_heads, g.n_kv_heads,
                                       g.head_dim, causal, ns, c->buf<float>(L.attn_part),
                                       c->buf<float2>(L.attn_ml), c->buf<int32_t>(L.sync) + rsync,
                                       c->buf<bf16_t>(L.attn_o)));
  STAGE(DG_STAGE_OPROJ, launch_resid(s, c->buf<bf16_t>(L.attn_o), rows, g.n_q_heads * g.head_dim, w.w_o, d, h,
                                     c->buf<float>(L.ss)));
  int32_t* items = c->buf<int32_t>(L.items);
  const RouterPermute rp = permute_outputs(c, rows);
  // shared-expert prefetch by the router's early leavers: only while the
  // router is one short round of work-groups (at more rows it lengthened the
  // router more than it saved) and has enough of them to split the 25 MB
  // (at one row its 7 early leavers took ~3.6 MB each, and the AR step went
  // from 2.9 to 4.0 ms)
  const void* const rpf[3] = {w.ws_gate, w.ws_up, w.ws_down};
  const bool prefetch = rows >= 256 && rows <= 512;
  STAGE(DG_STAGE_ROUTER, launch_router(s, h, c->buf<float>(L.ss), w.moe_norm, rows, d, g.rms_eps, w.w_router,
                                       g.n_experts, g.top_k, u, c->buf<float>(L.z), c->buf<float>(L.zpart),
                                       c->buf<int32_t>(L.sync), c->buf<int32_t>(L.idx), c->buf<float>(L.w), &rp,
                                       prefetch ? rpf : nullptr,
                                       (int64_t)g.d_shared * d * (g.expert_format == DG_WEIGHTS_FP8 ? 1 : 2)));
  bf16_t* y = c->buf<bf16_t>(L.y);
  float* ys = reinterpret_cast<float*>(y + (size_t)g.max_rows * g.top_k * d);
  STAGE(DG_STAGE_EXPERTS,
        launch_moe_experts(s, u, rows, d, g.d_expert, g.d_shared, g.n_experts, g.top_k, c->buf<int32_t>(L.perm),
                           c->buf<int32_t>(L.cnt), c->buf<int32_t>(L.off), c->buf<float>(L.w),
                           c->buf<int32_t>(L.wslot), items, w.w_gate, w.w_up, w.w_down, w.ws_gate, w.ws_up,
                           w.ws_down, g.expert_format == DG_WEIGHTS_FP8 ? &w.fp8 : nullptr,
                           c->buf<bf16_t>(L.hid), c->buf<bf16_t>(L.hid_s), y, ys));
  STAGE(DG_STAGE_COMBINE, launch_moe_combine(s, h, ys, y, c->buf<int32_t>(L.slot), rows, d, g.top_k,
                                             next_gain, g.rms_eps, u));
}

// Gain of the norm that follows layer l in a denoising pass.
const bf16_t* gain_after(const dg_ctx* c, int l) {
  return l + 1 < c->cfg.n_layers ? c->layers[l + 1].attn_norm : c->final_norm;
}

// Embedding rows plus the pre-norm of the first layer (or the final norm when
// the model has no layers); with sc, the slots' self-conditioning signals
// are added first.
void run_embed(dg_ctx* c, hipStream_t s, const int32_t* ids, int rows, bool to_head,
               const SelfCondIn* sc = nullptr) {
  const dg_config& g = c->cfg;
  const bf16_t* gain = g.n_layers > 0 ? c->layers[0].attn_norm : (to_head ? c->final_norm : nullptr);
  if (!gain) gain = c->final_norm;
  launch_embed(s, ids, rows, c->embed, g.d_model, g.vocab, c->buf<float>(c->lay.h), gain, g.rms_eps,
               c->buf<bf16_t>(c->lay.u), sc);
}

// Causal encoder pass over rows whose embeddings/pre-norm are in h/u: K/V of
// every layer land in the cache; the last layer needs only its K/V.
void run_encoder(dg_ctx* c, hipStream_t s, const ReqTable& rt) {
  const int L = c->cfg.n_layers;
  for (int l = 0; l < L; ++l)
    run_layer(c, s, l, rt, 1, l == L - 1, l + 1 < L ? c->layers[l + 1].attn_norm : nullptr);
}

float tau_for(const dg_config& g, int step, int n_steps) {
  if (n_steps <= 1) return g.tau_first;
  return g.tau_first + (g.tau_last - g.tau_first) * (float)(step - 1) / (float)(n_steps - 1);
}

// LM-head statistics and their merge over the rows in u (already final-normed).
void run_lm_stats(dg_ctx* c, hipStream_t s, const dg_step_args* a) {
  const dg_config& g = c->cfg;
  const dg_ws_layout& L = c->lay;
  const int rows = a->n_req * g.canvas;
  const float tau = tau_for(g, a->step, a->n_steps);
  dg_row_stats* stats = c->buf<dg_row_stats>(L.stats);
  const bool drawn = a->candidate == DG_CAND_SAMPLE;
  GumbelDraw gd{make_sample_table(a->n_req, a->seed, a->block, a->req), g.canvas, a->step, 1.0f / tau,
                c->buf<float4>(L.lm_gpart)};
  const SelfCondOut so{c->buf<bf16_t>(L.sc_p), c->buf<float2>(L.sc_qpart)};
  STAGE(DG_STAGE_LMHEAD, launch_lmhead(s, c->buf<bf16_t>(L.u), rows, g.d_model, c->embed, g.vocab, a->d_canvas,
                                      tau, c->buf<float4>(L.lm_part), &stats[0].held_logit,
                                      (int)(sizeof(dg_row_stats) / sizeof(float)), drawn ? &gd : nullptr,
                                      g.d_selfcond > 0 ? &so : nullptr, c->lm_fp8()));
  STAGE(DG_STAGE_MERGE, launch_lm_merge(s, c->buf<float4>(L.lm_part), lmhead_parts(g.vocab), rows, tau, stats,
                                        drawn ? c->buf<float4>(L.lm_gpart) : nullptr));
}

// The confidence sampler over the per-row statistics in the workspace.
void run_sampler(dg_ctx* c, hipStream_t s, const dg_step_args* a) {
  const dg_config& g = c->cfg;
  const dg_ws_layout& L = c->lay;
  const float tau = tau_for(g, a->step, a->n_steps);
  const int k_s = (int)(((int64_t)a->step * g.canvas) / a->n_steps);
  dg_row_stats* stats = c->buf<dg_row_stats>(L.stats);
  // the previous step's argmax of a slot counts only after a step of the
  // same block (host-side, in stream order)
  uint32_t prev_valid = 0;
  for (int r = 0; r < a->n_req; ++r) {
    if (c->prev_valid[a->req[r]]) prev_valid |= 1u << r;
    c->prev_valid[a->req[r]] = 1;
  }
  const SamplerMode mode{a->confidence, a->candidate, a->stop_entropy > 0.f ? a->stop_entropy : 0.f,
                         c->buf<int32_t>(L.prev), prev_valid, a->d_stop};
  STAGE(DG_STAGE_SAMPLER, launch_sampler(s, stats, a->n_req, g.canvas, g.vocab, a->d_canvas, a->d_committed,
                                         a->step, k_s, tau, a->seed, a->block, a->req, a->d_stats, mode));
}

ReqTable make_table(dg_ctx* c, int n_req, const int32_t* req, int rows_per_req);

// Self-conditioning signal of the step (the LM head left the unnormalised
// distribution in sc_p / sc_qpart): normalise, contract with the embedding
// over the vocabulary, the feed-forward layer, then store each row's signal
// under its request slot for the slot's next step.
void run_selfcond(dg_ctx* c, hipStream_t s, const dg_step_args* a) {
  const dg_config& g = c->cfg;
  const dg_ws_layout& L = c->lay;
  const int rows = a->n_req * g.canvas, d = g.d_model, F = g.d_selfcond;
  c->stage_begin(s, DG_STAGE_SELFCOND);
  launch_sc_norm(s, c->buf<bf16_t>(L.sc_p), c->buf<float2>(L.sc_qpart), rows, g.vocab);
  launch_sc_gemm(s, c->buf<bf16_t>(L.sc_p), rows, g.vocab, c->embed_t, d, c->buf<float>(L.sc_part));
  launch_sc_merge(s, c->buf<float>(L.sc_part), sc_gemm_splits(g.vocab), rows, d, c->buf<bf16_t>(L.sc_e));
  launch_zero_f32(s, c->buf<float>(L.sc_g), (int64_t)rows * F);
  launch_zero_f32(s, c->buf<float>(L.sc_u), (int64_t)rows * F);
  launch_zero_f32(s, c->buf<float>(L.sc_out), (int64_t)rows * d);
  launch_resid(s, c->buf<bf16_t>(L.sc_e), rows, d, c->sc_gate, F, c->buf<float>(L.sc_g), nullptr);
  launch_resid(s, c->buf<bf16_t>(L.sc_e), rows, d, c->sc_up, F, c->buf<float>(L.sc_u), nullptr);
  launch_swiglu_act(s, c->buf<float>(L.sc_g), c->buf<float>(L.sc_u), c->buf<bf16_t>(L.sc_hid), (int64_t)rows * F);
  launch_resid(s, c->buf<bf16_t>(L.sc_hid), rows, F, c->sc_down, d, c->buf<float>(L.sc_out), nullptr);
  const ReqTable rt = make_table(c, a->n_req, a->req, g.canvas);
  launch_sc_store(s, c->buf<float>(L.sc_out), rt, d, c->buf<float>(L.sc_state));
  c->stage_end();
  for (int r = 0; r < a->n_req; ++r) c->sc_valid[a->req[r]] = 1;
}

// LM-head statistics, merge and sampler over the rows in u (already
// final-normed), then the self-conditioning signal for the next step.
void run_head(dg_ctx* c, hipStream_t s, const dg_step_args* a) {
  run_lm_stats(c, s, a);
  run_sampler(c, s, a);
  if (c->cfg.d_selfcond > 0) run_selfcond(c, s, a);
}

dg_status check_ctx(dg_ctx* c) {
  if (!c) return DG_EINVAL;
  if (c->sticky) return DG_ESTATE;
  return DG_OK;
}

dg_status check_step_args(dg_ctx* c, const dg_step_args* a, bool need_step) {
  const dg_config& g = c->cfg;
  if (!a || a->n_req <= 0 || a->n_req > DG_MAX_REQ || !a->req || !a->d_canvas || !a->d_committed ||
      !a->seed || !a->block)
    return c->fail(DG_EINVAL, "step args: null pointer or n_req outside 1..32");
  if (a->n_req * g.canvas > g.max_rows) return c->fail(DG_ECAPACITY, "n_req * canvas exceeds max_rows");
  for (int r = 0; r < a->n_req; ++r) {
    if (a->req[r] < 0 || a->req[r] >= g.max_requests) return c->fail(DG_EINVAL, "request slot out of range");
    for (int q = 0; q < r; ++q)
      if (a->req[q] == a->req[r]) return c->fail(DG_EINVAL, "duplicate request slot");
  }
  if (need_step && (a->n_steps <= 0 || a->step < 1 || a->step > a->n_steps))
    return c->fail(DG_EINVAL, "need 1 <= step <= n_steps");
  if (need_step && a->confidence != DG_CONF_PROB && a->confidence != DG_CONF_ENTROPY)
    return c->fail(DG_EINVAL, "confidence must be DG_CONF_PROB or DG_CONF_ENTROPY");
  if (need_step && a->stop_entropy != a->stop_entropy) return c->fail(DG_EINVAL, "stop_entropy is NaN");
  if (need_step && a->candidate != DG_CAND_ARGMAX && a->candidate != DG_CAND_SAMPLE)
    return c->fail(DG_EINVAL, "candidate must be DG_CAND_ARGMAX or DG_CAND_SAMPLE");
  if (need_step && a->candidate == DG_CAND_SAMPLE) {
    if (a->n_steps >= (1 << 16)) return c->fail(DG_EINVAL, "sampled candidates need n_steps < 65536");
    for (int r = 0; r < a->n_req; ++r)
      if (a->block[r] < 0 || a->block[r] >= (1 << 15))
        return c->fail(DG_EINVAL, "sampled candidates need 0 <= block < 32768");
  }
  return DG_OK;
}

ReqTable make_table(dg_ctx* c, int n_req, const int32_t* req, int rows_per_req) {
  ReqTable rt;
  memset(&rt, 0, sizeof(rt));
  rt.n_req = n_req;
  rt.rows_per_req = rows_per_req;
  for (int r = 0; r < n_req; ++r) {
    rt.slot[r] = req[r];
    rt.pos0[r] = c->len[req[r]];
  }
  return rt;
}

}  // namespace

extern "C" {

size_t dg_kv_cache_bytes(const dg_config* c) {
  if (!c) return 0;
  return (size_t)c->n_layers * 2 * c->n_kv_heads * (size_t)c->max_ctx * c->head_dim * sizeof(bf16_t);
}

size_t dg_workspace_bytes(const dg_config* c) {
  if (!c || check_config(*c)) return 0;
  return make_layout(*c).total;
}

dg_status dg_workspace_layout(const dg_config* c, dg_ws_layout* out) {
  if (!c || !out || check_config(*c)) return DG_EINVAL;
  *out = make_layout(*c);
  return DG_OK;
}

dg_status dg_create(const dg_config* cfg, const dg_weights* w, void* d_kv_cache, void* d_workspace,
                    size_t workspace_bytes, dg_ctx** out) {
  if (!cfg || !w || !out || !d_kv_cache || !d_workspace || !w->embed || !w->final_norm ||
      (cfg->n_layers > 0 && !w->layers))
    return DG_EINVAL;
  *out = nullptr;
  if (check_config(*cfg)) return DG_EINVAL;
  const dg_ws_layout lay = make_layout(*cfg);
  if (workspace_bytes < lay.total) return DG_ECAPACITY;
  dg_ctx* c = new (std::nothrow) dg_ctx();
  if (!c) return DG_EINVAL;
  c->cfg = *cfg;
  c->lay = lay;
  c->ws = (char*)d_workspace;
  c->embed = (const bf16_t*)w->embed;
  c->final_norm = (const bf16_t*)w->final_norm;
  if (cfg->lmhead_format == DG_WEIGHTS_FP8) {
    if (!w->embed_fp8 || !w->embed_scale) {
      delete c;
      return DG_EINVAL;
    }
    c->lm8 = LmFp8{(const uint8_t*)w->embed_fp8, w->embed_scale};
  }
  if (cfg->d_selfcond > 0) {
    if (!w->sc_gate || !w->sc_up || !w->sc_down || !w->embed_t) {
      delete c;
      return DG_EINVAL;
    }
    c->sc_gate = (const bf16_t*)w->sc_gate;
    c->sc_up = (const bf16_t*)w->sc_up;
    c->sc_down = (const bf16_t*)w->sc_down;
    c->embed_t = (const bf16_t*)w->embed_t;
  }
  c->layers.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dg_layer_weights& s = w->layers[l];
    const void* ptrs[] = {s.attn_norm, s.w_qkv, s.w_o, s.moe_norm, s.w_router, s.w_gate,
                          s.w_up, s.w_down, s.ws_gate, s.ws_up, s.ws_down};
    const void* scales[] = {s.s_gate, s.s_up, s.s_down, s.ss_gate, s.ss_up, s.ss_down};
    bool ok = true;
    for (const void* p : ptrs) ok = ok && p;
    if (cfg->expert_format == DG_WEIGHTS_FP8)
      for (const void* p : scales) ok = ok && p;
    if (!ok) {
      delete c;
      return DG_EINVAL;
    }
    c->layers[l] = LayerW{(const bf16_t*)s.attn_norm, (const bf16_t*)s.w_qkv, (const bf16_t*)s.w_o,
                          (const bf16_t*)s.moe_norm,  (const bf16_t*)s.w_router, s.w_gate,
                          s.w_up,                     s.w_down,                   s.ws_gate,
                          s.ws_up,                    s.ws_down,
                          ExpertScales{s.s_gate, s.s_up, s.s_down, s.ss_gate, s.ss_up, s.ss_down}};
  }
  c->kv.base = (bf16_t*)d_kv_cache;
  c->kv.head_stride = (int64_t)cfg->max_ctx * cfg->head_dim;
  c->kv.layer_stride = 2 * (int64_t)cfg->n_kv_heads * c->kv.head_stride;
  c->kv.slot_stride = (int64_t)cfg->n_layers * c->kv.layer_stride;
  c->kv.n_kv_heads = cfg->n_kv_heads;
  c->kv.head_dim = cfg->head_dim;
  c->len.assign(cfg->max_requests, 0);
  c->prev_valid.assign(cfg->max_requests, 0);
  c->sc_valid.assign(cfg->max_requests, 0);
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* c) { delete c; }

dg_status dg_pack_weight(void* stream, const void* d_src, void* d_dst, int64_t n, int32_t k) {
  if (!d_src || !d_dst || n <= 0 || k <= 0 || n % 16 != 0 || k % 64 != 0) return DG_EINVAL;
  const char* s0 = (const char*)d_src;
  const char* d0 = (const char*)d_dst;
  const int64_t bytes = n * (int64_t)k * 2;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return DG_EINVAL;  // overlapping buffers
  launch_pack((hipStream_t)stream, (const bf16_t*)d_src, (bf16_t*)d_dst, n, k);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_EHIP;
}

dg_status dg_quantize_fp8(void* stream, const void* d_src, void* d_dst, float* d_scale, int64_t n, int32_t k) {
  if (!d_src || !d_dst || !d_scale || n <= 0 || k <= 0 || n % 16 != 0 || k % 64 != 0) return DG_EINVAL;
  const char* s0 = (const char*)d_src;
  const char* d0 = (const char*)d_dst;
  const int64_t src_bytes = n * (int64_t)k * 2, dst_bytes = n * (int64_t)k;
  if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return DG_EINVAL;  // overlapping buffers
  launch_quant_fp8((hipStream_t)stream, (const bf16_t*)d_src, (uint8_t*)d_dst, d_scale, n, k, false);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_EHIP;
}

dg_status dg_quantize_fp8_lmhead(void* stream, const void* d_src, void* d_dst, float* d_scale, int64_t n, int32_t k) {
  if (!d_src || !d_dst || !d_scale || n <= 0 || k <= 0 || n % 16 != 0 || k % 64 != 0) return DG_EINVAL;
  const char* s0 = (const char*)d_src;
  const char* d0 = (const char*)d_dst;
  const int64_t src_bytes = n * (int64_t)k * 2, dst_bytes = n * (int64_t)k;
  if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return DG_EINVAL;  // overlapping buffers
  launch_quant_fp8((hipStream_t)stream, (const bf16_t*)d_src, (uint8_t*)d_dst, d_scale, n, k, true);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_EHIP;
}

int32_t dg_cache_len(const dg_ctx* c, int32_t req) {
  if (!c || req < 0 || req >= c->cfg.max_requests) return -1;
  return c->len[req];
}

dg_status dg_reset(dg_ctx* c, int32_t req) {
  if (!c || req < 0 || req >= c->cfg.max_requests) return DG_EINVAL;
  c->len[req] = 0;
  c->prev_valid[req] = 0;
  c->sc_valid[req] = 0;
  return DG_OK;
}

dg_status dg_set_cache_len(dg_ctx* c, int32_t req, int32_t len) {
  if (!c || req < 0 || req >= c->cfg.max_requests) return DG_EINVAL;
  if (len < 0 || len > c->cfg.max_ctx) return c->fail(DG_ECAPACITY, "length beyond max_ctx");
  c->len[req] = len;
  return DG_OK;
}

const char* dg_last_error(const dg_ctx* c) { return c ? c->err.c_str() : "null context"; }

dg_status dg_sync(dg_ctx* c, void* stream) {
  dg_status st = check_ctx(c);
  if (st) return st;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  int32_t timeouts = 0;
  if (e == hipSuccess)
    e = hipMemcpy(&timeouts, c->buf<int32_t>(c->lay.items) + MOE_SPIN_TIMEOUTS, sizeof(int32_t),
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) return c->fail(DG_EHIP, std::string("dg_sync: ") + hipGetErrorString(e));
  if (timeouts != c->timeouts_seen) {
    const int32_t n = timeouts - c->timeouts_seen;
    c->timeouts_seen = timeouts;
    return c->fail(DG_EHIP, "dg_sync: " + std::to_string(n) +
                                " bounded wait(s) of the expert kernel ran out; results since the previous "
                                "dg_sync are unspecified");
  }
  return DG_OK;
}

dg_status dg_prefill(dg_ctx* c, void* stream, int32_t req, const int32_t* d_ids, int32_t n) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (req < 0 || req >= g.max_requests || n < 0 || (n > 0 && !d_ids))
    return c->fail(DG_EINVAL, "prefill: bad request slot, length or ids");
  if ((int64_t)c->len[req] + n > g.max_ctx)
    return c->fail(DG_ECAPACITY, "prefill: cache length plus prompt exceeds max_ctx");
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  for (int done = 0; done < n;) {
    const int chunk = std::min(g.max_rows, n - done);
    const int32_t slot = req;
    ReqTable rt = make_table(c, 1, &slot, chunk);
    launch_rope_table(s, rt, g.head_dim, g.rope_theta, c->buf<float2>(L.rope));
    run_embed(c, s, d_ids + done, chunk, false);
    run_encoder(c, s, rt);
    st = c->check_hip("dg_prefill");
    if (st) return st;
    c->len[req] += chunk;
    done += chunk;
  }
  return DG_OK;
}

dg_status dg_ar_step(dg_ctx* c, void* stream, int32_t n_req, const int32_t* req, const int32_t* d_tokens,
                     int32_t* d_next) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (n_req <= 0 || n_req > DG_MAX_REQ || !req || !d_tokens || !d_next)
    return c->fail(DG_EINVAL, "ar_step: null pointer or n_req outside 1..32");
  if (n_req > g.max_rows) return c->fail(DG_ECAPACITY, "ar_step: n_req exceeds max_rows");
  for (int r = 0; r < n_req; ++r) {
    if (req[r] < 0 || req[r] >= g.max_requests) return c->fail(DG_EINVAL, "ar_step: slot out of range");
    for (int q = 0; q < r; ++q)
      if (req[q] == req[r]) return c->fail(DG_EINVAL, "ar_step: duplicate slot");
    if ((int64_t)c->len[req[r]] + 1 > g.max_ctx) return c->fail(DG_ECAPACITY, "ar_step: cache is full");
  }
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  ReqTable rt = make_table(c, n_req, req, 1);
  launch_rope_table(s, rt, g.head_dim, g.rope_theta, c->buf<float2>(L.rope));
  run_embed(c, s, d_tokens, n_req, true);
  // causal, with every layer complete (the last one feeds the final norm)
  for (int l = 0; l < g.n_layers; ++l) run_layer(c, s, l, rt, 1, false, gain_after(c, l));
  dg_row_stats* stats = c->buf<dg_row_stats>(L.stats);
  launch_lmhead(s, c->buf<bf16_t>(L.u), n_req, g.d_model, c->embed, g.vocab, d_tokens, 1.0f,
                c->buf<float4>(L.lm_part), &stats[0].held_logit, (int)(sizeof(dg_row_stats) / sizeof(float)),
                nullptr, nullptr, c->lm_fp8());
  launch_lm_merge(s, c->buf<float4>(L.lm_part), lmhead_parts(g.vocab), n_req, 1.0f, stats, nullptr);
  const hipError_t ce = hipMemcpy2DAsync(d_next, sizeof(int32_t), &stats[0].argmax, sizeof(dg_row_stats),
                                         sizeof(int32_t), n_req, hipMemcpyDeviceToDevice, s);
  if (ce != hipSuccess) return c->fail(DG_EHIP, std::string("dg_ar_step: ") + hipGetErrorString(ce));
  st = c->check_hip("dg_ar_step");
  if (st) return st;
  for (int r = 0; r < n_req; ++r) c->len[req[r]] += 1;
  return DG_OK;
}

dg_status dg_init_canvas(dg_ctx* c, void* stream, const dg_step_args* a) {
  dg_status st = check_ctx(c);
  if (st) return st;
  st = check_step_args(c, a, false);
  if (st) return st;
  for (int r = 0; r < a->n_req; ++r) c->prev_valid[a->req[r]] = c->sc_valid[a->req[r]] = 0;  // a new block
  launch_init_canvas((hipStream_t)stream, a->n_req, c->cfg.canvas, c->cfg.vocab, a->d_canvas,
                     a->d_committed, a->seed, a->block, a->req);
  return c->check_hip("dg_init_canvas");
}

}  // extern "C"

namespace {

// The denoising step; with d_h_layers, the residual stream after the
// embedding and after every layer is copied out ([n_layers + 1][rows][d]);
// with d_idx_layers, every layer's expert choices ([n_layers][rows][k]).
dg_status denoise(dg_ctx* c, void* stream, const dg_step_args* a, float* d_h_layers, int32_t* d_idx_layers,
                  const char* name) {
  dg_status st = check_ctx(c);
  if (st) return st;
  st = check_step_args(c, a, true);
  if (st) return st;
  const dg_config& g = c->cfg;
  for (int r = 0; r < a->n_req; ++r)
    if ((int64_t)c->len[a->req[r]] + g.canvas > g.max_ctx)
      return c->fail(DG_ECAPACITY, "denoise: cache length plus canvas exceeds max_ctx");
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  ReqTable rt = make_table(c, a->n_req, a->req, g.canvas);
  const int rows = a->n_req * g.canvas;
  const size_t h_bytes = (size_t)rows * g.d_model * sizeof(float);
  auto copy_h = [&](int at) {
    if (d_h_layers)
      (void)hipMemcpyAsync((char*)d_h_layers + (size_t)at * h_bytes, c->buf<float>(L.h), h_bytes,
                           hipMemcpyDeviceToDevice, s);
  };
  SelfCondIn sci{nullptr, rt, 0u};
  if (g.d_selfcond > 0) {
    sci.state = c->buf<float>(L.sc_state);
    for (int r = 0; r < a->n_req; ++r)
      if (c->sc_valid[a->req[r]]) sci.valid |= 1u << r;
  }
  STAGE(DG_STAGE_EMBED, launch_rope_table(s, rt, g.head_dim, g.rope_theta, c->buf<float2>(L.rope));
        run_embed(c, s, a->d_canvas, rows, true, g.d_selfcond > 0 ? &sci : nullptr));
  copy_h(0);
  const size_t idx_bytes = (size_t)rows * g.top_k * sizeof(int32_t);
  for (int l = 0; l < g.n_layers; ++l) {
    run_layer(c, s, l, rt, 0, false, gain_after(c, l));
    copy_h(l + 1);
    if (d_idx_layers)
      (void)hipMemcpyAsync((char*)d_idx_layers + (size_t)l * idx_bytes, c->buf<int32_t>(L.idx), idx_bytes,
                           hipMemcpyDeviceToDevice, s);
  }
  run_head(c, s, a);
  return c->check_hip(name);
}

}  // namespace

extern "C" {

dg_status dg_denoise_step(dg_ctx* c, void* stream, const dg_step_args* a) {
  return denoise(c, stream, a, nullptr, nullptr, "dg_denoise_step");
}

dg_status dg_commit_block(dg_ctx* c, void* stream, int32_t n_req, const int32_t* req,
                          const int32_t* d_canvas) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (n_req <= 0 || n_req > DG_MAX_REQ || !req || !d_canvas)
    return c->fail(DG_EINVAL, "commit: bad arguments");
  if (n_req * g.canvas > g.max_rows) return c->fail(DG_ECAPACITY, "commit: n_req * canvas exceeds max_rows");
  for (int r = 0; r < n_req; ++r) {
    if (req[r] < 0 || req[r] >= g.max_requests) return c->fail(DG_EINVAL, "commit: slot out of range");
    for (int q = 0; q < r; ++q)
      if (req[q] == req[r]) return c->fail(DG_EINVAL, "commit: duplicate slot");
    if ((int64_t)c->len[req[r]] + g.canvas > g.max_ctx)
      return c->fail(DG_ECAPACITY, "commit: cache length plus block exceeds max_ctx");
  }
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  ReqTable rt = make_table(c, n_req, req, g.canvas);
  launch_rope_table(s, rt, g.head_dim, g.rope_theta, c->buf<float2>(L.rope));
  run_embed(c, s, d_canvas, n_req * g.canvas, false);
  run_encoder(c, s, rt);
  st = c->check_hip("dg_commit_block");
  if (st) return st;
  for (int r = 0; r < n_req; ++r) {
    c->len[req[r]] += g.canvas;
    c->prev_valid[req[r]] = c->sc_valid[req[r]] = 0;  // the next block starts without a previous step
  }
  return DG_OK;
}

// ---------------------------------------------------------------- test entry points

dg_status dg_test_layer(dg_ctx* c, void* stream, int32_t req, int32_t layer, float* d_h, int32_t n,
                        int32_t causal) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (req < 0 || req >= g.max_requests || layer < 0 || layer >= g.n_layers || !d_h || n <= 0 ||
      n > g.max_rows)
    return c->fail(DG_EINVAL, "test_layer: bad arguments");
  if ((int64_t)c->len[req] + n > g.max_ctx) return c->fail(DG_ECAPACITY, "test_layer: beyond max_ctx");
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  ReqTable rt = make_table(c, 1, &req, n);
  launch_rope_table(s, rt, g.head_dim, g.rope_theta, c->buf<float2>(L.rope));
  const size_t bytes = (size_t)n * g.d_model * sizeof(float);
  (void)hipMemcpyAsync(c->buf<float>(L.h), d_h, bytes, hipMemcpyDeviceToDevice, s);
  launch_rmsnorm(s, c->buf<float>(L.h), c->layers[layer].attn_norm, n, g.d_model, g.rms_eps,
                 c->buf<bf16_t>(L.u));
  run_layer(c, s, layer, rt, causal ? 1 : 0, false, nullptr);
  (void)hipMemcpyAsync(d_h, c->buf<float>(L.h), bytes, hipMemcpyDeviceToDevice, s);
  return c->check_hip("dg_test_layer");
}

dg_status dg_test_route(dg_ctx* c, void* stream, const float* d_z, int32_t rows, int32_t* d_idx,
                        float* d_w, int32_t* d_cnt, int32_t* d_off, int32_t* d_perm, int32_t* d_slot) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (!d_z || rows <= 0 || rows > g.max_rows) return c->fail(DG_EINVAL, "test_route: bad arguments");
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  const int E = g.n_experts, k = g.top_k;
  launch_topk(s, d_z, rows, E, k, c->buf<int32_t>(L.idx), c->buf<float>(L.w));
  launch_permute(s, c->buf<int32_t>(L.idx), rows, E, k, permute_outputs(c, rows));
  auto cp = [&](void* dst, size_t off, size_t bytes) {
    if (dst) (void)hipMemcpyAsync(dst, c->ws + off, bytes, hipMemcpyDeviceToDevice, s);
  };
  cp(d_idx, L.idx, (size_t)rows * k * 4);
  cp(d_w, L.w, (size_t)rows * k * 4);
  cp(d_cnt, L.cnt, (size_t)E * 4);
  cp(d_off, L.off, (size_t)(E + 1) * 4);
  cp(d_perm, L.perm, (size_t)rows * k * 4);
  cp(d_slot, L.slot, (size_t)rows * k * 4);
  return c->check_hip("dg_test_route");
}

dg_status dg_test_head(dg_ctx* c, void* stream, const dg_step_args* a, const float* d_h) {
  dg_status st = check_ctx(c);
  if (st) return st;
  st = check_step_args(c, a, true);
  if (st) return st;
  if (!d_h) return c->fail(DG_EINVAL, "test_head: null hidden state");
  hipStream_t s = (hipStream_t)stream;
  const int rows = a->n_req * c->cfg.canvas;
  const size_t bytes = (size_t)rows * c->cfg.d_model * sizeof(float);
  (void)hipMemcpyAsync(c->buf<float>(c->lay.h), d_h, bytes, hipMemcpyDeviceToDevice, s);
  launch_rmsnorm(s, c->buf<float>(c->lay.h), c->final_norm, rows, c->cfg.d_model, c->cfg.rms_eps,
                 c->buf<bf16_t>(c->lay.u));
  run_head(c, s, a);
  return c->check_hip("dg_test_head");
}

dg_status dg_test_forward(dg_ctx* c, void* stream, const dg_step_args* a, float* d_h_layers,
                          int32_t* d_idx_layers) {
  if (c && !c->sticky && !d_h_layers) return c->fail(DG_EINVAL, "test_forward: null hidden-state buffer");
  return denoise(c, stream, a, d_h_layers, d_idx_layers, "dg_test_forward");
}

dg_status dg_test_sample(dg_ctx* c, void* stream, const dg_step_args* a, const dg_row_stats* d_in) {
  dg_status st = check_ctx(c);
  if (st) return st;
  st = check_step_args(c, a, true);
  if (st) return st;
  if (!d_in) return c->fail(DG_EINVAL, "test_sample: null statistics");
  hipStream_t s = (hipStream_t)stream;
  const size_t bytes = (size_t)a->n_req * c->cfg.canvas * sizeof(dg_row_stats);
  (void)hipMemcpyAsync(c->buf<dg_row_stats>(c->lay.stats), d_in, bytes, hipMemcpyDeviceToDevice, s);
  run_sampler(c, s, a);
  return c->check_hip("dg_test_sample");
}

dg_status dg_test_attention(dg_ctx* c, void* stream, int32_t req, int32_t layer, const void* d_q, int32_t n,
                            int32_t causal, void* d_o) {
  dg_status st = check_ctx(c);
  if (st) return st;
  const dg_config& g = c->cfg;
  if (req < 0 || req >= g.max_requests || layer < 0 || layer >= g.n_layers || !d_q || !d_o || n <= 0 ||
      n > g.max_rows)
    return c->fail(DG_EINVAL, "test_attention: bad arguments");
  if ((int64_t)c->len[req] + n > g.max_ctx) return c->fail(DG_ECAPACITY, "test_attention: beyond max_ctx");
  hipStream_t s = (hipStream_t)stream;
  const dg_ws_layout& L = c->lay;
  ReqTable rt = make_table(c, 1, &req, n);
  const size_t qd = (size_t)g.n_q_heads * g.head_dim;
  const int rsync = router_sync_words(g.max_rows);
  (void)hipMemsetAsync(c->buf<int32_t>(L.sync) + rsync, 0,
                       attn_groups_bound(g.max_rows, g.n_q_heads, g.n_kv_heads) * sizeof(int32_t), s);
  (void)hipMemcpyAsync(c->buf<bf16_t>(L.q), d_q, (size_t)n * qd * 2, hipMemcpyDeviceToDevice, s);
  const int ns = attn_splits(rt, g.n_q_heads, g.n_kv_heads, g.max_rows);
  launch_attention(s, c->buf<bf16_t>(L.q), c->kv, layer, rt, g.n_q_heads, g.n_kv_heads, g.head_dim, causal ? 1 : 0,
                   ns, c->buf<float>(L.attn_part), c->buf<float2>(L.attn_ml), c->buf<int32_t>(L.sync) + rsync,
                   c->buf<bf16_t>(L.attn_o));
  (void)hipMemcpyAsync(d_o, c->buf<bf16_t>(L.attn_o), (size_t)n * qd * 2, hipMemcpyDeviceToDevice, s);
  return c->check_hip("dg_test_attention");
}

dg_status dg_timing_enable(dg_ctx* c, int32_t enable) {
  if (!c) return DG_EINVAL;
  c->timing = enable != 0;
  return DG_OK;
}

dg_status dg_timing_read(dg_ctx* c, double* ms, int32_t* launches, int32_t n_stages) {
  if (!c || !ms || !launches || n_stages < DG_STAGE_COUNT) return DG_EINVAL;
  for (int i = 0; i < n_stages; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  if (!c->pending.empty() && hipEventSynchronize(c->pending.back().b) != hipSuccess)
    return c->fail(DG_EHIP, "dg_timing_read: event wait failed");
  for (auto& p : c->pending) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.a, p.b) == hipSuccess) {
      ms[p.stage] += t;
      launches[p.stage] += 1;
    }
    c->free_events.push_back(p.a);
    c->free_events.push_back(p.b);
  }
  c->pending.clear();
  return DG_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- routing without allocation

// Scratch of dg_route_noalloc: the permutation kernel's work-list words and
// its slot -> (token, choice) index, sized for DG_ROUTE_NOALLOC_MAX_ROWS rows
// of 128 experts top-8. One copy per GPU, shared by every call on that GPU.
constexpr size_t ROUTE_ITEMS_WORDS = (size_t)MOE_DONE + 1024;
constexpr size_t ROUTE_SCRATCH_BYTES = ROUTE_ITEMS_WORDS * 4 + (size_t)DG_ROUTE_NOALLOC_MAX_ROWS * 8 * 4;
static __device__ __align__(256) unsigned char scratch[ROUTE_SCRATCH_BYTES];

namespace {
// Device address of `scratch` on each GPU, taken once per device with that
// device current (the host-side name is not a device address).
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

void* scratch_on_current_device(hipError_t& err) {
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" dg_status dg_route_noalloc(void* stream, const float* d_z, int32_t rows, int32_t n_experts, int32_t top_k,
                                      int32_t* d_idx, float* d_w, int32_t* d_cnt, int32_t* d_off, int32_t* d_perm,
                                      int32_t* d_slot) {
  if (!d_z || !d_idx || !d_w || !d_cnt || !d_off || !d_perm || !d_slot || rows <= 0 || n_experts <= 0 ||
      n_experts > 128 || n_experts % 8 || top_k <= 0 || top_k > 8 || top_k > n_experts)
    return DG_EINVAL;
  if (rows > DG_ROUTE_NOALLOC_MAX_ROWS || permute_lds_bytes(rows, n_experts, top_k) > 57344 ||
      (size_t)MOE_DONE + moe_chunk_bound(rows, n_experts, top_k) > ROUTE_ITEMS_WORDS)
    return DG_ECAPACITY;
  hipError_t err = hipSuccess;
  char* base = static_cast<char*>(scratch_on_current_device(err));
  if (!base) return DG_EHIP;
  int32_t* items = reinterpret_cast<int32_t*>(base);
  int32_t* widx = reinterpret_cast<int32_t*>(base + ROUTE_ITEMS_WORDS * 4);
  hipStream_t s = (hipStream_t)stream;
  launch_topk(s, d_z, rows, n_experts, top_k, d_idx, d_w);
  // the expert work list the permutation also writes is scratch here: one
  // 64-column gate/up tile, one shared tile and one down tile per chunk
  const RouterPermute rp{moe_rows_per_chunk(rows, n_experts, top_k), 1, 1, 1, d_cnt, d_off, d_perm, d_slot, widx,
                         items};
  launch_permute(s, d_idx, rows, n_experts, top_k, rp);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_EHIP;
}
