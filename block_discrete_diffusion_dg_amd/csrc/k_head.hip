// Vocabulary statistics merge and the confidence sampler.
//
// The LM-head kernel leaves, per row, one (max m, sum of exp z, argmax,
// entropy sum w) partial for every 256-column tile of the vocabulary, with
// t_v = (L_v - m) log2(e) / tau, z = sum 2^t_v and w = sum 2^t_v t_v. The
// merge rescales them to the global max (online log-sum-exp; a partial
// shifted by d = (m - M) log2(e)/tau contributes 2^d z and 2^d (w + d z)),
// keeps the lowest index among equal maxima, and gives
//   log Z = ln z,  H = ln z - ln2 * w / z  (entropy of softmax(L / tau)).
// The sampler then, per request (one work-group, one thread per canvas
// position):
//   y_i  = held token if committed, else the argmax (or the sampled
//          candidate: the largest L/tau + Gumbel noise over the tiles);
//   c_i  = (L_i[y_i] - M_i) / tau - log Z_i, or -H_i in entropy mode;
//   stop = mean_i H_i < threshold and every argmax equals the previous
//          step's (adaptive stopping; then every position is accepted);
//   rank = #{j : c_j > c_i or (c_j == c_i and j < i)};
//   rank < k_s: accept (x_i = y_i, committed); otherwise re-noise to a
//   uniform id drawn from Philox4x32-10 at counter (i, step, block, slot).
// (codemajin.net DiffusionGemma explainer §3.3; aibars.net news item,
// "Uniform State Diffusion" paragraph.)
#include "../../include/dg.h"
#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace {

__device__ __forceinline__ void lse_merge(float& m, float& z, float& w, int& a, float m2, float z2,
                                          float w2, int a2, float k2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    // the incoming partial has the larger max (or wins the tie on index)
    if (m == -INFINITY) {
      z = z2;
      w = w2;
    } else {
      const float d = (m - m2) * k2, f = exp2f(d);
      w = w2 + f * (w + d * z);
      z = z2 + f * z;
    }
    m = m2;
    a = a2;
  } else if (m2 != -INFINITY) {
    const float d = (m2 - m) * k2, f = exp2f(d);
    w += f * (w2 + d * z2);
    z += f * z2;
  }
}

// Larger key wins; equal keys go to the lower column.
__device__ __forceinline__ void key_merge(float& k, int& c, float& lg, float k2_, int c2, float lg2) {
  if (k2_ > k || (k2_ == k && c2 < c)) {
    k = k2_;
    c = c2;
    lg = lg2;
  }
}

__global__ __launch_bounds__(256) void lm_merge_kernel(const float4* __restrict__ part, int n_parts,
                                                       float k2, dg_row_stats* __restrict__ stats,
                                                       const float4* __restrict__ gpart) {
  __shared__ float sm[4], sz[4], sw[4], sk[4], sl[4];
  __shared__ int sa[4], sc[4];
  const int row = blockIdx.x;
  float m = -INFINITY, z = 0.f, w = 0.f;
  int a = 0x7fffffff;
  const float4* p = part + (int64_t)row * n_parts;
  for (int i = threadIdx.x; i < n_parts; i += 256) {
    const float4 v = p[i];
    lse_merge(m, z, w, a, v.x, v.y, v.w, __float_as_int(v.z), k2);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), z2 = __shfl_xor(z, o, WAVE), w2 = __shfl_xor(w, o, WAVE);
    const int a2 = __shfl_xor(a, o, WAVE);
    lse_merge(m, z, w, a, m2, z2, w2, a2, k2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    sz[wave] = z;
    sw[wave] = w;
    sa[wave] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < 4; ++q) lse_merge(m, z, w, a, sm[q], sz[q], sw[q], sa[q], k2);
    const float lz = logf(z);
    stats[row].max_logit = m;
    stats[row].log_z = lz;
    stats[row].argmax = a;
    stats[row].entropy = lz - 0.69314718055994531f * (w / z);
  }
  if (!gpart) return;
  // sampled candidate: the largest key over the tiles
  float gk = -INFINITY, gl = 0.f;
  int gc = 0x7fffffff;
  const float4* gp = gpart + (int64_t)row * n_parts;
  for (int i = threadIdx.x; i < n_parts; i += 256) {
    const float4 v = gp[i];
    key_merge(gk, gc, gl, v.x, __float_as_int(v.y), v.z);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float k_ = __shfl_xor(gk, o, WAVE), l_ = __shfl_xor(gl, o, WAVE);
    const int c_ = __shfl_xor(gc, o, WAVE);
    key_merge(gk, gc, gl, k_, c_, l_);
  }
  if ((threadIdx.x & 63) == 0) {
    sk[wave] = gk;
    sc[wave] = gc;
    sl[wave] = gl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < 4; ++q) key_merge(gk, gc, gl, sk[q], sc[q], sl[q]);
    stats[row].sample = gc;
    stats[row].sample_logit = gl;
  }
}

__global__ __launch_bounds__(1024) void sampler_kernel(dg_row_stats* __restrict__ stats, int C, int V,
                                                       int32_t* __restrict__ canvas,
                                                       uint8_t* __restrict__ committed, int step,
                                                       int k_s, float tau, SampleTable st,
                                                       dg_row_stats* __restrict__ stats_out, SamplerMode mode) {
  __shared__ float cs[1024], hs[1024];
  const int r = blockIdx.x, i = threadIdx.x, nt = blockDim.x;
  const int row = r * C + i;
  float c = 0.f, H = 0.f;
  int y = 0;
  bool held = false, moved = false;
  dg_row_stats sr;
  if (i < C) {
    sr = stats[row];
    held = committed[row] != 0;
    const bool drawn = mode.candidate == DG_CAND_SAMPLE;
    y = held ? canvas[row] : (drawn ? sr.sample : sr.argmax);
    H = sr.entropy;
    if (mode.confidence == DG_CONF_ENTROPY) {
      c = -H;
    } else {
      const float Ly = held ? sr.held_logit : (drawn ? sr.sample_logit : sr.max_logit);
      c = (Ly - sr.max_logit) / tau - sr.log_z;
    }
    cs[i] = c;
    int32_t* prev = mode.prev_argmax + (int64_t)st.slot[r] * C + i;
    moved = !((mode.prev_valid >> r) & 1u) || *prev != sr.argmax;
    *prev = sr.argmax;
  }
  hs[i] = H;
  // any position whose argmax changed since the previous step of the block
  const bool any_moved = __syncthreads_or(moved ? 1 : 0) != 0;
  // sum of the entropies in a fixed tree order (deterministic)
  for (int sft = 512; sft > 0; sft >>= 1) {
    if (i < sft && i + sft < nt) hs[i] += hs[i + sft];
    __syncthreads();
  }
  const bool stop = mode.stop_entropy > 0.f && !any_moved && hs[0] < mode.stop_entropy * (float)C;
  if (i == 0 && mode.stop) mode.stop[r] = stop ? 1 : 0;
  if (i >= C) return;
  const int k = stop ? C : k_s;
  int rank = 0;
  for (int j = 0; j < C; ++j) {
    const float cj = cs[j];
    rank += (cj > c || (cj == c && j < i)) ? 1 : 0;
  }
  const bool accept = rank < k;
  if (accept) {
    canvas[row] = y;
    committed[row] = 1;
  } else {
    const uint32_t w0 = philox4x32_10_word0(i, step, st.block[r], st.slot[r], st.key_lo[r], st.key_hi[r]);
    canvas[row] = (int32_t)(((uint64_t)w0 * (uint64_t)V) >> 32);
    committed[row] = 0;
  }
  sr.conf = c;
  sr.accepted = accept ? 1 : 0;
  stats[row] = sr;
  if (stats_out) stats_out[row] = sr;
}

}  // namespace

void launch_lm_merge(hipStream_t s, const float4* part, int n_parts, int rows, float tau,
                     void* stats, const float4* gpart) {
  const float k2 = 1.4426950408889634f / tau;
  hipLaunchKernelGGL(lm_merge_kernel, dim3(rows), dim3(256), 0, s, part, n_parts, k2,
                     (dg_row_stats*)stats, gpart);
}

void launch_sampler(hipStream_t s, void* stats, int n_req, int C, int V, int32_t* canvas,
                    uint8_t* committed, int step, int k_s, float tau, const uint64_t* seeds_host,
                    const int32_t* blocks_host, const int32_t* slots_host, void* stats_out,
                    const SamplerMode& mode) {
  SampleTable st = make_sample_table(n_req, seeds_host, blocks_host, slots_host);
  const int threads = ((C + 63) / 64) * 64;
  hipLaunchKernelGGL(sampler_kernel, dim3(n_req), dim3(threads), 0, s, (dg_row_stats*)stats, C, V,
                     canvas, committed, step, k_s, tau, st, (dg_row_stats*)stats_out, mode);
}
