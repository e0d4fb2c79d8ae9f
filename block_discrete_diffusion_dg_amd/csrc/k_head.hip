// Vocabulary statistics merge and the confidence sampler.
//
// The LM-head kernel leaves, per row, one (max, sum of exp, argmax) partial
// for every 256-column tile of the vocabulary. The merge rescales the sums to
// the global max (online log-sum-exp) and keeps the lowest index among equal
// maxima. The sampler then, per request (one work-group, one thread per
// canvas position):
//   y_i  = held token if committed, else the argmax;
//   c_i  = (L_i[y_i] - M_i) / tau - log Z_i;
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

__device__ __forceinline__ void lse_merge(float& m, float& z, int& a, float m2, float z2, int a2,
                                          float k2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    // the incoming partial has the larger max (or wins the tie on index)
    const float zz = (m == -INFINITY) ? 0.f : z * exp2f((m - m2) * k2);
    z = z2 + zz;
    m = m2;
    a = a2;
  } else {
    z += (m2 == -INFINITY) ? 0.f : z2 * exp2f((m2 - m) * k2);
  }
}

__global__ __launch_bounds__(256) void lm_merge_kernel(const float4* __restrict__ part, int n_parts,
                                                       float k2, dg_row_stats* __restrict__ stats) {
  __shared__ float sm[4], sz[4];
  __shared__ int sa[4];
  const int row = blockIdx.x;
  float m = -INFINITY, z = 0.f;
  int a = 0x7fffffff;
  const float4* p = part + (int64_t)row * n_parts;
  for (int i = threadIdx.x; i < n_parts; i += 256) {
    const float4 v = p[i];
    lse_merge(m, z, a, v.x, v.y, __float_as_int(v.z), k2);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), z2 = __shfl_xor(z, o, WAVE);
    const int a2 = __shfl_xor(a, o, WAVE);
    lse_merge(m, z, a, m2, z2, a2, k2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    sz[wave] = z;
    sa[wave] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) lse_merge(m, z, a, sm[w], sz[w], sa[w], k2);
    stats[row].max_logit = m;
    stats[row].log_z = logf(z);
    stats[row].argmax = a;
  }
}

__global__ __launch_bounds__(1024) void sampler_kernel(dg_row_stats* __restrict__ stats, int C, int V,
                                                       int32_t* __restrict__ canvas,
                                                       uint8_t* __restrict__ committed, int step,
                                                       int k_s, float tau, SampleTable st,
                                                       dg_row_stats* __restrict__ stats_out) {
  __shared__ float cs[1024];
  const int r = blockIdx.x, i = threadIdx.x;
  const int row = r * C + i;
  float c = 0.f;
  int y = 0;
  bool held = false;
  dg_row_stats sr;
  if (i < C) {
    sr = stats[row];
    held = committed[row] != 0;
    y = held ? canvas[row] : sr.argmax;
    const float Ly = held ? sr.held_logit : sr.max_logit;
    c = (Ly - sr.max_logit) / tau - sr.log_z;
    cs[i] = c;
  }
  __syncthreads();
  if (i >= C) return;
  int rank = 0;
  for (int j = 0; j < C; ++j) {
    const float cj = cs[j];
    rank += (cj > c || (cj == c && j < i)) ? 1 : 0;
  }
  const bool accept = rank < k_s;
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
  sr.pad[0] = sr.pad[1] = 0;
  stats[row] = sr;
  if (stats_out) stats_out[row] = sr;
}

}  // namespace

void launch_lm_merge(hipStream_t s, const float4* part, int n_parts, int rows, float tau,
                     void* stats) {
  const float k2 = 1.4426950408889634f / tau;
  hipLaunchKernelGGL(lm_merge_kernel, dim3(rows), dim3(256), 0, s, part, n_parts, k2,
                     (dg_row_stats*)stats);
}

void launch_sampler(hipStream_t s, void* stats, int n_req, int C, int V, int32_t* canvas,
                    uint8_t* committed, int step, int k_s, float tau, const uint64_t* seeds_host,
                    const int32_t* blocks_host, const int32_t* slots_host, void* stats_out) {
  SampleTable st = make_sample_table(n_req, seeds_host, blocks_host, slots_host);
  const int threads = ((C + 63) / 64) * 64;
  hipLaunchKernelGGL(sampler_kernel, dim3(n_req), dim3(threads), 0, s, (dg_row_stats*)stats, C, V,
                     canvas, committed, step, k_s, tau, st, (dg_row_stats*)stats_out);
}
