// Self-conditioning (codemajin.net DiffusionGemma explainer §3.2): the
// predicted clean-token distribution of a denoising step, p_i = softmax(L_i)
// over the vocabulary, goes through the tied embedding, e_i = sum_v p_iv E_v,
// and a small SwiGLU feed-forward layer; the result is added to the next
// step's input embedding of position i.
//
// The LM head leaves p_v = exp(L_v - m_q) per 64-column quarter q (bf16) and
// (m_q, z_q = sum of those exponentials); sc_norm_kernel turns them into the
// normalised distribution in place; the contraction with the embedding is a
// split-K matrix product over the vocabulary (k_lmhead.hip), whose partial
// sums sc_merge_kernel adds in split order (deterministic); the feed-forward
// layer runs on the dense projection kernels with the activation below.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

// One work-group per row: M = max_q m_q and Z1 = sum_q exp(m_q - M) z_q (a
// fixed reduction order), then p[v] = bf16(p[v] * exp(m_q - M) / Z1) for
// every v of the row, eight at a time (eight consecutive v share a quarter).
__global__ __launch_bounds__(256) void sc_norm_kernel(bf16_t* __restrict__ p, const float2* __restrict__ qpart,
                                                      int V) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int NQ = V / 64;
  const float2* q = qpart + (int64_t)row * NQ;
  float m = -INFINITY;
  for (int i = tid; i < NQ; i += 256) m = fmaxf(m, q[i].x);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float z = 0.f;
  for (int i = tid; i < NQ; i += 256) z += __expf(q[i].x - M) * q[i].y;
  z = wave_sum(z);
  if ((tid & 63) == 0) red[tid >> 6] = z;
  __syncthreads();
  const float inv = 1.0f / (((red[0] + red[1]) + red[2]) + red[3]);
  bf16_t* pr = p + (int64_t)row * V;
  for (int i = tid; i < V / 8; i += 256) {
    const float f = __expf(q[i >> 3].x - M) * inv;
    u32x4 v = *reinterpret_cast<const u32x4*>(pr + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = pack_bf16x2(__uint_as_float(v[j] << 16) * f, __uint_as_float(v[j] & 0xffff0000u) * f);
    *reinterpret_cast<u32x4*>(pr + 8 * i) = v;
  }
}

// e[row][c..c+3] = bf16(sum_s part[s][row][c..c+3]), splits in order.
__global__ __launch_bounds__(256) void sc_merge_kernel(const float* __restrict__ part, int nsplit, int rows, int d,
                                                       bf16_t* __restrict__ e) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t n = (int64_t)rows * d;
  if (i >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int sp = 1; sp < nsplit; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)sp * n + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<u32x2*>(e + i) = u32x2{pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

__global__ __launch_bounds__(256) void swiglu_act_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                         bf16_t* __restrict__ hid, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float a = g[i];
    hid[i] = f2bf(a / (1.0f + expf(-a)) * u[i]);
  }
}

// One work-group per call row: state[slot][i] = out[row] (d floats).
__global__ __launch_bounds__(256) void sc_store_kernel(const float* __restrict__ out, ReqTable rt, int d,
                                                       float* __restrict__ state) {
  const int row = blockIdx.x;
  const int r = row / rt.rows_per_req, i = row % rt.rows_per_req;
  const float* src = out + (int64_t)row * d;
  float* dst = state + ((int64_t)rt.slot[r] * rt.rows_per_req + i) * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024)
    *reinterpret_cast<float4*>(dst + c) = *reinterpret_cast<const float4*>(src + c);
}

}  // namespace

void launch_sc_norm(hipStream_t s, bf16_t* p, const float2* qpart, int rows, int V) {
  hipLaunchKernelGGL(sc_norm_kernel, dim3(rows), dim3(256), 0, s, p, qpart, V);
}

void launch_sc_merge(hipStream_t s, const float* part, int nsplit, int rows, int d, bf16_t* e) {
  const int64_t n4 = (int64_t)rows * d / 4;
  hipLaunchKernelGGL(sc_merge_kernel, dim3((unsigned)div_up((int)n4, 256)), dim3(256), 0, s, part, nsplit, rows, d, e);
}

void launch_zero_f32(hipStream_t s, float* x, int64_t n) {
  const int blocks = (int)std::min<int64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, x, n);
}

void launch_swiglu_act(hipStream_t s, const float* g, const float* u, bf16_t* hid, int64_t n) {
  const int blocks = (int)std::min<int64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(swiglu_act_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, g, u, hid, n);
}

void launch_sc_store(hipStream_t s, const float* out, const ReqTable& rt, int d, float* state) {
  hipLaunchKernelGGL(sc_store_kernel, dim3(rt.n_req * rt.rows_per_req), dim3(256), 0, s, out, rt, d, state);
}
