// MoE routing: top-k experts per token with a softmax over the selected
// logits, then the token -> expert permutation (counting sort by expert,
// tokens ascending inside an expert) built with wave ballots and a
// wave-level prefix sum.
#include "common.h"
#include "kernels.h"

size_t permute_lds_bytes(int rows, int E, int k);

namespace {

// One wave selects the top-k (k <= 8) of E <= 256 logits, lane l holding
// experts l, l+64, l+128, l+192 in v[0..3]: k rounds of a wave arg-max (ties
// to the lower expert id) pick the experts in descending order; lane 0 writes
// them and the softmax of the picked logits.
__device__ __forceinline__ void wave_topk(const float (&v)[4], int E, int k, int lane,
                                          int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  bool taken[4] = {false, false, false, false};
  float sel[8];
  int sid[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !taken[i]) argmax_merge(bv, bi, v[i], e);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, WAVE);
      const int i2 = __shfl_xor(bi, o, WAVE);
      argmax_merge(bv, bi, v2, i2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == lane + 64 * i) taken[i] = true;
    sel[j] = bv;
    sid[j] = bi;
  }
  if (lane == 0) {
    const float m = sel[0];
    float ex[8], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      ex[j] = expf(sel[j] - m);
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      idx_out[j] = sid[j];
      w_out[j] = ex[j] / sum;
    }
  }
}

// Top-k from given router logits: one wave per token.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int rows, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= rows) return;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? z[(int64_t)t * E + e] : -INFINITY;
  }
  wave_topk(v, E, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k);
}

// MoE pre-norm, router logits and top-k for one token row per work-group:
//   u = bf16(RMSNorm(h) * g)        (also the experts' input rows)
//   z[e] = u . W_r[e]               (fp32; wave w takes experts w, w+4, ...,
//                                    each lane 1/64 of the row, then a
//                                    wave-level sum)
//   top-k of z with softmax weights (wave_topk).
__global__ __launch_bounds__(256) void norm_router_topk_kernel(
    const float* __restrict__ h, const bf16_t* __restrict__ gain, int d, float eps,
    const bf16_t* __restrict__ wr, int E, int k, bf16_t* __restrict__ u, float* __restrict__ z,
    int32_t* __restrict__ idx, float* __restrict__ w) {
  extern __shared__ float sh[];  // u as fp32 [d], then z [E]
  __shared__ float red[4];
  float* us = sh;
  float* zl = sh + d;
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* x = h + (int64_t)row * d;
  float ss = 0.f;
  for (int c = tid * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
  bf16_t* uo = u + (int64_t)row * d;
  for (int c = tid * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    const bf16_t b0 = f2bf(v.x * inv * bf2f(gain[c])), b1 = f2bf(v.y * inv * bf2f(gain[c + 1]));
    const bf16_t b2 = f2bf(v.z * inv * bf2f(gain[c + 2])), b3 = f2bf(v.w * inv * bf2f(gain[c + 3]));
    *reinterpret_cast<u32x2*>(uo + c) =
        u32x2{(uint32_t)b0 | ((uint32_t)b1 << 16), (uint32_t)b2 | ((uint32_t)b3 << 16)};
    us[c] = bf2f(b0);
    us[c + 1] = bf2f(b1);
    us[c + 2] = bf2f(b2);
    us[c + 3] = bf2f(b3);
  }
  __syncthreads();
  const int per = d / 64;  // elements of the row per lane (multiple of 4)
  for (int e = wave; e < E; e += 4) {
    const bf16_t* wrow = wr + (int64_t)e * d + lane * per;
    const float* ur = us + lane * per;
    float acc = 0.f;
    for (int j = 0; j < per; j += 4) {
      const u32x2 wv = *reinterpret_cast<const u32x2*>(wrow + j);
      acc += ur[j] * __uint_as_float(wv.x << 16);
      acc += ur[j + 1] * __uint_as_float(wv.x & 0xffff0000u);
      acc += ur[j + 2] * __uint_as_float(wv.y << 16);
      acc += ur[j + 3] * __uint_as_float(wv.y & 0xffff0000u);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      zl[e] = acc;
      z[(int64_t)row * E + e] = acc;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? zl[e] : -INFINITY;
    }
    wave_topk(v, E, k, lane, idx + (int64_t)row * k, w + (int64_t)row * k);
  }
}

// Exclusive prefix sum of n <= 320 ints by one wave (5 consecutive per lane);
// out[n] receives the total.
__device__ void wave_exclusive_scan(const int32_t* in, int32_t* out, int n, int lane) {
  int local[5], acc = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = lane * 5 + i;
    local[i] = e < n ? in[e] : 0;
    acc += local[i];
  }
  int inc = acc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += y;
  }
  int run = inc - acc;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = lane * 5 + i;
    if (e < n) out[e] = run;
    run += local[i];
  }
  if (lane == 63) out[n] = inc;
}

// Single work-group of 1024 threads (16 waves).
//  1. mark (token, expert) bits in LDS, keep the choices as bytes in LDS;
//  2. cnt[e] = popcount of ballots over the token column of expert e;
//  3. off = exclusive prefix sum of cnt; work-item offsets of the grouped
//     expert kernels (E routed groups + the shared expert as group E, each
//     cut into chunks of ch rows, times its column tiles);
//  4. slot of (t, e) = off[e] + number of earlier tokens of e (ballot rank);
//     widx[slot] = t*k + j locates the slot's routing weight w[t][j].
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx, int rows, int E,
                                                       int k, int ch, int ft_routed, int ft_shared,
                                                       int dt, int32_t* __restrict__ cnt,
                                                       int32_t* __restrict__ off,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ slot,
                                                       int32_t* __restrict__ widx,
                                                       int32_t* __restrict__ items_gu,
                                                       int32_t* __restrict__ items_dn) {
  extern __shared__ uint32_t dyn[];  // bits [rows][ceil(E/32)], then choices [rows*k] bytes
  __shared__ int32_t s_cnt[257];
  __shared__ int32_t s_off[258];
  __shared__ int32_t s_ngu[257], s_ndn[257];
  __shared__ int32_t s_igu[258], s_idn[258];
  const int words = (E + 31) / 32;
  uint32_t* bits = dyn;
  uint8_t* choice = reinterpret_cast<uint8_t*>(dyn + rows * words);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < rows * words; i += 1024) bits[i] = 0u;
  __syncthreads();
  for (int i = tid; i < rows * k; i += 1024) {
    const int t = i / k, e = idx[i];
    choice[i] = (uint8_t)e;
    atomicOr(&bits[t * words + (e >> 5)], 1u << (e & 31));
  }
  __syncthreads();
  for (int e = wave; e < E; e += 16) {
    int c = 0;
    for (int t0 = 0; t0 < rows; t0 += 64) {
      const int t = t0 + lane;
      const bool bit = t < rows && ((bits[t * words + (e >> 5)] >> (e & 31)) & 1u);
      c += __popcll(__ballot(bit));
    }
    if (lane == 0) s_cnt[e] = c;
  }
  __syncthreads();
  for (int g = tid; g <= E; g += 1024) {
    const int n = g < E ? s_cnt[g] : rows;
    const int nmc = (n + ch - 1) / ch;
    s_ngu[g] = nmc * (g < E ? ft_routed : ft_shared);
    s_ndn[g] = nmc * dt;
  }
  __syncthreads();
  if (wave == 0) wave_exclusive_scan(s_cnt, s_off, E, lane);
  if (wave == 1) wave_exclusive_scan(s_ngu, s_igu, E + 1, lane);
  if (wave == 2) wave_exclusive_scan(s_ndn, s_idn, E + 1, lane);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = s_cnt[e];
    off[e] = s_off[e];
  }
  if (tid == 0) off[E] = s_off[E];
  for (int g = tid; g <= E + 1; g += 1024) {
    items_gu[g] = s_igu[g];
    items_dn[g] = s_idn[g];
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = wave; e < E; e += 16) {
    int run = s_off[e];
    for (int t0 = 0; t0 < rows; t0 += 64) {
      const int t = t0 + lane;
      const bool bit = t < rows && ((bits[t * words + (e >> 5)] >> (e & 31)) & 1u);
      const uint64_t m = __ballot(bit);
      if (bit) {
        const int pos = run + __popcll(m & lt);
        perm[pos] = t;
        for (int j = 0; j < k; ++j)
          if (choice[t * k + j] == e) {
            slot[t * k + j] = pos;
            widx[pos] = t * k + j;
          }
      }
      run += __popcll(m);
    }
  }
}

}  // namespace

void launch_topk(hipStream_t s, const float* z, int rows, int E, int k, int32_t* idx, float* w) {
  hipLaunchKernelGGL(topk_kernel, dim3(div_up(rows, 4)), dim3(256), 0, s, z, rows, E, k, idx, w);
}

void launch_norm_router_topk(hipStream_t s, const float* h, const bf16_t* gain, int rows, int d, float eps,
                             const bf16_t* wr, int E, int k, bf16_t* u, float* z, int32_t* idx, float* w) {
  const size_t lds = (size_t)(d + E) * sizeof(float);
  hipLaunchKernelGGL(norm_router_topk_kernel, dim3(rows), dim3(256), lds, s, h, gain, d, eps, wr, E, k, u, z,
                     idx, w);
}

void launch_permute(hipStream_t s, const int32_t* idx, int rows, int E, int k, int ch, int ft_routed,
                    int ft_shared, int dt, int32_t* cnt, int32_t* off, int32_t* perm, int32_t* slot,
                    int32_t* widx, int32_t* items_gu, int32_t* items_dn) {
  const size_t lds = permute_lds_bytes(rows, E, k);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, idx, rows, E, k, ch, ft_routed, ft_shared,
                     dt, cnt, off, perm, slot, widx, items_gu, items_dn);
}

size_t permute_lds_bytes(int rows, int E, int k) {
  return (size_t)rows * ((E + 31) / 32) * 4 + (((size_t)rows * k + 3) & ~(size_t)3);
}
