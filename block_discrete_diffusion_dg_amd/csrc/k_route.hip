// MoE routing: top-k experts per token with a softmax over the selected
// logits, then the token -> expert permutation (counting sort by expert,
// tokens ascending inside an expert) built with wave ballots and a
// wave-level prefix sum.
#include <type_traits>

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

// MoE pre-norm, router logits and top-k for 8 token rows per work-group.
//  1. RMSNorm: wave w normalises rows 2w and 2w+1; u goes to the workspace
//     (the experts' input rows) and to an LDS tile (bf16, [8][d + 8]).
//  2. z = u W_r^T on the matrix cores: wave w reduces over its quarter of d
//     for all experts (8 subtiles of 16 experts, indices clamped to E-1; the
//     A rows 8..15 repeat rows 0..7 and are discarded).
//  3. z = sum of the four partial sums (fixed order); wave w selects the
//     experts of rows 2w and 2w+1 (wave_topk).
constexpr int RT_ROWS = 8;

__global__ __launch_bounds__(256) void norm_router_topk_kernel(
    const float* __restrict__ h, const bf16_t* __restrict__ gain, int rows, int d, float eps,
    const bf16_t* __restrict__ wr, int E, int k, bf16_t* __restrict__ u, float* __restrict__ z,
    int32_t* __restrict__ idx, float* __restrict__ w) {
  extern __shared__ __align__(16) char rt_lds[];
  const int LDU = d + 8;
  bf16_t* Us = reinterpret_cast<bf16_t*>(rt_lds);   // [8][LDU]
  float* part = reinterpret_cast<float*>(rt_lds);   // after phase 2: [4][8][E], then z [8][E]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * RT_ROWS;

  for (int i = 0; i < 2; ++i) {
    const int rr = wave * 2 + i, t = t0 + rr;
    bf16_t* urow = Us + rr * LDU;
    if (t < rows) {
      const float* x = h + (int64_t)t * d;
      float ss = 0.f;
      for (int c = lane * 4; c < d; c += 256) {
        const float4 v = *reinterpret_cast<const float4*>(x + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)d + eps);
      for (int c = lane * 4; c < d; c += 256) {
        const float4 v = *reinterpret_cast<const float4*>(x + c);
        const u32x2 pk = {pack_bf16x2(v.x * inv * bf2f(gain[c]), v.y * inv * bf2f(gain[c + 1])),
                          pack_bf16x2(v.z * inv * bf2f(gain[c + 2]), v.w * inv * bf2f(gain[c + 3]))};
        *reinterpret_cast<u32x2*>(u + (int64_t)t * d + c) = pk;
        *reinterpret_cast<u32x2*>(urow + c) = pk;
      }
    } else {
      for (int c = lane * 4; c < d; c += 256) *reinterpret_cast<u32x2*>(urow + c) = u32x2{0u, 0u};
    }
  }
  __syncthreads();

  const int kq = d / 4, kb = wave * kq;
  const bf16_t* arow = Us + (l16 & 7) * LDU + kb + 8 * grp;
  const bf16_t* brow[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) brow[n] = wr + (int64_t)min(16 * n + l16, E - 1) * d + kb + 8 * grp;
  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Weight loads run two 32-wide steps ahead (three register sets, loop
  // unrolled by three; steps past the end reload the last step and are
  // multiplied by a zeroed A operand).
  const int nk = kq / 32;
  u32x4 b[3][8];
  auto issue = [&](auto S, int st) {
    constexpr int s = decltype(S)::value;
    const int k0 = min(st, nk - 1) * 32;
#pragma unroll
    for (int n = 0; n < 8; ++n) b[s][n] = ld16(brow[n] + k0);
  };
  auto compute = [&](auto S, int st) {
    constexpr int s = decltype(S)::value;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 a0 = ld16(arow + min(st, nk - 1) * 32);
    const u32x4 a = st < nk ? a0 : zero;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = mfma_bf16(a, b[s][n], acc[n]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  issue(I0{}, 0);
  issue(I1{}, 1);
  for (int it = 0; it < nk; it += 3) {
    issue(I2{}, it + 2);
    compute(I0{}, it);
    issue(I0{}, it + 3);
    compute(I1{}, it + 1);
    issue(I1{}, it + 4);
    compute(I2{}, it + 2);
  }
  __syncthreads();  // the u tile is no longer read: reuse the LDS for partial sums
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int e = 16 * n + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 4 * grp + r;  // rows 0..15 of the MFMA tile; 8..15 are repeats
      if (rr < RT_ROWS && e < E) part[(wave * RT_ROWS + rr) * E + e] = acc[n][r];
    }
  }
  __syncthreads();
  float* zl = part + 4 * RT_ROWS * E;
  for (int i = tid; i < RT_ROWS * E; i += 256) {
    const float v = part[i] + part[RT_ROWS * E + i] + part[2 * RT_ROWS * E + i] + part[3 * RT_ROWS * E + i];
    zl[i] = v;
    const int t = t0 + i / E;
    if (t < rows) z[(int64_t)t * E + (i % E)] = v;
  }
  __syncthreads();
  for (int i = 0; i < 2; ++i) {
    const int rr = wave * 2 + i, t = t0 + rr;
    if (t >= rows) break;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? zl[rr * E + e] : -INFINITY;
    }
    wave_topk(v, E, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k);
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
                                                       int32_t* __restrict__ items) {
  extern __shared__ uint32_t dyn[];  // bits [rows][ceil(E/32)], then choices [rows*k] bytes
  __shared__ int32_t s_cnt[257];
  __shared__ int32_t s_off[258];
  __shared__ int32_t s_ngu[MOE_MAX_GROUPS], s_ndn[MOE_MAX_GROUPS], s_nch[MOE_MAX_GROUPS];
  __shared__ int32_t s_igu[MOE_MAX_GROUPS + 1], s_idn[MOE_MAX_GROUPS + 1], s_ich[MOE_MAX_GROUPS + 1];
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
  // groups: 0 = shared expert (all rows), 1 + e = routed expert e
  for (int g = tid; g <= E; g += 1024) {
    const int n = g == 0 ? rows : s_cnt[g - 1];
    const int nmc = (n + ch - 1) / ch;
    s_nch[g] = nmc;
    s_ngu[g] = nmc * (g == 0 ? ft_shared : ft_routed);
    s_ndn[g] = nmc * dt;
  }
  __syncthreads();
  if (wave == 0) wave_exclusive_scan(s_cnt, s_off, E, lane);
  if (wave == 1) wave_exclusive_scan(s_ngu, s_igu, E + 1, lane);
  if (wave == 2) wave_exclusive_scan(s_ndn, s_idn, E + 1, lane);
  if (wave == 3) wave_exclusive_scan(s_nch, s_ich, E + 1, lane);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = s_cnt[e];
    off[e] = s_off[e];
  }
  if (tid == 0) {
    off[E] = s_off[E];
    items[MOE_QUEUE] = 0;
  }
  if (wave == 4) {  // running statistics: experts touched per call
    int touched = 0;
    for (int e0 = 0; e0 < E; e0 += 64) touched += __popcll(__ballot(e0 + lane < E && s_cnt[e0 + lane] > 0));
    if (lane == 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(items + MOE_TOUCHED_TOTAL), (unsigned long long)touched);
      atomicAdd(reinterpret_cast<unsigned long long*>(items + MOE_PERMUTE_CALLS), 1ull);
    }
  }
  for (int g = tid; g <= E + 1; g += 1024) {
    items[MOE_ITEMS_GU + g] = s_igu[g];
    items[MOE_ITEMS_DN + g] = s_idn[g];
    items[MOE_CHUNKS + g] = s_ich[g];
  }
  for (int c = tid; c < s_ich[E + 1]; c += 1024) items[MOE_DONE + c] = 0;
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
  const size_t tile = (size_t)RT_ROWS * (d + 8) * sizeof(bf16_t);
  const size_t sums = (size_t)5 * RT_ROWS * E * sizeof(float);
  const size_t lds = tile > sums ? tile : sums;
  hipLaunchKernelGGL(norm_router_topk_kernel, dim3(div_up(rows, RT_ROWS)), dim3(256), lds, s, h, gain, rows, d,
                     eps, wr, E, k, u, z, idx, w);
}

void launch_permute(hipStream_t s, const int32_t* idx, int rows, int E, int k, int ch, int ft_routed,
                    int ft_shared, int dt, int32_t* cnt, int32_t* off, int32_t* perm, int32_t* slot,
                    int32_t* widx, int32_t* items) {
  const size_t lds = permute_lds_bytes(rows, E, k);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, idx, rows, E, k, ch, ft_routed, ft_shared,
                     dt, cnt, off, perm, slot, widx, items);
}

size_t permute_lds_bytes(int rows, int E, int k) {
  return (size_t)rows * ((E + 31) / 32) * 4 + (((size_t)rows * k + 3) & ~(size_t)3);
}
