// Row-wise kernels of the step: embedding gather, RMSNorm, the RoPE table,
// the uniform initial canvas, and the weight repacking into the
// fragment-major layout of the streaming tile.
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "philox.h"
#include "stream.h"

namespace {

// h[row] = E[ids[row]] (+ the request slot's self-conditioning signal, when
// sc.state is set and the request's bit of sc.valid is) in fp32, and
// u[row] = bf16(RMSNorm(h[row]) * gain).
// E is fragment-major (it is also the LM head's streamed matrix): 8
// consecutive elements of a row are contiguous, so the row is gathered in
// 16-byte pieces through pack_index. Ids outside [0, V) are clamped (no fault).
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids,
                                                    const bf16_t* __restrict__ E, int d, int V,
                                                    float* __restrict__ h,
                                                    const bf16_t* __restrict__ gain, float eps,
                                                    bf16_t* __restrict__ u, SelfCondIn sc) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  int id = ids[row];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  float* dst = h + (int64_t)row * d;
  const float* add = nullptr;
  if (sc.state) {
    const int r = row / sc.rt.rows_per_req, i = row % sc.rt.rows_per_req;
    if ((sc.valid >> r) & 1u) add = sc.state + ((int64_t)sc.rt.slot[r] * sc.rt.rows_per_req + i) * d;
  }
  float ss = 0.f;
  for (int c = tid * 8; c < d; c += 256 * 8) {
    const u32x4 v = ld16(E + pack_index(id, c, d));
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
    if (add) {
      const float4 a0 = *reinterpret_cast<const float4*>(add + c);
      const float4 a1 = *reinterpret_cast<const float4*>(add + c + 4);
      x[0] += a0.x;
      x[1] += a0.y;
      x[2] += a0.z;
      x[3] += a0.w;
      x[4] += a1.x;
      x[5] += a1.y;
      x[6] += a1.z;
      x[7] += a1.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[c + j] = x[j];
      ss += x[j] * x[j];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
  for (int c = tid * 8; c < d; c += 256 * 8) {
    // the thread reads back the elements it wrote above
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(dst[c + 2 * j] * inv * bf2f(gain[c + 2 * j]), dst[c + 2 * j + 1] * inv * bf2f(gain[c + 2 * j + 1]));
    *reinterpret_cast<u32x4*>(u + (int64_t)row * d + c) = o;
  }
}

// u[row] = bf16( h[row] / sqrt(mean(h[row]^2) + eps) * gain )
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h,
                                                      const bf16_t* __restrict__ gain, int d,
                                                      float eps, bf16_t* __restrict__ u) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float* x = h + (int64_t)row * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  bf16_t* o = u + (int64_t)row * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    const uint32_t lo = pack_bf16x2(v.x * inv * bf2f(gain[c]), v.y * inv * bf2f(gain[c + 1]));
    const uint32_t hi = pack_bf16x2(v.z * inv * bf2f(gain[c + 2]), v.w * inv * bf2f(gain[c + 3]));
    *reinterpret_cast<u32x2*>(o + c) = u32x2{lo, hi};
  }
}

// cs[row][j] = (cos, sin)(pos * theta^(-2j/dh)), evaluated in double and
// rounded once to fp32.
__global__ void rope_table_kernel(ReqTable rt, int dh, double theta, float2* __restrict__ cs) {
  const int row = blockIdx.x, j = threadIdx.x, half = dh >> 1;
  if (j >= half) return;
  const int r = row / rt.rows_per_req, i = row % rt.rows_per_req;
  const double pos = (double)(rt.pos0[r] + i);
  const double ang = pos * pow(theta, -2.0 * (double)j / (double)dh);
  cs[(int64_t)row * half + j] = float2{(float)cos(ang), (float)sin(ang)};
}

__global__ void init_canvas_kernel(SampleTable st, int C, int V, int32_t* __restrict__ canvas,
                                   uint8_t* __restrict__ committed) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    const uint32_t w0 = philox4x32_10_word0(i, 0, st.block[r], st.slot[r], st.key_lo[r], st.key_hi[r]);
    canvas[r * C + i] = (int32_t)(((uint64_t)w0 * (uint64_t)V) >> 32);
    committed[r * C + i] = 0;
  }
}

// dst = fragment-major copy of the row-major [n][k] matrix src: thread c
// writes the c-th 16-byte piece of dst, read from the 8 elements of src that
// pack_index maps there.
__global__ void pack_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int64_t n, int k) {
  const int64_t pieces = n * (k / 8);
  const int steps = k / 64;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < pieces;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    int64_t t = c >> 6;
    const int q = (int)(t & 1);
    t >>= 1;
    const int ks = (int)(t % steps);
    const int64_t nb = t / steps;
    const int64_t row = nb * 16 + (lane & 15);
    const int col = ks * 64 + q * 32 + (lane >> 4) * 8;
    *reinterpret_cast<u32x4*>(dst + c * 8) = ld16(src + row * k + col);
  }
}

// OCP E4M3 code of v (finite, |v| <= 448), rounded to nearest with ties to
// even: below 2^-6 the representable values are multiples of 2^-9 (a result
// of 8 is the smallest normal number, whose code is also 8); in
// [2^E, 2^(E+1)) they are multiples of 2^(E-3). Sign bit from the value.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = __float_as_uint(v) >> 31;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    int x;
    (void)frexpf(a, &x);  // a = f * 2^x with f in [0.5, 1)
    int E = x - 1;
    float q = rintf(ldexpf(a, 3 - E));  // in [8, 16]; exact scaling, then round half to even
    if (q == 16.0f) {
      E += 1;
      q = 8.0f;
    }
    code = ((uint32_t)(E + 7) << 3) | ((uint32_t)q - 8u);
  }
  return (sign << 7) | code;
}

// FP8 weights from a row-major bf16 matrix src [n][k], one wave per row:
// scale[row] = 2^e for the smallest integer e with max_k |src| <= 448 * 2^e
// (e = 0 for a zero row; 448 = 0.875 * 2^9), and dst holds the E4M3 code of
// src * 2^-e (exact scaling) of every element at its pack8_index position.
// Each lane encodes 8 consecutive elements (8 contiguous bytes of dst).
// LM: codes in the step-major LM-head layout (lm8_index) instead of pack8_index.
template <bool LM>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const bf16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        float* __restrict__ scale, int64_t n, int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n) return;  // wave-uniform
  const bf16_t* r = src + row * k;
  float amax = 0.f;
  for (int c = lane; c < k; c += 64) amax = fmaxf(amax, fabsf(bf2f(r[c])));
  amax = wave_max(amax);
  int e = 0;
  if (amax > 0.f) {
    int x;
    const float f = frexpf(amax, &x);
    e = f <= 0.875f ? x - 9 : x - 8;
  }
  if (lane == 0) scale[row] = ldexpf(1.0f, e);
  for (int c0 = lane * 8; c0 < k; c0 += 512) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j >> 2] |= e4m3_code(ldexpf(bf2f(r[c0 + j]), -e)) << (8 * (j & 3));
    *reinterpret_cast<u32x2*>(dst + (LM ? lm8_index(row, c0, n) : pack8_index(row, c0, k))) = u32x2{w[0], w[1]};
  }
}

}  // namespace

void launch_quant_fp8(hipStream_t s, const bf16_t* src, uint8_t* dst, float* scale, int64_t n, int k, bool lmhead) {
  const int64_t blocks = (n + 3) / 4;
  if (lmhead)
    hipLaunchKernelGGL(quant_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, scale, n, k);
  else
    hipLaunchKernelGGL(quant_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, scale, n, k);
}

void launch_pack(hipStream_t s, const bf16_t* src, bf16_t* dst, int64_t n, int k) {
  const int64_t pieces = n * (k / 8);
  const int64_t want = (pieces + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n, k);
}

void launch_embed(hipStream_t s, const int32_t* ids, int rows, const bf16_t* embed, int d, int V,
                  float* h, const bf16_t* gain, float eps, bf16_t* u, const SelfCondIn* sc) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, ids, embed, d, V, h, gain, eps, u,
                     sc ? *sc : SelfCondIn{});
}

void launch_rmsnorm(hipStream_t s, const float* h, const bf16_t* gain, int rows, int d, float eps,
                    bf16_t* u) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, h, gain, d, eps, u);
}

void launch_rope_table(hipStream_t s, const ReqTable& rt, int dh, float theta, float2* cs) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(rt.n_req * rt.rows_per_req), dim3(64), 0, s, rt, dh,
                     (double)theta, cs);
}

void launch_init_canvas(hipStream_t s, int n_req, int C, int V, int32_t* canvas, uint8_t* committed,
                        const uint64_t* seeds_host, const int32_t* blocks_host,
                        const int32_t* slots_host) {
  SampleTable st = make_sample_table(n_req, seeds_host, blocks_host, slots_host);
  hipLaunchKernelGGL(init_canvas_kernel, dim3(n_req), dim3(256), 0, s, st, C, V, canvas, committed);
}
