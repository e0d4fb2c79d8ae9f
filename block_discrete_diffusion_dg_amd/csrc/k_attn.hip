// Canvas attention: every canvas (or block) position of a request attends to
// the request's cached prefix and to the block itself, with GQA (q heads
// h = g*rep .. g*rep+rep-1 read kv head g). Denoising uses no mask inside the
// block; the causal encoder (commit / prefill) masks keys after the query.
//
// Flash-style with split keys: a work-group takes 64 query vectors of one
// (request, kv head) and one contiguous range of 64-key tiles, keeps an
// online softmax, and writes an unnormalised partial output with its running
// max and sum; a merge kernel combines the splits.
//
// The wave computes S^T = K Q^T (16 queries x 64 keys per tile) so that the
// score accumulators are already laid out as the B operand of O^T = V^T P^T:
// the lane holding query column q has keys {32kk + 4g + r} and
// {32kk + 16 + 4g + r} of k-step kk, which is the same key set the A operand
// (V^T, staged transposed in LDS) supplies for that lane group.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int KT = 64;  // keys per tile

template <int DH>
__global__ __launch_bounds__(256) void attn_kernel(const bf16_t* __restrict__ q, KvGeom kv, int layer,
                                                   ReqTable rt, int Hq, int Hkv, int causal,
                                                   int nsplit, float scale_log2,
                                                   float* __restrict__ opart,
                                                   float2* __restrict__ ml) {
  constexpr int LDKs = DH + 8;
  constexpr int LDV = KT + 8;
  __shared__ __align__(16) bf16_t Ks[KT * LDKs];
  __shared__ __align__(16) bf16_t Vt[DH * LDV];

  const int rep = Hq / Hkv;
  const int n = rt.rows_per_req;
  const int rows_total = rt.n_req * n;
  const int nqv = n * rep;
  const int qblocks = div_up(nqv, 64);
  int b = blockIdx.x;
  const int split = b % nsplit;
  b /= nsplit;
  const int qb = b % qblocks;
  b /= qblocks;
  const int g = b % Hkv;
  const int r = b / Hkv;

  const int P = rt.pos0[r];
  const int nk = P + n;
  const int tiles = div_up(nk, KT);
  const int per = div_up(tiles, nsplit);
  const int t0 = split * per;
  const int t1 = min(tiles, t0 + per);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int qv = qb * 64 + wave * 16 + l16;
  const bool qvalid = qv < nqv;
  const int qi = qvalid ? qv / rep : 0;
  const int qh = g * rep + (qvalid ? qv % rep : 0);
  const int row = r * n + qi;

  u32x4 qf[DH / 32];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < DH / 32; ++s)
    qf[s] = qvalid ? ld16(q + ((int64_t)row * Hq + qh) * DH + 32 * s + 8 * grp) : zero;

  f32x4 oacc[DH / 16];
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int slot = rt.slot[r];
  const bf16_t* Kp = kv.k_plane(slot, layer, g);
  const bf16_t* Vp = kv.v_plane(slot, layer, g);
  const int qlimit = P + qi;  // causal: keys at positions <= P + qi

  for (int tile = t0; tile < t1; ++tile) {
    const int k0 = tile * KT;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DH / 32; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (DH / 8), dc = (c % (DH / 8)) * 8;
      // keys past nk re-read the last key (finite values; their scores are masked)
      const int kr = min(k0 + key, nk - 1);
      const u32x4 kk = ld16(Kp + (int64_t)kr * DH + dc);
      const u32x4 vv = ld16(Vp + (int64_t)kr * DH + dc);
      *reinterpret_cast<u32x4*>(Ks + key * LDKs + dc) = kk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(dc + 2 * e) * LDV + key] = (bf16_t)(vv[e] & 0xffffu);
        Vt[(dc + 2 * e + 1) * LDV + key] = (bf16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();

    f32x4 s[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < DH / 32; ++st) {
        const u32x4 kf = ld16(Ks + (16 * ks + l16) * LDKs + 32 * st + 8 * grp);
        s[ks] = mfma_bf16(kf, qf[st], s[ks]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = k0 + 16 * ks + 4 * grp + rr;
        float v = s[ks][rr] * scale_log2;
        if (key >= nk || (causal && key > qlimit)) v = -INFINITY;
        s[ks][rr] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) oacc[dt] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pv = exp2f(s[ks][rr] - m_use);
        s[ks][rr] = pv;
        l_run += pv;
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pf = {pack_bf16x2(s[2 * kk][0], s[2 * kk][1]), pack_bf16x2(s[2 * kk][2], s[2 * kk][3]),
                        pack_bf16x2(s[2 * kk + 1][0], s[2 * kk + 1][1]),
                        pack_bf16x2(s[2 * kk + 1][2], s[2 * kk + 1][3])};
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        const bf16_t* vr = Vt + (16 * dt + l16) * LDV + 32 * kk + 4 * grp;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
        const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
        oacc[dt] = mfma_bf16(vf, pf, oacc[dt]);
      }
    }
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
  if (qvalid) {
    const int64_t base = ((int64_t)split * rows_total + row) * Hq + qh;
    float* op = opart + base * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) op[16 * dt + 4 * grp + rr] = oacc[dt][rr];
    if (grp == 0) ml[base] = float2{m_run, l_tot};
  }
}

// out[row][h*DH + d] = sum_s 2^(m_s - M) O_s[d] / sum_s 2^(m_s - M) l_s
template <int DH>
__global__ void attn_merge_kernel(const float* __restrict__ opart, const float2* __restrict__ ml,
                                  int rows_total, int Hq, int nsplit, bf16_t* __restrict__ out) {
  const int rh = blockIdx.x;  // row * Hq + h
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[(int64_t)s * rows_total * Hq + rh].x);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float2 v = ml[(int64_t)s * rows_total * Hq + rh];
    if (v.x == -INFINITY) continue;
    const float w = exp2f(v.x - M);
    num += w * opart[((int64_t)s * rows_total * Hq + rh) * DH + d];
    den += w * v.y;
  }
  out[(int64_t)rh * DH + d] = f2bf(num / den);
}

}  // namespace

int attn_splits(const ReqTable& rt, int Hq, int Hkv, int max_rows) {
  (void)max_rows;
  const int rep = Hq / Hkv;
  const int base = rt.n_req * Hkv * div_up(rt.rows_per_req * rep, 64);
  int max_pos = 0;
  for (int r = 0; r < rt.n_req; ++r) max_pos = max(max_pos, rt.pos0[r]);
  const int tiles = div_up(max_pos + rt.rows_per_req, KT);
  int ns = div_up(1024, base);
  ns = min(ns, DG_ATTN_SPLITS);
  ns = min(ns, tiles);
  return max(ns, 1);
}

void launch_attention(hipStream_t s, const bf16_t* q, const KvGeom& kv, int layer,
                      const ReqTable& rt, int Hq, int Hkv, int dh, int causal, int nsplit,
                      float* opart, float2* ml, bf16_t* out) {
  const int rep = Hq / Hkv;
  const int blocks = rt.n_req * Hkv * div_up(rt.rows_per_req * rep, 64) * nsplit;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  const int rows_total = rt.n_req * rt.rows_per_req;
  if (dh == 128) {
    hipLaunchKernelGGL(attn_kernel<128>, dim3(blocks), dim3(256), 0, s, q, kv, layer, rt, Hq, Hkv,
                       causal, nsplit, scale_log2, opart, ml);
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(rows_total * Hq), dim3(128), 0, s, opart, ml,
                       rows_total, Hq, nsplit, out);
  } else {
    hipLaunchKernelGGL(attn_kernel<64>, dim3(blocks), dim3(256), 0, s, q, kv, layer, rt, Hq, Hkv,
                       causal, nsplit, scale_log2, opart, ml);
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(rows_total * Hq), dim3(64), 0, s, opart, ml,
                       rows_total, Hq, nsplit, out);
  }
}
