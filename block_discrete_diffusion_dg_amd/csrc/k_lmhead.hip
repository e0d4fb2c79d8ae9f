// LM head: logits L = u E^T on the gfx950 matrix cores (u: the final-normed
// token rows, bf16; E: the tied embedding in the fragment-major layout of
// stream.h), with an epilogue that reduces every row of each 256-column tile
// to (max, first argmax, sum of exp), so the vocabulary-wide softmax is never
// materialised (the statistics the confidence sampler needs: codemajin.net
// DiffusionGemma explainer §3.3).
//
// A work-group covers CH = 16*MT token rows by 256 vocabulary columns on the
// weight-streaming tile: wave w owns columns 64w .. 64w+63 as four 16-row
// blocks of the packed embedding, streamed from HBM into registers, so each
// A fragment read from LDS feeds four matrix-core products. The row chunks
// of one column tile get work-group ids 8 apart (same XCD): the embedding is
// read from HBM once and re-read by the other chunks from L2.
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace {

constexpr int LM_NB = 4;                 // 16-column weight blocks per wave
constexpr int LM_COLS = 4 * 16 * LM_NB;  // columns per work-group

// part[row][nt] = (max, sum exp2((L - max) * k2), first argmax bits, 0) over
// the 256 columns of tile nt, k2 = log2(e) / tau; the lane holding the column
// of the row's held token writes that logit to held_logit[row * held_stride].
// Requires K % 64 == 0 and V % 256 == 0 (the configuration check enforces both).
template <int MT>
__global__ __launch_bounds__(256) void lmhead_kernel(const bf16_t* __restrict__ A, int rows, int K,
                                                     const bf16_t* __restrict__ E, int V,
                                                     const int32_t* __restrict__ held, float k2,
                                                     float4* __restrict__ part, float* __restrict__ held_logit,
                                                     int held_stride) {
  using T = StreamTile<MT>;
  constexpr int CH = T::CH;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  __shared__ float4 red[4][CH];
  __shared__ int s_held[CH];

  const int NT = V / LM_COLS, MC = div_up(rows, CH);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int row0 = mc * CH, nrows = min(CH, rows - row0);
  const int c0 = nt * LM_COLS + wave * 64;  // the wave's first column
  if (tid < CH) s_held[tid] = tid < nrows ? held[row0 + tid] : -1;

  const bf16_t* const wblk = E + (int64_t)(c0 / 16) * 16 * K;
  const bf16_t* const w[LM_NB] = {wblk, wblk + 16 * K, wblk + 32 * K, wblk + 48 * K};
  f32x4 acc[LM_NB][MT];
  stream_tile_n<MT, LM_NB>(A, K, nullptr, row0, nrows, w, K, acc, lds);

  // Per row (16mt + 4grp + r of the chunk), over the wave's 64 columns
  // (16nb + l16): max, the smallest column holding it, and sum exp2((L - max) k2).
  // All rows are reduced first (independent chains on the DPP network), then
  // the held-token logits are picked out.
  float m[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      m[mt][r] = row16_max(fmaxf(fmaxf(acc[0][mt][r], acc[1][mt][r]), fmaxf(acc[2][mt][r], acc[3][mt][r])));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int ix = 0x7fffffff;
      float z = 0.f;
#pragma unroll
      for (int nb = LM_NB - 1; nb >= 0; --nb) {
        const float v = acc[nb][mt][r];
        if (v == m[mt][r]) ix = c0 + 16 * nb + l16;
        z += __builtin_amdgcn_exp2f((v - m[mt][r]) * k2);
      }
      ix = row16_min(ix);
      z = row16_sum(z);
      if (l16 == 0) red[wave][16 * mt + 4 * grp + r] = float4{m[mt][r], z, __int_as_float(ix), 0.f};
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = 16 * mt + 4 * grp + r;
      const int hc = s_held[rl] - c0;
      if (hc >= 0 && hc < 64 && (hc & 15) == l16) {
        float hv = acc[0][mt][r];
#pragma unroll
        for (int nb = 1; nb < LM_NB; ++nb)
          if (nb == (hc >> 4)) hv = acc[nb][mt][r];
        held_logit[(int64_t)(row0 + rl) * held_stride] = hv;
      }
    }
  __syncthreads();
  if (tid < nrows) {
    // merge the four waves in column order: the first wave holding the
    // maximum also holds its smallest column
    float4 p = red[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 o = red[w][tid];
      if (o.x > p.x) {
        p.y = o.y + p.y * __builtin_amdgcn_exp2f((p.x - o.x) * k2);
        p.x = o.x;
        p.z = o.z;
      } else {
        p.y += o.y * __builtin_amdgcn_exp2f((o.x - p.x) * k2);
      }
    }
    part[(int64_t)(row0 + tid) * NT + nt] = p;
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers

int lmhead_parts(int V) { return V / LM_COLS; }

void launch_lmhead(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* embed, int V,
                   const int32_t* held, float tau, float4* part, float* held_logit, int held_stride) {
  const float k2 = 1.4426950408889634f / tau;
  const int NT = V / LM_COLS;
#define DG_LMHEAD(MT_)                                                                                    \
  hipLaunchKernelGGL(lmhead_kernel<MT_>, dim3(NT * div_up(rows, 16 * MT_)), dim3(256), 0, s, a, rows, K, \
                     embed, V, held, k2, part, held_logit, held_stride)
  if (rows <= 32)
    DG_LMHEAD(2);
  else if (rows <= 64)
    DG_LMHEAD(4);
  else
    DG_LMHEAD(8);
#undef DG_LMHEAD
}
