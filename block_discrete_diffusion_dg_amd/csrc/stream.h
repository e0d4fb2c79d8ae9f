// Weight-streaming tile for skinny GEMMs on the gfx950 matrix cores.
//
// In a denoising step every weight matrix meets at most a few hundred token
// rows, so the weights are read from HBM once (straight into MFMA B
// operands, no LDS) while the token rows ride along. A work-group covers a
// chunk of CH = 16*MT rows against 64 weight rows (16 per wave); with
// GATED the lane also owns a second weight row (the "up" row of a SwiGLU, or
// the rotate-half partner of a RoPE pair) and a second accumulator.
//
// The A rows (optionally gathered through a row map) are staged per K-step in
// a double-buffered LDS tile shared by the four waves. The next K-step's A
// and B loads are issued before the current step's MFMAs; one barrier per
// step.
//
// Reduction-index assignment per K-step of BK: lane group g, MFMA step s
// uses k0 + g*(BK/4) + 8s .. +7 for both operands, so each lane reads BK/2
// contiguous bytes of its weight row per step.
#pragma once

#include "common.h"

template <int MT, int BK>
struct StreamTile {
  static constexpr int CH = 16 * MT;          // rows per chunk
  static constexpr int LDA = BK + 8;          // padded LDS row (bf16)
  static constexpr int S = BK / 32;           // MFMA steps per K-step
  static constexpr int ACH = CH * BK / 8 / 256;  // 16-byte A chunks per thread
  static constexpr int LDS_ELEMS = 2 * CH * LDA;
  static_assert(ACH >= 1, "tile too small for 256 threads");
};

// acc0[mt][r] (and acc1 when GATED) = sum_k A[row][k] * W[k] for
// row = row0 + 16*mt + 4*(lane/16) + r of the chunk, against the lane's
// weight row(s) w0 (w1). A row i of the chunk is A + map(row0 + i) * lda with
// map = rowmap or identity. Rows past nrows repeat the chunk's first row; their
// accumulators are meaningless and must not be stored.
template <int MT, int BK, bool GATED>
__device__ __forceinline__ void stream_tile(const bf16_t* __restrict__ A, int lda,
                                            const int32_t* __restrict__ rowmap, int row0, int nrows,
                                            const bf16_t* __restrict__ w0,
                                            const bf16_t* __restrict__ w1, int K,
                                            f32x4 (&acc0)[MT], f32x4 (&acc1)[MT], bf16_t* lds) {
  using T = StreamTile<MT, BK>;
  constexpr int S = T::S, ACH = T::ACH, LDA = T::LDA, CH = T::CH;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int kl = grp * (BK / 4);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc0[mt] = acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rows past nrows re-read the chunk's first row (branch-free loads; their
  // results are never stored).
  const bf16_t* arow[ACH];
  int aoff[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + 256 * i, r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
    const int rr = r < nrows ? r : 0;
    const int row = rowmap ? rowmap[row0 + rr] : row0 + rr;
    arow[i] = A + (int64_t)row * lda + kc;
    aoff[i] = r * LDA + kc;
  }
  u32x4 ra[ACH];
  u32x4 b0[2][S], b1[2][S];

  auto loadA = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = ld16(arow[i] + k0);
  };
  auto storeA = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(lds + buf * CH * LDA + aoff[i]) = ra[i];
  };
  auto loadB = [&](int buf, int k0) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      b0[buf][s] = ld16(w0 + k0 + kl + 8 * s);
      if (GATED) b1[buf][s] = ld16(w1 + k0 + kl + 8 * s);
    }
  };
  auto compute = [&](int buf) {
    const bf16_t* As = lds + buf * CH * LDA;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = ld16(As + (16 * mt + l16) * LDA + kl + 8 * s);
        acc0[mt] = mfma_bf16(a, b0[buf][s], acc0[mt]);
        if (GATED) acc1[mt] = mfma_bf16(a, b1[buf][s], acc1[mt]);
      }
  };

  const int nk = K / BK;
  loadA(0);
  loadB(0, 0);
  storeA(0);
  __syncthreads();
  for (int it = 0; it < nk; it += 2) {
    const bool more1 = it + 1 < nk;
    if (more1) {
      loadA((it + 1) * BK);
      loadB(1, (it + 1) * BK);
    }
    compute(0);
    if (more1) storeA(1);
    __syncthreads();
    if (!more1) break;
    const bool more2 = it + 2 < nk;
    if (more2) {
      loadA((it + 2) * BK);
      loadB(0, (it + 2) * BK);
    }
    compute(1);
    if (more2) storeA(0);
    __syncthreads();
  }
}

// Locate work item b in a list of groups with exclusive item offsets
// s_items[0..n_groups] (LDS): the group g with s_items[g] <= b < s_items[g+1].
__device__ __forceinline__ int find_group(const int32_t* s_items, int n_groups, int b) {
  int lo = 0, hi = n_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_items[mid] <= b)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}
