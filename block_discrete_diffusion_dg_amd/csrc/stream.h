// Weight-streaming tile for skinny GEMMs on the gfx950 matrix cores.
//
// In a denoising step every weight matrix meets at most a few hundred token
// rows, so the weights are read from HBM once (straight into MFMA B
// operands, no LDS) while the token rows ride along. A work-group covers a
// chunk of CH = 16*MT rows against 64 weight rows (16 per wave); with
// GATED the lane also owns a second weight row (the "up" row of a SwiGLU, or
// the rotate-half partner of a RoPE pair) and a second accumulator.
//
// Weights are in the fragment-major layout (see pack_index below): the 16
// rows a wave owns form one contiguous block, and each K-step of that block
// is 2 KB in the exact order the lanes consume it, so every weight load of a
// wave is one fully used, contiguous 1 KB request.
//
// Pipeline: K advances in steps of BK = 64. Loads run two steps ahead of the
// matrix cores: while step it is multiplied, the loads of steps it+1 and
// it+2 are in flight (three register sets for the weights and for the A
// staging; a double-buffered LDS tile for A, shared by the four waves). The
// loop is unrolled by three so every register set has a static index; steps
// past the end reload the last step (in-bounds, branch-free) and their
// weight operands are zeroed, so the matrix-core instructions never sit under
// control flow.
//
// Reduction-index assignment per K-step: MFMA step q in {0,1}, lane group g
// uses k0 + 32q + 8g .. +7 for both operands.
#pragma once

#include <type_traits>

#include "common.h"

template <int MT>
struct StreamTile {
  static constexpr int BK = 64;
  static constexpr int CH = 16 * MT;             // rows per chunk
  static constexpr int LDA = BK + 8;             // padded LDS row (bf16)
  static constexpr int ACH = CH * BK / 8 / 256;  // 16-byte A chunks per thread and step
  static constexpr int LDS_ELEMS = 2 * CH * LDA;
  static_assert(ACH >= 1, "tile too small for 256 threads");
};

// Fragment-major index of W[n][k] for a [N][K] matrix (N % 16 == 0,
// K % 64 == 0): block n/16 of 16 rows is contiguous (16*K elements); inside
// it, K-step k/64 is 1024 elements ordered [q][lane][8] with
// q = (k%64)/32, lane = 16*((k%32)/8) + n%16 and element k%8.
__host__ __device__ __forceinline__ int64_t pack_index(int64_t n, int64_t k, int64_t K) {
  const int64_t kk = k & 63;
  return (n >> 4) * 16 * K + (k >> 6) * 1024 + (kk >> 5) * 512 + (((kk & 31) >> 3) * 16 + (n & 15)) * 8 +
         (kk & 7);
}

// acc0[mt][r] (and acc1 when GATED) = sum_k A[row][k] * W[n][k] for
// row = row0 + 16*mt + 4*(lane/16) + r of the chunk and n = the lane's weight
// row: lane l16 of the wave's 16-row block(s) w0 (w1), packed fragment-major
// (w0 = packed matrix + 16*K * block index). A row i of the chunk is
// A + map(row0 + i) * lda with map = rowmap or identity. Rows past nrows
// repeat the chunk's first row; their accumulators are meaningless and must
// not be stored. K % 64 == 0.
template <int MT, bool GATED>
__device__ __forceinline__ void stream_tile(const bf16_t* __restrict__ A, int lda,
                                            const int32_t* __restrict__ rowmap, int row0, int nrows,
                                            const bf16_t* __restrict__ w0,
                                            const bf16_t* __restrict__ w1, int K,
                                            f32x4 (&acc0)[MT], f32x4 (&acc1)[MT], bf16_t* lds) {
  using T = StreamTile<MT>;
  constexpr int BK = T::BK, ACH = T::ACH, LDA = T::LDA, CH = T::CH;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc0[mt] = acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

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
  const int nk = K / BK;
  const bf16_t* wl0 = w0 + lane * 8;
  const bf16_t* wl1 = GATED ? w1 + lane * 8 : nullptr;

  u32x4 ra[3][ACH];
  u32x4 b0[3][2], b1[3][2];

  // A loads first, then weights: the wait for A of the next step (in-order
  // completion) then never waits on weights issued after it.
  auto issue = [&](auto S, int st) {
    constexpr int s = decltype(S)::value;
    const int k0 = min(st, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[s][i] = ld16(arow[i] + k0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      b0[s][q] = ld16(wl0 + k0 * 16 + q * 512);
      if (GATED) b1[s][q] = ld16(wl1 + k0 * 16 + q * 512);
    }
  };
  auto stage = [&](auto S, int buf) {
    constexpr int s = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(lds + buf * CH * LDA + aoff[i]) = ra[s][i];
  };
  auto compute = [&](auto S, int buf, int st) {
    constexpr int s = decltype(S)::value;
    const bool live = st < nk;  // past the end: weight operands zeroed
    const bf16_t* As = lds + buf * CH * LDA;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 bq0 = live ? b0[s][q] : zero;
      const u32x4 bq1 = live ? b1[s][q] : zero;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = ld16(As + (16 * mt + l16) * LDA + 32 * q + 8 * grp);
        acc0[mt] = mfma_bf16(a, bq0, acc0[mt]);
        if (GATED) acc1[mt] = mfma_bf16(a, bq1, acc1[mt]);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  issue(I0{}, 0);
  issue(I1{}, 1);
  stage(I0{}, 0);
  __syncthreads();
  // Step it multiplies LDS buffer it&1 with weight set it%3. Before it, the
  // loads of step it+2 are issued into set (it+2)%3; after it, step it+1's A
  // (set (it+1)%3) moves into LDS buffer (it+1)&1, last read by step it-1.
  for (int it = 0; it < nk; it += 3) {
    issue(I2{}, it + 2);
    compute(I0{}, it & 1, it);
    stage(I1{}, (it + 1) & 1);
    __syncthreads();
    issue(I0{}, it + 3);
    compute(I1{}, (it + 1) & 1, it + 1);
    stage(I2{}, it & 1);
    __syncthreads();
    issue(I1{}, it + 4);
    compute(I2{}, it & 1, it + 2);
    stage(I0{}, (it + 1) & 1);
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
