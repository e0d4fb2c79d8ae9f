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
// Pipeline: K advances in steps of BK = 64. The A rows are loaded DA steps
// ahead (DA + 1 register sets, then a double-buffered LDS tile shared by the
// four waves) and the weights DW steps ahead (DW + 1 register sets). The loop is
// unrolled so every register set has a static index; steps past the end
// reload the last step (in-bounds, branch-free) and their weight operands are
// zeroed, so the matrix-core instructions never sit under control flow.
//
// Reduction-index assignment per K-step: MFMA step q in {0,1}, lane group g
// uses k0 + 32q + 8g .. +7 for both operands.
//
// FP8 weights (W8): OCP E4M3 codes in the fragment-major byte layout of
// pack8_index, with one power-of-two scale per weight row. A lane's 16 bytes
// of a K-step hold its row's 8 codes of MFMA step 0, then the 8 of step 1;
// one 16-byte load per block and step brings them in, and the hardware
// conversion widens them to bf16 times the row scale, which is exact (every
// E4M3 value times a power of two within range is a bf16 value). The
// products and accumulation are then those of the bf16 tile, on half the
// weight bytes.
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

// Byte index of W[n][k] in the FP8 fragment-major layout of an [N][K] matrix
// (N % 16 == 0, K % 64 == 0): block n/16 of 16 rows is contiguous (16*K
// bytes); inside it, K-step k/64 is 1024 bytes ordered [lane][q][8] with
// lane = 16*((k%32)/8) + n%16, q = (k%64)/32 and byte k%8.
__host__ __device__ __forceinline__ int64_t pack8_index(int64_t n, int64_t k, int64_t K) {
  const int64_t kk = k & 63;
  return (n >> 4) * 16 * K + (k >> 6) * 1024 + (((kk & 31) >> 3) * 16 + (n & 15)) * 16 + (kk >> 5) * 8 + (kk & 7);
}

// Byte index of W[n][k] in the step-major FP8 layout of the LM head, for an
// [N][K] matrix (N % 16 == 0, K % 32 == 0): each 32-wide K-step holds all N
// rows (N*32 bytes), every 16-row block of it as 512 bytes ordered [lane][8]
// with lane = 16*((k%32)/8) + n%16 and byte k%8. The 16 blocks one LM-head
// tile streams per step are then 8 KB of consecutive bytes.
__host__ __device__ __forceinline__ int64_t lm8_index(int64_t n, int64_t k, int64_t N) {
  return (k >> 5) * N * 32 + (n >> 4) * 512 + ((((k & 31) >> 3) * 16 + (n & 15)) * 8) + (k & 7);
}

// Eight E4M3 codes (two words) -> eight bf16 values times scale s.
__device__ __forceinline__ u32x4 widen_fp8(uint32_t w0, uint32_t w1, float s) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// acc[nb][mt][r] = sum_k A[row][k] * W_nb[n][k] for row = row0 + 16*mt +
// 4*(lane/16) + r of the chunk and n = the lane's weight row: lane l16 of the
// wave's nb-th 16-row block w[nb], packed fragment-major (a block is the
// packed matrix + 16*K * block index). A row i of the chunk is
// A + map(row0 + i) * lda with map = rowmap or identity. Rows past nrows
// repeat the chunk's first row; their accumulators are meaningless and must
// not be stored. K % 64 == 0.
// NB blocks per wave: each A fragment read from LDS feeds NB products (a
// SwiGLU gate/up pair, a RoPE rotate-half pair, or several output blocks).
// DW / DA: weight loads run DW steps ahead (DW + 1 register sets), A-row
// loads DA steps ahead (DA + 1 sets). Deeper pipelines keep more bytes in
// flight per work-group, which matters when few work-groups share a compute
// unit or when a step has little matrix-core work to hide latency behind.
template <int A_, int B_>
struct Lcm {
  static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
  static constexpr int value = A_ / gcd(A_, B_) * B_;
};

// W8: the blocks hold FP8 codes (pack8_index) and wsc[nb] points at the
// block's 16 row scales; otherwise bf16 (pack_index) and wsc is unused.
// EARLY_W: the first DW steps of weights are issued before the token-row
// indices are read (costs registers; off where the register budget is tight).
template <int MT, int NB, int DW = 2, int DA = 2, bool W8 = false, bool EARLY_W = false>
__device__ __forceinline__ void stream_tile_n(const bf16_t* __restrict__ A, int lda,
                                              const int32_t* __restrict__ rowmap, int row0, int nrows,
                                              const void* const (&w)[NB], const float* const (&wsc)[NB], int K,
                                              f32x4 (&acc)[NB][MT], bf16_t* lds) {
  using T = StreamTile<MT>;
  constexpr int BK = T::BK, ACH = T::ACH, LDA = T::LDA, CH = T::CH;
  constexpr int NW = DW + 1, NA = DA + 1, U = Lcm<NW, NA>::value;
  constexpr int NQ = W8 ? 1 : 2;                  // 16-byte weight loads per block and K-step
  constexpr int STEP_BYTES = W8 ? 1024 : 2048;    // bytes of one K-step of a 16-row block
  static_assert(DW >= 2 && DA >= 2, "loads run at least two steps ahead");
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  const char* wl[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wl[nb] = static_cast<const char*>(w[nb]) + lane * 16;
  u32x4 ra[NA][ACH];
  u32x4 b[NW][NB][NQ];
  // Loads of step st (clamped to the last step) into weight register set sw.
  auto issue_w = [&](int sw, int st) {
    const int64_t off = (int64_t)min(st, nk - 1) * STEP_BYTES;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[sw][nb][q] = ld16(wl[nb] + off + q * 1024);
  };
  // With EARLY_W the first DW steps of weights go out before anything else:
  // they depend on nothing, while the token rows wait for their row indices
  // (a gather through rowmap), so the weight stream starts a memory round
  // trip sooner.
  if constexpr (EARLY_W) {
#pragma unroll
    for (int j = 0; j < DW; ++j) issue_w(j, j);
  }

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
  float sc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) sc[nb] = W8 ? wsc[nb][l16] : 1.0f;

  // Loads of step st (clamped to the last step) into A register set sa. In
  // the loop, A loads go first in each step, so the wait for the next step's
  // A rows (in-order completion) never waits on weights issued after them.
  auto issue_a = [&](int sa, int st) {
    const int k0 = min(st, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[sa][i] = ld16(arow[i] + k0);
  };
  auto stage = [&](int sa, int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(lds + buf * CH * LDA + aoff[i]) = ra[sa][i];
  };
  auto compute = [&](int sw, int buf, int st) {
    const bool live = st < nk;  // past the end: weight operands zeroed
    const bf16_t* As = lds + buf * CH * LDA;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 bq[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // FP8: code 0 is +0, so zeroing the codes zeroes the widened operand
        if constexpr (W8)
          bq[nb] = widen_fp8(live ? b[sw][nb][0][2 * q] : 0u, live ? b[sw][nb][0][2 * q + 1] : 0u, sc[nb]);
        else
          bq[nb] = live ? b[sw][nb][q] : zero;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = ld16(As + (16 * mt + l16) * LDA + 32 * q + 8 * grp);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][mt] = mfma_bf16(a, bq[nb], acc[nb][mt]);
      }
    }
  };

#pragma unroll
  for (int j = 0; j < (DA > DW ? DA : DW); ++j) {
    if (j < DA) issue_a(j, j);
    if (!EARLY_W && j < DW) issue_w(j, j);
  }
  stage(0, 0);
  __syncthreads();
  // Step st multiplies LDS buffer st&1 with weight set st%NW. Before it, the
  // A rows of step st+DA and the weights of step st+DW are issued; after it,
  // step st+1's A rows move into LDS buffer (st+1)&1, last read by step st-1.
  // The loop is unrolled by U (a multiple of both set counts) so every set
  // index is a compile-time constant.
  for (int it = 0; it < nk; it += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int st = it + j;
      issue_a((j + DA) % NA, st + DA);
      issue_w((j + DW) % NW, st + DW);
      compute(j % NW, (it + j) & 1, st);
      stage((j + 1) % NA, (st + 1) & 1);
      __syncthreads();
    }
  }
}

// One weight row per lane (acc0), or with GATED two (acc0 from w0, acc1 from
// w1): the single-block and paired forms of stream_tile_n.
template <int MT, bool GATED, int DW = 2, int DA = 2, bool W8 = false, bool EARLY_W = false>
__device__ __forceinline__ void stream_tile(const bf16_t* __restrict__ A, int lda,
                                            const int32_t* __restrict__ rowmap, int row0, int nrows,
                                            const void* __restrict__ w0, const void* __restrict__ w1,
                                            const float* s0, const float* s1, int K,
                                            f32x4 (&acc0)[MT], f32x4 (&acc1)[MT], bf16_t* lds) {
  if constexpr (GATED) {
    const void* const w[2] = {w0, w1};
    const float* const ws[2] = {s0, s1};
    f32x4 acc[2][MT];
    stream_tile_n<MT, 2, DW, DA, W8, EARLY_W>(A, lda, rowmap, row0, nrows, w, ws, K, acc, lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = acc[0][mt];
      acc1[mt] = acc[1][mt];
    }
  } else {
    const void* const w[1] = {w0};
    const float* const ws[1] = {s0};
    f32x4 acc[1][MT];
    stream_tile_n<MT, 1, DW, DA, W8, EARLY_W>(A, lda, rowmap, row0, nrows, w, ws, K, acc, lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc0[mt] = acc[0][mt];
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
