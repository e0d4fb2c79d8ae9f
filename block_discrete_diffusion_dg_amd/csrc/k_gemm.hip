// LM head: bf16 GEMM L = h_f E^T on the gfx950 matrix cores whose epilogue
// reduces every row of each tile to (max / argmax / sum of exp / held-token
// logit), so the full-vocabulary softmax is never materialised.
//
// Tile: 256 threads = 4 waves in a 2 (rows) x 2 (cols) grid. A wave owns
// 16*MT rows and four 16-column subtiles interleaved with stride 32
// (columns 16*wn + 32*t + lane%16, t = 0..3), so a work-group covers
// BM = 32*MT rows by BN = 128 columns.
// K advances 64 at a time through padded LDS tiles; the next tile's global
// loads are issued before the current tile's MFMAs.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16) against bank conflicts

template <int MT>
struct Tile {
  static constexpr int BM = 32 * MT;
  static constexpr int LDS_ELEMS = (BM + BN) * LDK;
};

// Map the work-group id to (m-block, n-block). When the n-block count is a
// multiple of 8, the m-blocks of one n-block get ids that differ by 8, so
// they land on the same XCD (dispatch is round-robin over the 8 XCDs) and
// share that XCD's L2 copy of the B tile.
__device__ __forceinline__ void block_coords(int MB, int NB, int& mb, int& nb) {
  const int b = blockIdx.x;
  if (MB == 1) {
    mb = 0;
    nb = b;
  } else if ((NB & 7) == 0) {
    const int x = b & 7, j = b >> 3;
    mb = j % MB;
    nb = (j / MB) * 8 + x;
  } else {
    mb = b % MB;
    nb = b / MB;
  }
}

// Accumulate the (m0, n0) tile of A[M][K] * B[N][K]^T into acc.
// acc[mt][t][r] = C[m0 + wm*16*MT + 16*mt + 4*(lane/16) + r][n0 + 16*wn + 32*t + lane%16].
template <int MT>
__device__ __forceinline__ void gemm_tile(const bf16_t* __restrict__ A, int lda, int M,
                                          const bf16_t* __restrict__ B, int ldb, int N, int K,
                                          int m0, int n0, f32x4 (&acc)[MT][4], bf16_t* lds) {
  constexpr int BM = Tile<MT>::BM;
  bf16_t* As = lds;
  bf16_t* Bs = lds + BM * LDK;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // global -> register staging: A has BM*8 16-byte chunks (MT per thread),
  // B has 128*8 (4 per thread); 8 consecutive threads cover one 128-byte row.
  u32x4 ra[MT], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = (c & 7) * 8;
      const int gm = min(m0 + row, M - 1);  // rows past M repeat the last row (never stored)
      ra[i] = ld16(A + (int64_t)gm * lda + k0 + kc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, col = c >> 3, kc = (c & 7) * 8;
      const int gn = min(n0 + col, N - 1);  // columns past N are excluded by the epilogue
      rb[i] = ld16(B + (int64_t)gn * ldb + k0 + kc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(As + row * LDK + kc) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, col = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(Bs + col * LDK + kc) = rb[i];
    }
  };

  const int nk = K / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a[MT], b[4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[mt] = ld16(As + (wm * 16 * MT + 16 * mt + l16) * LDK + 32 * s + 8 * grp);
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = ld16(Bs + (16 * wn + 32 * t + l16) * LDK + 32 * s + 8 * grp);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_bf16(a[mt], b[t], acc[mt][t]);
    }
  }
}

// LM head: logits never leave registers. Each wave reduces its 64 columns of
// every row to (max, first argmax, sum exp2((L - max) * k2)) with
// k2 = log2(e) / tau, written as partial wn of n-block nb:
// part[row][2*nb + wn]. The lane that holds the column of the row's held
// token writes that logit.
template <int MT>
__global__ __launch_bounds__(256) void gemm_lmhead_kernel(const bf16_t* __restrict__ A, int M, int K,
                                                          const bf16_t* __restrict__ B, int N,
                                                          const int32_t* __restrict__ held,
                                                          float k2, float4* __restrict__ part,
                                                          float* __restrict__ held_logit,
                                                          int held_stride) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int MB = div_up(M, Tile<MT>::BM), NB = div_up(N, BN);
  int mb, nb;
  block_coords(MB, NB, mb, nb);
  const int m0 = mb * Tile<MT>::BM, n0 = nb * BN;
  f32x4 acc[MT][4];
  gemm_tile<MT>(A, K, M, B, K, N, K, m0, n0, acc, lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_parts = 2 * NB;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 16 * MT + 16 * mt + 4 * grp + r;
      float mv = -INFINITY;
      int mi = 0x7fffffff;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = n0 + 16 * wn + 32 * t + l16;
        if (col < N) argmax_merge(mv, mi, acc[mt][t][r], col);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float v2 = __shfl_xor(mv, o, WAVE);
        const int i2 = __shfl_xor(mi, o, WAVE);
        argmax_merge(mv, mi, v2, i2);
      }
      float z = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = n0 + 16 * wn + 32 * t + l16;
        if (col < N) z += exp2f((acc[mt][t][r] - mv) * k2);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, WAVE);
      if (row < M) {
        if (l16 == 0) part[(int64_t)row * n_parts + 2 * nb + wn] = float4{mv, z, __int_as_float(mi), 0.f};
        const int hc = held[row] - n0;
        if (hc >= 0 && hc < BN && ((hc >> 4) & 1) == wn && (hc & 15) == l16) {
          const int t = hc >> 5;
          float hv = acc[mt][0][r];
#pragma unroll
          for (int tt = 1; tt < 4; ++tt)
            if (tt == t) hv = acc[mt][tt][r];
          held_logit[(int64_t)row * held_stride] = hv;
        }
      }
    }
}

template <int MT>
size_t lds_bytes() {
  return (size_t)Tile<MT>::LDS_ELEMS * sizeof(bf16_t);
}

template <int MT>
int grid_for(int M, int N) {
  return div_up(M, Tile<MT>::BM) * div_up(N, BN);
}

}  // namespace

// ---------------------------------------------------------------- launchers

#define DG_MT_DISPATCH(mt, ...)           \
  switch (mt) {                           \
    case 2: { constexpr int MT = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int MT = 4; __VA_ARGS__; } break; \
    default: { constexpr int MT = 8; __VA_ARGS__; } break; \
  }

void launch_gemm_lmhead(hipStream_t s, int mt, const bf16_t* a, int rows, int K, const bf16_t* embed,
                        int V, const int32_t* held, float tau, float4* part, float* held_logit,
                        int held_stride) {
  const float k2 = 1.4426950408889634f / tau;
  DG_MT_DISPATCH(mt, hipLaunchKernelGGL(gemm_lmhead_kernel<MT>, dim3(grid_for<MT>(rows, V)), dim3(256),
                                        lds_bytes<MT>(), s, a, rows, K, embed, V, held, k2, part,
                                        held_logit, held_stride));
}

int lmhead_parts(int V) { return 2 * div_up(V, BN); }
