// LM head: logits L = u E^T on the gfx950 matrix cores (u: the final-normed
// token rows, bf16; E: the tied embedding in the fragment-major layout of
// stream.h), with an epilogue that reduces every row of each 256-column tile
// to (max, first argmax, sum of exp, entropy sum), so the vocabulary-wide
// softmax is never materialised (the statistics the confidence sampler and
// adaptive stopping need: codemajin.net DiffusionGemma explainer §3.3).
//
// A work-group of 512 threads covers 256 token rows x 256 vocabulary
// columns. K advances in 32-wide steps; each step's operands are 32
// fragments of 1 KB (16 token-row blocks, 16 vocabulary blocks), copied
// global -> LDS by the load-to-LDS DMA path into a ring of four distinct LDS
// buffers, three steps ahead of their use. Wave w computes token rows
// 128(w/4) .. +127 against columns 64(w%4) .. +63, reading both operands from
// LDS, so each operand byte is fetched into the compute unit once per tile.
// Why this shape: the launch is bound by how many bytes each compute unit
// keeps in flight (about 2.5 us of load latency at full load), and the ring
// holds 96 KB in flight per compute unit while the 256 x 256 tile halves the
// bytes per product of a 128-row tile. (The load-to-LDS path addresses the
// first 128 KB of LDS only: a fifth buffer placed above that corrupts the
// first one.) Tiles of one column range get work-group ids 8 apart (same XCD)
// when there are several row chunks.
#include "common.h"
#include "kernels.h"
#include "philox.h"
#include "stream.h"

namespace {

constexpr int LM_ROWS = 256, LM_COLS = 256, LM_BK = 32;
constexpr int LM_FRAGS = LM_ROWS / 16 + LM_COLS / 16;  // 1 KB fragments per step

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// The 256 x 256 tile's K loop on the ring of four LDS buffers: acc[nb][mt]
// of wave w = A rows row0 + 128(w/4) + 16mt + 4(lane/16) .. +3 against
// columns 64(w%4) + 16nb + lane%16 of the matrix W, over the nst 32-wide
// K-steps st0 .. st0 + nst - 1. A is row-major with lda (= K) columns; rows
// past nrows repeat the last row.
// bf16 W: fragment-major (pack_index), W points at the tile's first column
// block. W8: FP8 codes in the step-major layout (lm8_index) of a matrix with
// n_w rows, W8 points at the tile's first block inside step 0 (byte c0 * 32),
// w8s at the tile's 256 row scales; each step's 16 blocks are 8 KB of
// consecutive bytes, copied by one load-to-LDS operation per wave, and the
// codes are widened to bf16 times the row scale as they are read.
template <bool W8>
__device__ __forceinline__ void ring_gemm_256(const bf16_t* __restrict__ A, int lda, int row0, int nrows,
                                              const bf16_t* __restrict__ W, const uint8_t* __restrict__ W8b,
                                              const float* __restrict__ w8s, int64_t n_w, int nst, int st0,
                                              f32x4 (&acc)[4][8], u32x4 (&r0)[LM_FRAGS][64],
                                              u32x4 (&r1)[LM_FRAGS][64], u32x4 (&r2)[LM_FRAGS][64],
                                              u32x4 (&r3)[LM_FRAGS][64]) {
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave >> 2, cq = wave & 3;  // the wave's row half and column quarter
  const int K = lda;
  // Fragments of a step: token-row block b at b (lane (g, i) holds row 16b + i,
  // reduction indices 8g .. 8g+7 of the step; rows past the end repeat the
  // last row), column block b at 16 + b (the packed matrix's 512
  // contiguous elements of that block and step; with W8 the 16 blocks' codes
  // fill entries 16 .. 23, 512 bytes a block). Wave w copies token-row
  // blocks w, w + 8 and column blocks w, w + 8 (W8: bytes 1024w .. +1023).
  const bf16_t* const srcA0 = A + (int64_t)(row0 + min(16 * wave + l16, nrows - 1)) * lda + 8 * grp;
  const bf16_t* const srcA1 = A + (int64_t)(row0 + min(16 * (wave + 8) + l16, nrows - 1)) * lda + 8 * grp;
  const bf16_t* const srcW0 = W8 ? nullptr : W + (int64_t)(16 * wave) * K + lane * 8;
  const bf16_t* const srcW1 = W8 ? nullptr : W + (int64_t)(16 * (wave + 8)) * K + lane * 8;
  const uint8_t* const src8 = W8 ? W8b + 1024 * wave + 16 * lane : nullptr;
  float sc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) sc[nb] = W8 ? w8s[16 * (4 * cq + nb) + l16] : 1.0f;
  // steps past the end reload the last step (in bounds; never used), so every
  // step issues the same copies and the wait counts stay static
  auto copy = [&](u32x4 (&buf)[LM_FRAGS][64], int st) {
    st = st0 + min(st, nst - 1);
    const bf16_t* pa0 = srcA0 + st * LM_BK;
    const bf16_t* pa1 = srcA1 + st * LM_BK;
    __builtin_amdgcn_global_load_lds(pa0, (__attribute__((address_space(3))) void*)&buf[wave][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(pa1, (__attribute__((address_space(3))) void*)&buf[wave + 8][0], 16, 0, 0);
    if constexpr (W8) {
      __builtin_amdgcn_global_load_lds(src8 + (int64_t)st * n_w * 32,
                                       (__attribute__((address_space(3))) void*)&buf[16 + wave][0], 16, 0, 0);
    } else {
      const int64_t wo = (int64_t)(st >> 1) * 1024 + (st & 1) * 512;
      __builtin_amdgcn_global_load_lds(srcW0 + wo, (__attribute__((address_space(3))) void*)&buf[16 + wave][0], 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(srcW1 + wo, (__attribute__((address_space(3))) void*)&buf[24 + wave][0], 16,
                                       0, 0);
    }
  };
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&buf)[LM_FRAGS][64]) {
    u32x4 wf[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if constexpr (W8) {
        const int b = 4 * cq + nb;  // block b: bytes 512b .. of entries 16 ..
        const u32x2 c = reinterpret_cast<const u32x2*>(&buf[16][0])[64 * b + lane];
        wf[nb] = widen_fp8(c.x, c.y, sc[nb]);
      } else {
        wf[nb] = buf[16 + 4 * cq + nb][lane];
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const u32x4 af = buf[8 * rh + mt][lane];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb][mt] = mfma_bf16(af, wf[nb], acc[nb][mt]);
    }
  };
  // Step st: wait until this wave's copies of step st have landed (the two
  // later steps' copies may still be in flight: four per step, three with
  // W8), then a barrier without a memory fence (a fence would wait for every
  // copy in flight): after it, every wave's copies of step st are in place
  // and every wave has finished step st - 1, whose buffer the next copy
  // reuses.
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(W8 ? 6 : 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  copy(r0, 0);
  copy(r1, 1);
  copy(r2, 2);
  for (int st = 0; st < nst; st += 4) {
    sync();
    copy(r3, st + 3);
    compute(r0);
    sync();
    copy(r0, st + 4);
    compute(r1);
    sync();
    copy(r1, st + 5);
    compute(r2);
    sync();
    copy(r2, st + 6);
    compute(r3);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// part[row][nt] = (max, sum 2^t, first argmax bits, sum 2^t t) over the 256
// columns of tile nt, t = (L - max) * k2, k2 = log2(e) / tau; the lane holding the column
// of the row's held token writes that logit to held_logit[row * held_stride].
// Requires K % 128 == 0 and V % 256 == 0 (the configuration check enforces
// d % 256 == 0 and V % 256 == 0).
// With GUMBEL the epilogue also draws each row's sampled candidate over the
// tile: the column with the largest L / tau + G (G the Gumbel noise of the
// row's canvas position and that column, lowest column on ties) goes to
// gpart[row][nt] = (key, column bits, its logit, 0).
// With SC (self-conditioning) the epilogue also writes, for every row and
// 64-column quarter of the tile, p_v = exp(L_v - m) (bf16, temperature 1, m
// the quarter's maximum) to sc.p[row][v] and (m, sum of p_v in fp32) to
// sc.qpart[row][v / 64]: the unnormalised predicted distribution that
// sc_norm_kernel normalises.
// With W8 the embedding is read as FP8 codes (lm8_index layout) with row
// scales instead (the tied LM head's weights at reduced precision).
template <bool GUMBEL, bool SC, bool W8>
__global__ __launch_bounds__(512) void lmhead_kernel(const bf16_t* __restrict__ A, int rows, int K,
                                                     const bf16_t* __restrict__ E, int V,
                                                     const int32_t* __restrict__ held, float k2,
                                                     float4* __restrict__ part, float* __restrict__ held_logit,
                                                     int held_stride, GumbelDraw gd, SelfCondOut sc, LmFp8 e8) {
  // four distinct objects: the compiler then orders each buffer's LDS reads
  // only after the copies into that buffer
  __shared__ __align__(16) u32x4 r0[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r1[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r2[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r3[LM_FRAGS][64];
  const int NT = V / LM_COLS, MC = div_up(rows, LM_ROWS);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave >> 2, cq = wave & 3;  // the wave's row half and column quarter
  const int row0 = mc * LM_ROWS, nrows = min(LM_ROWS, rows - row0);
  const int c0 = nt * LM_COLS;

  f32x4 acc[4][8];  // [column block][row block] of the wave
  ring_gemm_256<W8>(A, K, row0, nrows, E + (int64_t)c0 * K, W8 ? e8.codes + (int64_t)c0 * 32 : nullptr,
                    W8 ? e8.scale + c0 : nullptr, V, K / LM_BK, 0, acc, r0, r1, r2, r3);

  // Epilogue in the ring's memory: red[4][256] (max, sum, argmax, entropy
  // sum) per column quarter and row, and the rows' held tokens.
  float4* red = reinterpret_cast<float4*>(&r0[0][0]);
  int* s_held = reinterpret_cast<int*>(&r1[0][0]);
  if (tid < LM_ROWS) s_held[tid] = tid < nrows ? held[row0 + tid] : -1;
  // Per row (128rh + 16mt + 4grp + r), over the wave's 64 columns
  // (cw + 16nb + l16): max, the smallest column holding it,
  // sum 2^t and sum 2^t t with t = (L - max) k2, on the DPP network. All rows
  // are reduced first (independent chains), then the held-token logits are
  // picked out.
  const int cw = c0 + 64 * cq;
  float m[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      m[mt][r] = row16_max(fmaxf(fmaxf(acc[0][mt][r], acc[1][mt][r]), fmaxf(acc[2][mt][r], acc[3][mt][r])));
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int ix = 0x7fffffff;
      float z = 0.f, zt = 0.f;
#pragma unroll
      for (int nb = 3; nb >= 0; --nb) {
        const float v = acc[nb][mt][r];
        if (v == m[mt][r]) ix = cw + 16 * nb + l16;
        const float t = (v - m[mt][r]) * k2, e = __builtin_amdgcn_exp2f(t);
        z += e;
        zt = fmaf(e, t, zt);
      }
      ix = row16_min(ix);
      z = row16_sum(z);
      zt = row16_sum(zt);
      if (l16 == 0)
        red[cq * LM_ROWS + 128 * rh + 16 * mt + 4 * grp + r] = float4{m[mt][r], z, __int_as_float(ix), zt};
    }
  if constexpr (SC) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 128 * rh + 16 * mt + 4 * grp + r;
        float z1 = 0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float pv = __builtin_amdgcn_exp2f((acc[nb][mt][r] - m[mt][r]) * 1.4426950408889634f);
          z1 += pv;
          if (row < rows) sc.p[(int64_t)row * V + cw + 16 * nb + l16] = f2bf(pv);
        }
        z1 = row16_sum(z1);
        if (l16 == 0 && row < rows) sc.qpart[(int64_t)row * (V / 64) + (cw >> 6)] = float2{m[mt][r], z1};
      }
  }
  float4* red2 = reinterpret_cast<float4*>(&r2[0][0]);  // [4][256] sampled-candidate partials
  if constexpr (GUMBEL) {
    // one Philox call per (lane, row) gives the noise of the lane's four
    // columns cw + 16 nb + l16: they share the counter, word nb each
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = 128 * rh + 16 * mt + 4 * grp + r;
        const int rowc = min(row0 + rl, rows - 1);
        const int rq = rowc / gd.C, pos = rowc - rq * gd.C;
        const u32x4 wd = philox4x32_10((uint32_t)(cw + l16), (uint32_t)pos,
                                       ((uint32_t)gd.st.block[rq] << 16) | (uint32_t)gd.step,
                                       0x80000000u | (uint32_t)gd.st.slot[rq], gd.st.key_lo[rq], gd.st.key_hi[rq]);
        float best = -INFINITY, bl = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float key = acc[nb][mt][r] * gd.k1 + gumbel_of_word(wd[nb]);
          if (key > best) {
            best = key;
            bi = cw + 16 * nb + l16;
            bl = acc[nb][mt][r];
          }
        }
        const float mk = row16_max(best);
        const int ci = row16_min(best == mk ? bi : 0x7fffffff);
        const float lg = row16_max(bi == ci ? bl : -INFINITY);
        if (l16 == 0) red2[cq * LM_ROWS + rl] = float4{mk, __int_as_float(ci), lg, 0.f};
      }
  }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = 128 * rh + 16 * mt + 4 * grp + r;
      const int hc = s_held[rl] - cw;
      if (hc >= 0 && hc < 64 && (hc & 15) == l16) {
        float hv = acc[0][mt][r];
#pragma unroll
        for (int nb = 1; nb < 4; ++nb)
          if (nb == (hc >> 4)) hv = acc[nb][mt][r];
        held_logit[(int64_t)(row0 + rl) * held_stride] = hv;
      }
    }
  if (tid < nrows) {
    // merge the four column quarters in column order: the first holding the
    // maximum also holds its smallest column
    float4 p = red[tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      // a partial shifted down by d (= (max - new max) k2 <= 0) scales its
      // sums by 2^d and its entropy sum picks up d times its sum
      const float4 o = red[w * LM_ROWS + tid];
      if (o.x > p.x) {
        const float d = (p.x - o.x) * k2, f = __builtin_amdgcn_exp2f(d);
        p.w = o.w + f * fmaf(d, p.y, p.w);
        p.y = o.y + p.y * f;
        p.x = o.x;
        p.z = o.z;
      } else {
        const float d = (o.x - p.x) * k2, f = __builtin_amdgcn_exp2f(d);
        p.w += f * fmaf(d, o.y, o.w);
        p.y += o.y * f;
      }
    }
    part[(int64_t)(row0 + tid) * NT + nt] = p;
    if constexpr (GUMBEL) {
      // column quarters in column order: a later quarter wins only with a larger key
      float4 g = red2[tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 o = red2[w * LM_ROWS + tid];
        if (o.x > g.x) g = o;
      }
      gd.gpart[(int64_t)(row0 + tid) * NT + nt] = g;
    }
  }
}

// Self-conditioning contraction over the vocabulary, split over K:
// part[split][row][col] = sum over v in the split's range of P[row][v] ET[col][v],
// P the normalised predicted distribution (bf16 [rows][V]), ET the tied
// embedding transposed ([d][V], fragment-major). Work-group (column tile nt
// of 256, split) of a grid of (d/256) x nsplit; each split covers nst
// 32-wide steps of V.
__global__ __launch_bounds__(512) void sc_gemm_kernel(const bf16_t* __restrict__ P, int rows, int V,
                                                      const bf16_t* __restrict__ ET, int d, int nst,
                                                      float* __restrict__ part) {
  __shared__ __align__(16) u32x4 r0[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r1[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r2[LM_FRAGS][64];
  __shared__ __align__(16) u32x4 r3[LM_FRAGS][64];
  const int NT = d / LM_COLS;
  const int nt = blockIdx.x % NT, split = blockIdx.x / NT;
  const int lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rh = wave >> 2, cq = wave & 3;
  const int c0 = nt * LM_COLS;
  for (int row0 = 0; row0 < rows; row0 += LM_ROWS) {
    const int nrows = min(LM_ROWS, rows - row0);
    f32x4 acc[4][8];
    ring_gemm_256<false>(P, V, row0, nrows, ET + (int64_t)c0 * V, nullptr, nullptr, 0, nst, split * nst, acc, r0, r1,
                         r2, r3);
    float* out = part + (int64_t)split * rows * d;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 128 * rh + 16 * mt + 4 * grp + r;
        if (row < rows)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) out[(int64_t)row * d + c0 + 64 * cq + 16 * nb + l16] = acc[nb][mt][r];
      }
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers

int sc_gemm_splits(int V) {
  // enough splits for about one work-group per compute unit at d = 2048;
  // each split a multiple of four 32-wide steps (the ring's unrolled loop)
  int ns = 32;
  while (ns > 1 && (V / 32) % (4 * ns)) ns >>= 1;
  return ns;
}

void launch_sc_gemm(hipStream_t s, const bf16_t* p, int rows, int V, const bf16_t* et, int d, float* part) {
  const int ns = sc_gemm_splits(V);
  const int nst = V / 32 / ns;
  hipLaunchKernelGGL(sc_gemm_kernel, dim3((d / LM_COLS) * ns), dim3(512), 0, s, p, rows, V, et, d, nst, part);
}

int lmhead_parts(int V) { return V / LM_COLS; }

void launch_lmhead(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* embed, int V,
                   const int32_t* held, float tau, float4* part, float* held_logit, int held_stride,
                   const GumbelDraw* gumbel, const SelfCondOut* sc, const LmFp8* fp8) {
  const float k2 = 1.4426950408889634f / tau;
  const int NT = V / LM_COLS;
  const dim3 grid(NT * div_up(rows, LM_ROWS));
  const GumbelDraw gd = gumbel ? *gumbel : GumbelDraw{};
  const SelfCondOut so = sc ? *sc : SelfCondOut{};
  const LmFp8 e8 = fp8 ? *fp8 : LmFp8{};
#define DG_LMHEAD(G_, S_, W_)                                                                                  \
  hipLaunchKernelGGL((lmhead_kernel<G_, S_, W_>), grid, dim3(512), 0, s, a, rows, K, embed, V, held, k2, part, \
                     held_logit, held_stride, gd, so, e8)
#define DG_LMHEAD_W(G_, S_)   \
  if (fp8)                    \
    DG_LMHEAD(G_, S_, true);  \
  else                        \
    DG_LMHEAD(G_, S_, false)
  if (gumbel && sc) {
    DG_LMHEAD_W(true, true);
  } else if (gumbel) {
    DG_LMHEAD_W(true, false);
  } else if (sc) {
    DG_LMHEAD_W(false, true);
  } else {
    DG_LMHEAD_W(false, false);
  }
#undef DG_LMHEAD_W
#undef DG_LMHEAD
}
