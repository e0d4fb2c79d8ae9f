// Dense projections of a layer on the weight-streaming tile (stream.h), with
// fragment-major packed weights:
//   QKV + RoPE: every lane owns a rotate-half pair (head row j and j + dh/2)
//     as the tile's two weight rows, so the rotation is lane-local; a wave's
//     16 pairs are two 16-row blocks (dh/2 is a multiple of 16). q goes to
//     the workspace, k (rotated) and v to the request's KV-cache rows.
//   output projection: h[row][col] += (o W_o^T)[row][col].
// All token rows form one group cut into chunks of 16*MT rows; the chunks
// of one column tile get work-group ids 8 apart (same XCD, shared L2 copy of
// the weight tile) when the tile count is a multiple of 8.
//
// Two tile forms. The streaming tile (stream.h) walks K in 64-wide steps,
// one after another, with a barrier per step; at a few hundred token rows
// and K = 2048 that chain of 32 dependent steps, not bandwidth, sets the
// launch time. The split-K form (used when K / 256 is 1, 2, 4 or 8) gives
// each of the four waves of a work-group its own quarter of K over the same
// 32 rows x 64 weight rows: both operands go straight from global memory into
// registers, three steps ahead, with no LDS and no barrier in the K loop,
// and the four partial tiles are added through LDS in wave order
// (deterministic). The streaming form stays for other K.
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace {

constexpr int DMT = 2;  // rows per chunk = 32
// These launches give about one work-group per compute unit and little
// matrix-core work per K-step, so each keeps its weights and its token rows
// five steps ahead instead of relying on other work-groups to hide latency.
constexpr int DENSE_DW = 5;

// ---------------------------------------------------------------- split-K form
constexpr int SK_MT = 2, SK_NB = 4, SK_DW = 3;
constexpr int SK_ROWS = 16 * SK_MT, SK_COLS = 16 * SK_NB;
constexpr int SK_RS = SK_COLS + 4;  // padded LDS row: the four lane groups of a store hit distinct banks

// acc[nb][mt][r] = sum over this wave's quarter of K (NST steps of 64) of
// A[row][k] * W_nb[n][k], row = row0 + 16mt + 4(lane/16) + r of the chunk
// (rows past nrows repeat the chunk's last row), n = lane % 16 of block
// w[nb] (fragment-major, see stream.h). K = 4 * 64 * NST.
template <int NST>
__device__ __forceinline__ void splitk_tile(const bf16_t* __restrict__ A, int lda, int row0, int nrows,
                                            const bf16_t* const (&w)[SK_NB], f32x4 (&acc)[SK_NB][SK_MT]) {
  constexpr int NR = SK_DW + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  const int kb = wave * NST * 64;
  const bf16_t* arow[SK_MT];
#pragma unroll
  for (int mt = 0; mt < SK_MT; ++mt)
    arow[mt] = A + (int64_t)(row0 + min(16 * mt + l16, nrows - 1)) * lda + kb + 8 * grp;
  const bf16_t* wl[SK_NB];
#pragma unroll
  for (int nb = 0; nb < SK_NB; ++nb) wl[nb] = w[nb] + kb * 16 + lane * 8;
  u32x4 ra[NR][SK_MT][2], rb[NR][SK_NB][2];
#pragma unroll
  for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < SK_MT; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto issue = [&](int set, int st) {
    const int k0 = st * 64;
#pragma unroll
    for (int mt = 0; mt < SK_MT; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) ra[set][mt][q] = ld16(arow[mt] + k0 + 32 * q);
#pragma unroll
    for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
      for (int q = 0; q < 2; ++q) rb[set][nb][q] = ld16(wl[nb] + k0 * 16 + q * 512);
  };
  // The scheduling barriers keep every step's loads issued SK_DW steps
  // before their use (left alone, the scheduler sinks them towards the
  // products to save registers, and the pipeline collapses).
#pragma unroll
  for (int j = 0; j < SK_DW && j < NST; ++j) issue(j, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    if (st + SK_DW < NST) issue((st + SK_DW) % NR, st + SK_DW);
    __builtin_amdgcn_sched_barrier(0);
    const int set = st % NR;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mt = 0; mt < SK_MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < SK_NB; ++nb) acc[nb][mt] = mfma_bf16(ra[set][mt][q], rb[set][nb][q], acc[nb][mt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The wave's partial tile -> red[wave][row][col] (fp32, SK_RS floats a row).
__device__ __forceinline__ void splitk_stage(const f32x4 (&acc)[SK_NB][SK_MT], float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < SK_MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * SK_ROWS + 16 * mt + 4 * grp + r) * SK_RS + 16 * nb + l16] = acc[nb][mt][r];
}

// Columns col .. col+3 of tile row rr, the four waves' partials added in wave order.
__device__ __forceinline__ float4 splitk_sum4(const float* red, int rr, int col) {
  float4 v = *reinterpret_cast<const float4*>(red + rr * SK_RS + col);
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float4 o = *reinterpret_cast<const float4*>(red + (w * SK_ROWS + rr) * SK_RS + col);
    v.x += o.x;
    v.y += o.y;
    v.z += o.z;
    v.w += o.w;
  }
  return v;
}

struct QkvArgs {
  bf16_t* q;  // [rows][Hq*dh]
  KvGeom kv;
  int layer, Hq, Hkv, dh;
  const float2* rope;  // [rows][dh/2] (cos, sin)
  ReqTable rt;
  int32_t* sync;  // arrival counters of the layer's router and attention, zeroed here
  int n_sync;
};

__global__ __launch_bounds__(256) void qkv_kernel(const bf16_t* __restrict__ u, int rows, int d,
                                                  const bf16_t* __restrict__ w, QkvArgs p) {
  using T = StreamTile<DMT>;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  if (blockIdx.x == 0 && p.sync)
    for (int i = threadIdx.x; i < p.n_sync; i += 256) p.sync[i] = 0;
  const int dh = p.dh, half = dh >> 1;
  const int NT = (p.Hq + 2 * p.Hkv) * half / 64, MC = div_up(rows, T::CH);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  const int pw = nt * 64 + wave * 16;  // the wave's first pair
  const int head = pw / half, j = pw % half + l16;
  const int64_t r0 = (int64_t)head * dh + pw % half;  // first row of the wave's block
  const int row0 = mc * T::CH, nrows = min(T::CH, rows - row0);
  f32x4 a0[DMT], a1[DMT];
  stream_tile<DMT, true, DENSE_DW, DENSE_DW>(u, d, nullptr, row0, nrows, w + r0 * d, w + (r0 + half) * d, nullptr,
                                             nullptr, d, a0, a1, lds);
  const bool rotate = head < p.Hq + p.Hkv;
#pragma unroll
  for (int mt = 0; mt < DMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * mt + 4 * grp + r;
      if (row >= rows) continue;
      float x1 = a0[mt][r], x2 = a1[mt][r];
      if (rotate) {
        const float2 cs = p.rope[(int64_t)row * half + j];
        const float y1 = x1 * cs.x - x2 * cs.y;
        const float y2 = x2 * cs.x + x1 * cs.y;
        x1 = y1;
        x2 = y2;
      }
      if (head < p.Hq + p.Hkv) {
        bf16_t* dst;
        if (head < p.Hq) {
          dst = p.q + (int64_t)row * p.Hq * dh + (int64_t)head * dh;
        } else {
          const int rq = row / p.rt.rows_per_req, i = row % p.rt.rows_per_req;
          dst = p.kv.k_plane(p.rt.slot[rq], p.layer, head - p.Hq) + (int64_t)(p.rt.pos0[rq] + i) * dh;
        }
        dst[j] = f2bf(x1);
        dst[j + half] = f2bf(x2);
      } else {  // V: matrix-core operand order inside 32-key blocks
        const int rq = row / p.rt.rows_per_req, i = row % p.rt.rows_per_req;
        const int64_t pos = p.rt.pos0[rq] + i;
        bf16_t* vp = p.kv.v_plane(p.rt.slot[rq], p.layer, head - p.Hq - p.Hkv);
        vp[v_index(pos, j, dh)] = f2bf(x1);
        vp[v_index(pos, j + half, dh)] = f2bf(x2);
      }
    }
}

// h[row][col] += (A W^T)[row][col]; with ss, also the sum over the
// work-group's 64 columns of the updated h[row][col]^2 -> ss[nt][row] (the
// MoE pre-norm then needs no second pass over whole rows).
__global__ __launch_bounds__(256) void resid_kernel(const bf16_t* __restrict__ a, int rows, int K,
                                                    const bf16_t* __restrict__ w, int N,
                                                    float* __restrict__ h, float* __restrict__ ss) {
  using T = StreamTile<DMT>;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  __shared__ float red[4][T::CH];
  const int NT = N / 64, MC = div_up(rows, T::CH);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  const int col0 = nt * 64 + wave * 16, col = col0 + l16;
  const int row0 = mc * T::CH, nrows = min(T::CH, rows - row0);
  f32x4 acc[DMT], unused[DMT];
  stream_tile<DMT, false, DENSE_DW, DENSE_DW>(a, K, nullptr, row0, nrows, w + (int64_t)col0 * K, nullptr, nullptr,
                                              nullptr, K, acc, unused, lds);
#pragma unroll
  for (int mt = 0; mt < DMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * mt + 4 * grp + r;
      float sq = 0.f;
      if (row < rows) {
        const float v = h[(int64_t)row * N + col] + acc[mt][r];
        h[(int64_t)row * N + col] = v;
        sq = v * v;
      }
      // sum over the wave's 16 columns (the lanes of one DPP row)
      sq = row16_sum(sq);
      if (l16 == 0) red[wave][16 * mt + 4 * grp + r] = sq;
    }
  if (!ss) return;
  __syncthreads();
  if (threadIdx.x < T::CH && row0 + (int)threadIdx.x < rows) {
    const int i = threadIdx.x;
    ss[(int64_t)nt * rows + row0 + i] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
  }
}

// Split-K QKV + RoPE: a work-group covers 32 token rows x 32 rotate-half
// pairs (pairs p .. p+15 and p+16 .. p+31 of one head, each as its two
// 16-row weight blocks j and j + dh/2); same outputs as qkv_kernel.
template <int NST>
__global__ __launch_bounds__(256) void qkv_sk_kernel(const bf16_t* __restrict__ u, int rows, int d,
                                                     const bf16_t* __restrict__ w, QkvArgs p) {
  __shared__ __align__(16) float red[4 * SK_ROWS * SK_RS];
  if (blockIdx.x == 0 && p.sync)
    for (int i = threadIdx.x; i < p.n_sync; i += 256) p.sync[i] = 0;
  const int dh = p.dh, half = dh >> 1;
  const int NT = (p.Hq + 2 * p.Hkv) * half / 32, MC = div_up(rows, SK_ROWS);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int pw = nt * 32;  // the work-group's first pair
  const int head = pw / half, j0 = pw % half;
  const int64_t r0 = (int64_t)head * dh + j0;  // first weight row
  const int row0 = mc * SK_ROWS, nrows = min(SK_ROWS, rows - row0);
  const bf16_t* const wb[SK_NB] = {w + r0 * d, w + (r0 + half) * d, w + (r0 + 16) * d, w + (r0 + 16 + half) * d};
  f32x4 acc[SK_NB][SK_MT];
  splitk_tile<NST>(u, d, row0, nrows, wb, acc);
  splitk_stage(acc, red);
  __syncthreads();
  // thread -> tile row rr, pairs pq .. pq+3 (columns of block 2(pq/16) and
  // the partner block after it)
  const int rr = threadIdx.x >> 3, pq = (threadIdx.x & 7) * 4;
  const int row = row0 + rr;
  if (row >= rows) return;
  const int c1 = (pq >> 4) * 32 + (pq & 15);
  const float4 v1 = splitk_sum4(red, rr, c1), v2 = splitk_sum4(red, rr, c1 + 16);
  float x1[4] = {v1.x, v1.y, v1.z, v1.w}, x2[4] = {v2.x, v2.y, v2.z, v2.w};
  const int j = j0 + pq;
  if (head < p.Hq + p.Hkv) {
    const float4* cs4 = reinterpret_cast<const float4*>(p.rope + (int64_t)row * half + j);
    const float4 ca = cs4[0], cb = cs4[1];
    const float cs[4][2] = {{ca.x, ca.y}, {ca.z, ca.w}, {cb.x, cb.y}, {cb.z, cb.w}};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y1 = x1[i] * cs[i][0] - x2[i] * cs[i][1];
      const float y2 = x2[i] * cs[i][0] + x1[i] * cs[i][1];
      x1[i] = y1;
      x2[i] = y2;
    }
    bf16_t* dst;
    if (head < p.Hq) {
      dst = p.q + (int64_t)row * p.Hq * dh + (int64_t)head * dh;
    } else {
      const int rq = row / p.rt.rows_per_req, i = row % p.rt.rows_per_req;
      dst = p.kv.k_plane(p.rt.slot[rq], p.layer, head - p.Hq) + (int64_t)(p.rt.pos0[rq] + i) * dh;
    }
    *reinterpret_cast<u32x2*>(dst + j) = u32x2{pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
    *reinterpret_cast<u32x2*>(dst + j + half) = u32x2{pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3])};
  } else {  // V: matrix-core operand order inside 32-key blocks
    const int rq = row / p.rt.rows_per_req, i = row % p.rt.rows_per_req;
    const int64_t pos = p.rt.pos0[rq] + i;
    bf16_t* vp = p.kv.v_plane(p.rt.slot[rq], p.layer, head - p.Hq - p.Hkv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vp[v_index(pos, j + e, dh)] = f2bf(x1[e]);
      vp[v_index(pos, j + e + half, dh)] = f2bf(x2[e]);
    }
  }
}

// Split-K output projection: h[row][col] += (A W^T)[row][col] on a tile of
// 32 rows x 64 columns, with the same per-64-column sums of squares as
// resid_kernel.
template <int NST>
__global__ __launch_bounds__(256) void resid_sk_kernel(const bf16_t* __restrict__ a, int rows, int K,
                                                       const bf16_t* __restrict__ w, int N, float* __restrict__ h,
                                                       float* __restrict__ ss) {
  __shared__ __align__(16) float red[4 * SK_ROWS * SK_RS];
  const int NT = N / SK_COLS, MC = div_up(rows, SK_ROWS);
  int nt, mc;
  xcd_tile_coords(NT, MC, nt, mc);
  const int col0 = nt * SK_COLS;
  const int row0 = mc * SK_ROWS, nrows = min(SK_ROWS, rows - row0);
  const bf16_t* const wb[SK_NB] = {w + (int64_t)col0 * K, w + (int64_t)(col0 + 16) * K, w + (int64_t)(col0 + 32) * K,
                                   w + (int64_t)(col0 + 48) * K};
  f32x4 acc[SK_NB][SK_MT];
  splitk_tile<NST>(a, K, row0, nrows, wb, acc);
  splitk_stage(acc, red);
  __syncthreads();
  // thread -> tile row rr, columns cc .. cc+7; the row's 8 threads are
  // consecutive lanes (half a DPP row)
  const int rr = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 8;
  const int row = row0 + rr;
  float sq = 0.f;
  if (row < rows) {
    float4* hp = reinterpret_cast<float4*>(h + (int64_t)row * N + col0 + cc);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float4 v = splitk_sum4(red, rr, cc + 4 * i);
      float4 x = hp[i];
      x.x += v.x;
      x.y += v.y;
      x.z += v.z;
      x.w += v.w;
      hp[i] = x;
      sq += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
    }
  }
  if (!ss) return;
  sq += dpp_movf<DPP_XOR1>(sq);
  sq += dpp_movf<DPP_XOR2>(sq);
  sq += dpp_movf<DPP_HALF_MIRROR>(sq);
  if ((threadIdx.x & 7) == 0 && row < rows) ss[(int64_t)nt * rows + row] = sq;
}

}  // namespace

void launch_qkv(hipStream_t s, const bf16_t* u, int rows, int d, const bf16_t* w, bf16_t* q,
                const KvGeom& kv, int layer, int Hq, int Hkv, int dh, const float2* rope,
                const ReqTable& rt, int32_t* sync, int n_sync) {
  QkvArgs p{q, kv, layer, Hq, Hkv, dh, rope, rt, sync, n_sync};
  const int nst = d % 256 == 0 ? d / 256 : 0;
  if ((dh / 2) % 32 == 0 && (nst == 1 || nst == 2 || nst == 4 || nst == 8)) {
    const int grid = (Hq + 2 * Hkv) * (dh / 2) / 32 * div_up(rows, SK_ROWS);
#define DG_QKV_SK(NST_) hipLaunchKernelGGL(qkv_sk_kernel<NST_>, dim3(grid), dim3(256), 0, s, u, rows, d, w, p)
    if (nst == 1)
      DG_QKV_SK(1);
    else if (nst == 2)
      DG_QKV_SK(2);
    else if (nst == 4)
      DG_QKV_SK(4);
    else
      DG_QKV_SK(8);
#undef DG_QKV_SK
    return;
  }
  const int NT = (Hq + 2 * Hkv) * (dh / 2) / 64;
  const int MC = div_up(rows, StreamTile<DMT>::CH);
  hipLaunchKernelGGL(qkv_kernel, dim3(NT * MC), dim3(256), 0, s, u, rows, d, w, p);
}

void launch_resid(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* w, int N, float* h, float* ss) {
  const int nst = K % 256 == 0 ? K / 256 : 0;
  if (N % SK_COLS == 0 && (nst == 1 || nst == 2 || nst == 4 || nst == 8)) {
    const int grid = (N / SK_COLS) * div_up(rows, SK_ROWS);
#define DG_RESID_SK(NST_) \
  hipLaunchKernelGGL(resid_sk_kernel<NST_>, dim3(grid), dim3(256), 0, s, a, rows, K, w, N, h, ss)
    if (nst == 1)
      DG_RESID_SK(1);
    else if (nst == 2)
      DG_RESID_SK(2);
    else if (nst == 4)
      DG_RESID_SK(4);
    else
      DG_RESID_SK(8);
#undef DG_RESID_SK
    return;
  }
  const int MC = div_up(rows, StreamTile<DMT>::CH);
  hipLaunchKernelGGL(resid_kernel, dim3((N / 64) * MC), dim3(256), 0, s, a, rows, K, w, N, h, ss);
}
