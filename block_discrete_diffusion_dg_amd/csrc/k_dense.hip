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
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace {

constexpr int DMT = 2;  // rows per chunk = 32
// These launches give about one work-group per compute unit and little
// matrix-core work per K-step, so each keeps its weights and its token rows
// five steps ahead instead of relying on other work-groups to hide latency.
constexpr int DENSE_DW = 5;

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
  stream_tile<DMT, true, DENSE_DW, DENSE_DW>(u, d, nullptr, row0, nrows, w + r0 * d, w + (r0 + half) * d, d, a0, a1, lds);
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
  stream_tile<DMT, false, DENSE_DW, DENSE_DW>(a, K, nullptr, row0, nrows, w + (int64_t)col0 * K, nullptr, K, acc, unused, lds);
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

}  // namespace

void launch_qkv(hipStream_t s, const bf16_t* u, int rows, int d, const bf16_t* w, bf16_t* q,
                const KvGeom& kv, int layer, int Hq, int Hkv, int dh, const float2* rope,
                const ReqTable& rt, int32_t* sync, int n_sync) {
  QkvArgs p{q, kv, layer, Hq, Hkv, dh, rope, rt, sync, n_sync};
  const int NT = (Hq + 2 * Hkv) * (dh / 2) / 64;
  const int MC = div_up(rows, StreamTile<DMT>::CH);
  hipLaunchKernelGGL(qkv_kernel, dim3(NT * MC), dim3(256), 0, s, u, rows, d, w, p);
}

void launch_resid(hipStream_t s, const bf16_t* a, int rows, int K, const bf16_t* w, int N, float* h, float* ss) {
  const int MC = div_up(rows, StreamTile<DMT>::CH);
  hipLaunchKernelGGL(resid_kernel, dim3((N / 64) * MC), dim3(256), 0, s, a, rows, K, w, N, h, ss);
}
