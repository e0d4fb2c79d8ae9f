// Grouped SwiGLU experts over a device-built work list.
//
// A group is a routed expert (its tokens are the permutation slots
// off[e] .. off[e+1]) or the shared expert (all tokens). Each group's rows are
// cut into chunks of CH = 16*MT rows, and every (group, column tile, row
// chunk) is one work item; the permutation kernel writes the exclusive item
// offsets per group, so any routing, however uneven, becomes a flat list of
// equal-sized items: a group with many tokens gets many items.
//
// gate/up:  hid[slot][f] = silu(x W_gate[f]) * (x W_up[f])   (bf16)
// down:     y[slot][c]   = w_slot * (hid[slot] W_down[c])     (fp32; shared: ys[t][c])
// combine:  h[t] += ys[t] + sum_j y[slot[t][j]]               (fixed order)
#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace {

// Both expert kernels are persistent: a fixed grid of work-groups takes work
// items from an atomic counter (zeroed by the permutation kernel) until the
// list is exhausted, so a launch never ends with a second, mostly idle round
// of work-groups. Every work-group exits once the counter passes the item
// count.
__device__ __forceinline__ int next_item(int32_t* counter, int* s_slot) {
  __syncthreads();  // everyone has read the previous item
  if (threadIdx.x == 0) *s_slot = atomicAdd(counter, 1);
  __syncthreads();
  return *s_slot;
}

template <int MT>
__global__ __launch_bounds__(256) void moe_gateup_kernel(
    const bf16_t* __restrict__ u, int rows, int d, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ items, int32_t* __restrict__ queue, const bf16_t* __restrict__ wg,
    const bf16_t* __restrict__ wu, int F, int E, const bf16_t* __restrict__ sg,
    const bf16_t* __restrict__ su, int Fs, bf16_t* __restrict__ hid, bf16_t* __restrict__ hid_s) {
  using T = StreamTile<MT>;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  __shared__ int32_t s_items[258];
  __shared__ int s_item;
  const int n_groups = E + 1;
  for (int i = threadIdx.x; i <= n_groups; i += 256) s_items[i] = items[i];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  for (;;) {
    const int b = next_item(queue, &s_item);
    if (b >= s_items[n_groups]) break;
    const int g = find_group(s_items, n_groups, b);
    int n, ldo;
    const int32_t* rowmap;
    const bf16_t *W0, *W1;
    bf16_t* out;
    if (g < E) {
      n = cnt[g];
      const int base = off[g];
      rowmap = perm + base;
      W0 = wg + (int64_t)g * F * d;
      W1 = wu + (int64_t)g * F * d;
      out = hid + (int64_t)base * F;
      ldo = F;
    } else {
      n = rows;
      rowmap = nullptr;
      W0 = sg;
      W1 = su;
      out = hid_s;
      ldo = Fs;
    }
    const int nmc = div_up(n, T::CH);
    const int local = b - s_items[g];
    const int nt = local / nmc, mc = local % nmc;
    const int row0 = mc * T::CH, nrows = min(T::CH, n - row0);
    const int col = nt * 64 + wave * 16 + l16;
    f32x4 ag[MT], au[MT];
    stream_tile<MT, true>(u, d, rowmap, row0, nrows, W0 + (int64_t)col * d, W1 + (int64_t)col * d, d, ag, au,
                          lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = row0 + 16 * mt + 4 * grp + r;
        if (p < n) {
          const float gv = ag[mt][r];
          out[(int64_t)p * ldo + col] = f2bf(gv / (1.0f + expf(-gv)) * au[mt][r]);
        }
      }
  }
}

template <int MT>
__global__ __launch_bounds__(256) void moe_down_kernel(
    const bf16_t* __restrict__ hid, const bf16_t* __restrict__ hid_s, int rows, int d,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const float* __restrict__ wts_all, const int32_t* __restrict__ widx,
    const int32_t* __restrict__ items, int32_t* __restrict__ queue, const bf16_t* __restrict__ wd, int F,
    int E, const bf16_t* __restrict__ sd, int Fs, float* __restrict__ y, float* __restrict__ ys) {
  using T = StreamTile<MT>;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  __shared__ int32_t s_items[258];
  __shared__ float s_w[T::CH];
  __shared__ int s_item;
  const int n_groups = E + 1;
  for (int i = threadIdx.x; i <= n_groups; i += 256) s_items[i] = items[i];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  for (;;) {
    const int b = next_item(queue, &s_item);
    if (b >= s_items[n_groups]) break;
    const int g = find_group(s_items, n_groups, b);
    int n, K;
    const bf16_t *A, *W;
    float* out;
    const bool routed = g < E;
    int base = 0;
    if (routed) {
      n = cnt[g];
      base = off[g];
      A = hid + (int64_t)base * F;
      K = F;
      W = wd + (int64_t)g * d * F;
      out = y + (int64_t)base * d;
    } else {
      n = rows;
      A = hid_s;
      K = Fs;
      W = sd;
      out = ys;
    }
    const int nmc = div_up(n, T::CH);
    const int local = b - s_items[g];
    const int nt = local / nmc, mc = local % nmc;
    const int row0 = mc * T::CH, nrows = min(T::CH, n - row0);
    // routing weights of the chunk's slots, staged while the weights stream
    if (threadIdx.x < T::CH)
      s_w[threadIdx.x] = (routed && threadIdx.x < nrows) ? wts_all[widx[base + row0 + threadIdx.x]] : 1.0f;
    const int col = nt * 64 + wave * 16 + l16;
    f32x4 acc[MT], unused[MT];
    stream_tile<MT, false>(A, K, nullptr, row0, nrows, W + (int64_t)col * K, nullptr, K, acc, unused, lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = 16 * mt + 4 * grp + r;
        const int p = row0 + q;
        if (p < n) out[(int64_t)p * d + col] = acc[mt][r] * s_w[q];
      }
  }
}

// h[t] += ys[t] + sum_j y[slot[t][j]]  (fixed order: deterministic); then, when
// next_gain is given, u[t] = bf16(RMSNorm(h[t]) * next_gain): the pre-norm of
// the next layer (or the final norm) on the row just completed.
__global__ __launch_bounds__(256) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ ys,
                                                          const float* __restrict__ y,
                                                          const int32_t* __restrict__ slot, int d,
                                                          int k, const bf16_t* __restrict__ next_gain,
                                                          float eps, bf16_t* __restrict__ u) {
  __shared__ int32_t sl[8];
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) sl[tid] = slot[t * k + tid];
  __syncthreads();
  constexpr int MAXV = 4;  // float4 per thread: d <= 4096
  float4 hv[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = tid * 4 + 1024 * i;
    if (c >= d) break;
    float4 acc = *reinterpret_cast<const float4*>(ys + (int64_t)t * d + c);
    for (int j = 0; j < k; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)sl[j] * d + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    float4* hp = reinterpret_cast<float4*>(h + (int64_t)t * d + c);
    float4 x = *hp;
    x.x += acc.x;
    x.y += acc.y;
    x.z += acc.z;
    x.w += acc.w;
    *hp = x;
    hv[i] = x;
    ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
  if (!next_gain) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
  bf16_t* uo = u + (int64_t)t * d;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = tid * 4 + 1024 * i;
    if (c >= d) break;
    const float4 x = hv[i];
    const uint32_t lo = pack_bf16x2(x.x * inv * bf2f(next_gain[c]), x.y * inv * bf2f(next_gain[c + 1]));
    const uint32_t hi = pack_bf16x2(x.z * inv * bf2f(next_gain[c + 2]), x.w * inv * bf2f(next_gain[c + 3]));
    *reinterpret_cast<u32x2*>(uo + c) = u32x2{lo, hi};
  }
}

}  // namespace

// Rows per work item. 128-row chunks let one work-group reuse each weight
// tile across all the tokens of a busy expert (routing is far from uniform);
// small experts waste matrix-core work on empty rows, which is cheap next to
// the weight stream. Tiny batches use 32-row chunks.
int moe_rows_per_chunk(int rows, int E, int k) {
  return rows * k >= 8 * E ? 128 : 32;
}

int moe_item_bound(int rows, int E, int k, int n_tiles_routed, int n_tiles_shared) {
  const int CH = moe_rows_per_chunk(rows, E, k);
  const int chunks = div_up(rows * k, CH) + min(E, rows * k);
  return chunks * n_tiles_routed + div_up(rows, CH) * n_tiles_shared;
}

// Persistent grid: as many work-groups as the GPU holds at once (queried
// once per kernel from its resource use), never more than the item bound.
template <typename Kernel>
static int persistent_grid(Kernel kernel, int bound, int& resident) {
  if (resident == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0)
      resident = 1024;
    else
      resident = cus * per_cu;
  }
  return bound < resident ? bound : resident;
}
static int g_resident[4];  // gate/up MT=8, MT=2; down MT=8, MT=2

void launch_moe_gateup(hipStream_t s, const bf16_t* u, int rows, int d, const int32_t* perm,
                       const int32_t* cnt, const int32_t* off, const int32_t* items, int32_t* queue,
                       const bf16_t* wg, const bf16_t* wu, int F, int E, int k, const bf16_t* sg,
                       const bf16_t* su, int Fs, bf16_t* hid, bf16_t* hid_s) {
  const int bound = moe_item_bound(rows, E, k, F / 64, Fs / 64);
  if (moe_rows_per_chunk(rows, E, k) == 128)
    hipLaunchKernelGGL(moe_gateup_kernel<8>, dim3(persistent_grid(moe_gateup_kernel<8>, bound, g_resident[0])), dim3(256), 0,
                       s, u, rows, d, perm, cnt, off, items, queue, wg, wu, F, E, sg, su, Fs, hid, hid_s);
  else
    hipLaunchKernelGGL(moe_gateup_kernel<2>, dim3(persistent_grid(moe_gateup_kernel<2>, bound, g_resident[1])), dim3(256), 0,
                       s, u, rows, d, perm, cnt, off, items, queue, wg, wu, F, E, sg, su, Fs, hid, hid_s);
}

void launch_moe_down(hipStream_t s, const bf16_t* hid, const bf16_t* hid_s, int rows, int d,
                     const int32_t* cnt, const int32_t* off, const float* w, const int32_t* widx,
                     const int32_t* items, int32_t* queue, const bf16_t* wd, int F, int E, int k,
                     const bf16_t* sd, int Fs, float* y, float* ys) {
  const int bound = moe_item_bound(rows, E, k, d / 64, d / 64);
  if (moe_rows_per_chunk(rows, E, k) == 128)
    hipLaunchKernelGGL(moe_down_kernel<8>, dim3(persistent_grid(moe_down_kernel<8>, bound, g_resident[2])), dim3(256), 0, s,
                       hid, hid_s, rows, d, cnt, off, w, widx, items, queue, wd, F, E, sd, Fs, y, ys);
  else
    hipLaunchKernelGGL(moe_down_kernel<2>, dim3(persistent_grid(moe_down_kernel<2>, bound, g_resident[3])), dim3(256), 0, s,
                       hid, hid_s, rows, d, cnt, off, w, widx, items, queue, wd, F, E, sd, Fs, y, ys);
}

void launch_moe_combine(hipStream_t s, float* h, const float* ys, const float* y,
                        const int32_t* slot, int rows, int d, int k, const bf16_t* next_gain,
                        float eps, bf16_t* u) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(rows), dim3(256), 0, s, h, ys, y, slot, d, k, next_gain, eps,
                     u);
}
