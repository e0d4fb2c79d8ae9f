// Grouped SwiGLU experts over a device-built work list, in one persistent
// kernel.
//
// A group is the shared expert (group 0: all tokens) or a routed expert
// (group 1+e: the permutation slots off[e] .. off[e+1]). Each group's rows are
// cut into chunks of CH = 16*MT rows, and every (group, column tile, row
// chunk) is one work item, of one of two kinds:
//   gate/up:  hid[slot][f] = silu(x W_gate[f]) * (x W_up[f])   (bf16; 64 columns f)
//   (weights bf16, or FP8 codes with per-row scales widened to bf16 in the tile)
//   down:     y[slot][c]   = w_slot * (hid[slot] W_down[c])     (bf16, 128 columns c;
//                                                              shared: ys[t][c], fp32)
// The permutation kernel writes the exclusive item offsets of both kinds and
// the chunk offsets per group, and zeroes the queue head and the per-chunk
// completion counters. Work-groups take items from the queue: all gate/up
// items first, then all down items, so a work-group that runs out of gate/up
// work starts on down items while the last gate/up items are still streaming
// (no second launch, no idle tail). A down item waits until every gate/up
// column tile of its chunk has published its rows to device-coherent memory
// (those items may run on another XCD, whose L2 is not coherent with this
// one). Every gate/up item is taken before any down item and
// never waits, so the wait always ends; it is still bounded, and a wait that
// runs out counts itself in the spin-timeout word instead of hanging.
//
// combine:  h[t] += ys[t] + sum_j y[slot[t][j]]               (fixed order)
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "stream.h"

namespace {

constexpr int SPIN_LIMIT = 1 << 20;  // polls (about a second) before giving up

struct MoeArgs {
  const bf16_t* u;  // [rows][d] normalised tokens
  int rows, d, F, Fs, E;
  const int32_t *perm, *cnt, *off;  // permutation (slot -> token), per-expert counts and offsets
  const float* wts;                 // routing weights [rows*k]
  const int32_t* widx;              // slot -> index into wts
  int32_t* items;                   // MoeItems layout
  const void *wg, *wu, *wd, *sg, *su, *sd;  // fragment-major weights (bf16, or FP8 codes)
  ExpertScales sc;                          // FP8 row scales (unused for bf16)
  bf16_t *hid, *hid_s;
  bf16_t* y;  // routed outputs [slots][d], weighted, rounded to bf16
  float* ys;  // shared expert's outputs [rows][d]
};

// Start of weight row `row` of a fragment-major matrix with K columns (rows
// in multiples of 16): 16-row blocks are contiguous, so the block holding
// row r starts r*K elements in.
template <bool W8>
__device__ __forceinline__ const void* wrow(const void* base, int64_t row, int K) {
  return static_cast<const char*>(base) + row * K * (W8 ? 1 : 2);
}

// 16-byte store that writes through to device-coherent memory (visible to
// every XCD once complete; no L2 write-back needed). The nop covers the
// store-data read hazard of wide vector stores.
__device__ __forceinline__ void store16_coherent(bf16_t* dst, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int next_item(int32_t* counter, int* s_slot) {
  __syncthreads();  // everyone has read the previous item
  if (threadIdx.x == 0) *s_slot = atomicAdd(counter, 1);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_slot);  // wave-uniform: branches stay scalar
}

template <int MT, bool W8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT >= 8 ? 2 : 3))) void moe_experts_kernel(MoeArgs p) {
  using T = StreamTile<MT>;
  __shared__ __align__(16) bf16_t lds[T::LDS_ELEMS];
  __shared__ int32_t s_gu[MOE_MAX_GROUPS + 1], s_dn[MOE_MAX_GROUPS + 1], s_ch[MOE_MAX_GROUPS + 1];
  __shared__ int32_t s_cnt[MOE_MAX_GROUPS], s_off[MOE_MAX_GROUPS];
  __shared__ float s_w[T::CH];
  __shared__ int s_item;
  const int G = p.E + 1;
  int32_t* queue = p.items + MOE_QUEUE;
  // The work-list tables: item and chunk offsets, and each expert's row
  // count and offset, which every item needs before its weights can stream.
  // (Taking the first ticket together with these loads made every
  // work-group hit the queue counter at the same instant: the atomics
  // serialise, and the launch started ~12 us later.)
  for (int i = threadIdx.x; i <= G; i += 256) {
    s_gu[i] = p.items[MOE_ITEMS_GU + i];
    s_dn[i] = p.items[MOE_ITEMS_DN + i];
    s_ch[i] = p.items[MOE_CHUNKS + i];
    if (i < p.E) {
      s_cnt[i] = p.cnt[i];
      s_off[i] = p.off[i];
    }
  }
  // weight loads run this many K-steps ahead (for FP8 too: five steps ahead,
  // which would keep as many bytes in flight as bf16, spilled registers and
  // measured slower)
  constexpr int EXPERT_DW = 2;
  int32_t* done = p.items + MOE_DONE;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  // Gate/up items beyond the first round of the resident grid start only as
  // work-groups free up, and the down items of their chunks wait for them.
  // Each runs as two half items of 32 columns instead, taken by two
  // work-groups, so that the last gate/up work streams with twice the
  // concurrency. With bf16 weights, and while its halves fill at most a
  // quarter of the first round, the shared expert's items run as halves
  // from the start: its chain (gate/up, then down items with K = Fs) is the
  // longest in the launch, and halves start its down items about half a
  // gate/up item sooner, without streaming any weight twice (experts 3.77 ->
  // 3.75 ms per step at 256 rows; with FP8 weights, whose items are half as
  // long, the launch took 94 instead of 91 us). Queue: 2*n_sh shared
  // halves, n_full whole items, 2*n_split halves, then the down items. Chunk
  // counters count 32-column units (a whole item adds 2).
  __syncthreads();  // the item tables above are in LDS for every thread
  const int n_gu = s_gu[G];
  const int n_sh = (!W8 && 8 * s_gu[1] <= (int)gridDim.x) ? s_gu[1] : 0;
  const int n_r = n_gu - n_sh;
  const int n_full = min(n_r, max(0, (int)gridDim.x - 2 * n_sh));
  const int n_split = n_r - n_full;
  const int n_gu_q = 2 * n_sh + n_full + 2 * n_split;
  for (;;) {
    const int b = next_item(queue, &s_item);
    const int total = n_gu_q + s_dn[G];
    if (b >= total) break;
    const bool up = b < n_gu_q;
    const int32_t* s_it = up ? s_gu : s_dn;
    int bl, half = -1;  // half item: which 32 of the item's 64 columns
    if (!up) {
      bl = b - n_gu_q;
    } else if (b < 2 * n_sh) {
      bl = b >> 1;
      half = b & 1;
    } else if (b - 2 * n_sh < n_full) {
      bl = n_sh + (b - 2 * n_sh);
    } else {
      const int unit = 2 * (n_sh + n_full) + (b - 2 * n_sh - n_full);
      bl = unit >> 1;
      half = unit & 1;
    }
    const int gi = __builtin_amdgcn_readfirstlane(find_group(s_it, G, bl));
    const bool shared = gi == 0;
    const int e = gi - 1;
    const int n = shared ? p.rows : s_cnt[e];
    const int base = shared ? 0 : s_off[e];
    const int nmc = div_up(n, T::CH);
    const int local = bl - s_it[gi];
    const int nt = local / nmc, mc = local % nmc;
    const int row0 = mc * T::CH, nrows = min(T::CH, n - row0);
    const int chunk = s_ch[gi] + mc;
    if (up) {
      const int col0 = nt * 64 + wave * 16;
      const int ldo = shared ? p.Fs : p.F;
      // weight row of column col0 in the gate / up matrices (an expert bank
      // is one [E*F][d] matrix)
      const int64_t wr = shared ? col0 : (int64_t)e * p.F + col0;
      const void* W0 = wrow<W8>(shared ? p.sg : p.wg, wr, p.d);
      const void* W1 = wrow<W8>(shared ? p.su : p.wu, wr, p.d);
      const float* S0 = W8 ? (shared ? p.sc.sg : p.sc.g) + wr : nullptr;
      const float* S1 = W8 ? (shared ? p.sc.su : p.sc.u) + wr : nullptr;
      bf16_t* out = shared ? p.hid_s : p.hid + (int64_t)base * p.F;
      // The tile takes the smallest row count that holds the chunk's rows
      // (32, 64 or CH): most chunks of a small batch hold far fewer rows than
      // CH, and the smaller tile stages, reads and multiplies only those.
      auto gate_up = [&](auto mt_tag) {
        constexpr int MTI = decltype(mt_tag)::value;
        f32x4 ag[MTI], au[MTI];
        stream_tile<MTI, true, EXPERT_DW, 2, W8, (MT >= 8)>(p.u, p.d, shared ? nullptr : p.perm + base, row0, nrows, W0, W1, S0, S1,
                                         p.d, ag, au, lds);
        // Publish: stage the 64-column tile in LDS, write whole 128-byte row
        // segments with write-through (agent-coherent) stores, wait until they
        // complete, then move the chunk's counter. An agent-scope release fence
        // would instead write back this XCD's whole L2 for every item.
        __syncthreads();   // the tile's last LDS reads are done
        bf16_t* st = lds;  // [16 MTI][72] bf16, inside the A tile buffers
#pragma unroll
        for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = ag[mt][r];
            st[(16 * mt + 4 * grp + r) * 72 + wave * 16 + l16] = f2bf(gv / (1.0f + expf(-gv)) * au[mt][r]);
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16 * MTI * 8 / 256; ++i) {
          const int c = threadIdx.x + 256 * i, rr = c >> 3, seg = (c & 7) * 8;
          if (row0 + rr < n)
            store16_coherent(out + (int64_t)(row0 + rr) * ldo + nt * 64 + seg,
                             *reinterpret_cast<const u32x4*>(st + rr * 72 + seg));
        }
      };
      // Half item: 32 columns; waves 0-1 stream the gate rows of its two
      // 16-column blocks, waves 2-3 the up rows, and the SwiGLU is formed
      // from both halves staged in LDS (same products, same results as the
      // whole item).
      const bool is_up = wave >= 2;
      const int colh = nt * 64 + half * 32;
      const int64_t wrh = (shared ? 0 : (int64_t)e * p.F) + colh + 16 * (wave & 1);
      const void* Wh = wrow<W8>(is_up ? (shared ? p.su : p.wu) : (shared ? p.sg : p.wg), wrh, p.d);
      const float* Sh = W8 ? (is_up ? (shared ? p.sc.su : p.sc.u) : (shared ? p.sc.sg : p.sc.g)) + wrh : nullptr;
      auto gate_up_half = [&](auto mt_tag) {
        constexpr int MTI = decltype(mt_tag)::value;
        constexpr int LDF = 33;  // padded fp32 row of the staging tiles
        f32x4 acc[MTI], unused[MTI];
        stream_tile<MTI, false, EXPERT_DW, 2, W8, (MT >= 8)>(p.u, p.d, shared ? nullptr : p.perm + base, row0, nrows, Wh, nullptr,
                                                  Sh, nullptr, p.d, acc, unused, lds);
        __syncthreads();  // the tile's last LDS reads are done
        float* stf = reinterpret_cast<float*>(lds);  // [gate, up][16 MTI][LDF] fp32
        float* mine = stf + (is_up ? 16 * MTI * LDF : 0);
#pragma unroll
        for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mine[(16 * mt + 4 * grp + r) * LDF + 16 * (wave & 1) + l16] = acc[mt][r];
        __syncthreads();
        for (int c = threadIdx.x; c < 16 * MTI * 4; c += 256) {
          const int rr = c >> 2, seg = (c & 3) * 8;
          if (row0 + rr < n) {
            u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float g0 = stf[rr * LDF + seg + 2 * j], g1 = stf[rr * LDF + seg + 2 * j + 1];
              const float u0 = stf[(16 * MTI + rr) * LDF + seg + 2 * j];
              const float u1 = stf[(16 * MTI + rr) * LDF + seg + 2 * j + 1];
              v[j] = (uint32_t)f2bf(g0 / (1.0f + expf(-g0)) * u0) | ((uint32_t)f2bf(g1 / (1.0f + expf(-g1)) * u1) << 16);
            }
            store16_coherent(out + (int64_t)(row0 + rr) * ldo + colh + seg, v);
          }
        }
      };
      if (half < 0) {
        if (MT >= 8 && nrows > 64)
          gate_up(std::integral_constant<int, (MT >= 8 ? 8 : MT)>{});
        else if (MT >= 4 && nrows > 32)
          gate_up(std::integral_constant<int, (MT >= 4 ? 4 : MT)>{});
        else
          gate_up(std::integral_constant<int, 2>{});
      } else {
        if (MT >= 8 && nrows > 64)
          gate_up_half(std::integral_constant<int, (MT >= 8 ? 8 : MT)>{});
        else if (MT >= 4 && nrows > 32)
          gate_up_half(std::integral_constant<int, (MT >= 4 ? 4 : MT)>{});
        else
          gate_up_half(std::integral_constant<int, 2>{});
      }
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(done + chunk, half < 0 ? 2 : 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int need = (shared ? p.Fs : p.F) / 32;  // 32-column units of the chunk's gate/up work
      // Poll with device-coherent relaxed loads. No cache invalidation is
      // needed after the wait (an agent-scope acquire would invalidate this
      // XCD's whole L2 on every poll): caches start the kernel invalidated,
      // and the chunk's rows of hid are read only by down items of this
      // chunk, all after the wait, so no L1 or L2 can hold a stale copy.
      if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(done + chunk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++spins > SPIN_LIMIT) {
            atomicAdd(p.items + MOE_SPIN_TIMEOUTS, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
      const int K = shared ? p.Fs : p.F;
      const bf16_t* A = shared ? p.hid_s : p.hid + (int64_t)base * p.F;
      float* outs = p.ys;                              // shared: fp32 rows
      bf16_t* outr = p.y + (int64_t)base * p.d;        // routed: bf16 slots
      // routing weights of the chunk's slots, staged while the weights stream
      if (threadIdx.x < T::CH)
        s_w[threadIdx.x] = (!shared && threadIdx.x < nrows) ? p.wts[p.widx[base + row0 + threadIdx.x]] : 1.0f;
      // 128 output columns per item: the wave owns two 16-row weight blocks;
      // the tile takes the smallest row count that holds the chunk's rows
      const int c0 = nt * 128 + wave * 32;
      const int64_t wr = shared ? c0 : (int64_t)e * p.d + c0;  // weight row of output column c0
      const void* Wd = shared ? p.sd : p.wd;
      const float* Sd = W8 ? (shared ? p.sc.sd : p.sc.d) + wr : nullptr;
      auto down = [&](auto mt_tag) {
        constexpr int MTI = decltype(mt_tag)::value;
        f32x4 acc0[MTI], acc1[MTI];
        stream_tile<MTI, true, EXPERT_DW, 2, W8, (MT >= 8)>(A, K, nullptr, row0, nrows, wrow<W8>(Wd, wr, K), wrow<W8>(Wd, wr + 16, K),
                                         Sd, W8 ? Sd + 16 : nullptr, K, acc0, acc1, lds);
        if (shared) {
#pragma unroll
          for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int q = 16 * mt + 4 * grp + r;
              if (row0 + q < n) {
                float* o = outs + (int64_t)(row0 + q) * p.d + c0 + l16;
                o[0] = acc0[mt][r];
                o[16] = acc1[mt][r];
              }
            }
        } else {
#pragma unroll
          for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int q = 16 * mt + 4 * grp + r;
              if (row0 + q < n) {
                bf16_t* o = outr + (int64_t)(row0 + q) * p.d + c0 + l16;
                o[0] = f2bf(acc0[mt][r] * s_w[q]);
                o[16] = f2bf(acc1[mt][r] * s_w[q]);
              }
            }
        }
      };
      if (MT >= 8 && nrows > 64)
        down(std::integral_constant<int, (MT >= 8 ? 8 : MT)>{});
      else if (MT >= 4 && nrows > 32)
        down(std::integral_constant<int, (MT >= 4 ? 4 : MT)>{});
      else
        down(std::integral_constant<int, 2>{});
    }
  }
}

// h[t] += ys[t] + sum_j y[slot[t][j]]  (fixed order: deterministic); then, when
// next_gain is given, u[t] = bf16(RMSNorm(h[t]) * next_gain): the pre-norm of
// the next layer (or the final norm) on the row just completed.
template <int MAXV>  // float4 per thread: d <= 1024 * MAXV
__global__ __launch_bounds__(256) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ ys,
                                                          const bf16_t* __restrict__ y,
                                                          const int32_t* __restrict__ slot, int d,
                                                          int k, const bf16_t* __restrict__ next_gain,
                                                          float eps, bf16_t* __restrict__ u) {
  __shared__ int32_t sl[8];
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) sl[tid] = slot[t * k + tid];
  __syncthreads();
  constexpr int MAXK = 8;  // k <= 8
  // Every load is issued before any sum (the k expert rows are independent
  // loads; a loop over k that adds as it loads would wait for each in turn).
  float4 ysv[MAXV], hv[MAXV];
  u32x2 yv[MAXV][MAXK], gv[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = min(tid * 4 + 1024 * i, d - 4);  // clamped: in bounds, unused past d
    ysv[i] = *reinterpret_cast<const float4*>(ys + (int64_t)t * d + c);
    hv[i] = *reinterpret_cast<const float4*>(h + (int64_t)t * d + c);
#pragma unroll
    for (int j = 0; j < MAXK; ++j)
      yv[i][j] = *reinterpret_cast<const u32x2*>(y + (int64_t)sl[min(j, k - 1)] * d + c);
    gv[i] = next_gain ? *reinterpret_cast<const u32x2*>(next_gain + c) : u32x2{0u, 0u};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = tid * 4 + 1024 * i;
    if (c >= d) break;
    float4 acc = ysv[i];
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
      if (j >= k) break;
      acc.x += __uint_as_float(yv[i][j].x << 16);
      acc.y += __uint_as_float(yv[i][j].x & 0xffff0000u);
      acc.z += __uint_as_float(yv[i][j].y << 16);
      acc.w += __uint_as_float(yv[i][j].y & 0xffff0000u);
    }
    float4 x = hv[i];
    x.x += acc.x;
    x.y += acc.y;
    x.z += acc.z;
    x.w += acc.w;
    *reinterpret_cast<float4*>(h + (int64_t)t * d + c) = x;
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
    const uint32_t lo = pack_bf16x2(x.x * inv * __uint_as_float(gv[i].x << 16),
                                    x.y * inv * __uint_as_float(gv[i].x & 0xffff0000u));
    const uint32_t hi = pack_bf16x2(x.z * inv * __uint_as_float(gv[i].y << 16),
                                    x.w * inv * __uint_as_float(gv[i].y & 0xffff0000u));
    *reinterpret_cast<u32x2*>(uo + c) = u32x2{lo, hi};
  }
}

}  // namespace

// Rows per work item. Every chunk of an expert streams all of that expert's
// weights, so a hot expert cut into many small chunks multiplies its weight
// traffic: 128-row chunks once experts average at least 16 rows, 64 from 8,
// else 32 (tiny batches).
int moe_rows_per_chunk(int rows, int E, int k) {
  return rows * k >= 16 * E ? 128 : rows * k >= 8 * E ? 64 : 32;
}

// Chunks over all groups: sum_e ceil(cnt_e / ch) + ceil(rows / ch) is at most
// rows*k/ch + E + rows/ch + 1; bounded with the smallest chunk size, so that
// it holds for every call of at most `rows` rows.
int moe_chunk_bound(int rows, int E, int k) {
  return div_up(rows * k, 32) + E + div_up(rows, 32) + 1;
}

// Persistent grid: as many work-groups as the GPU holds at once (queried
// once per kernel from its resource use).
template <typename Kernel>
static int resident_blocks(Kernel kernel, int& cache) {
  if (cache == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0)
      cache = 1024;
    else
      cache = cus * per_cu;
  }
  return cache;
}
static int g_resident[2][3];  // [bf16, fp8][MT=8, MT=4, MT=2]

template <bool W8>
static void launch_experts_fmt(hipStream_t s, const MoeArgs& p, int ch) {
  int* res = g_resident[W8 ? 1 : 0];
  if (ch == 128)
    hipLaunchKernelGGL((moe_experts_kernel<8, W8>), dim3(resident_blocks(moe_experts_kernel<8, W8>, res[0])),
                       dim3(256), 0, s, p);
  else if (ch == 64)
    hipLaunchKernelGGL((moe_experts_kernel<4, W8>), dim3(resident_blocks(moe_experts_kernel<4, W8>, res[1])),
                       dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((moe_experts_kernel<2, W8>), dim3(resident_blocks(moe_experts_kernel<2, W8>, res[2])),
                       dim3(256), 0, s, p);
}

void launch_moe_experts(hipStream_t s, const bf16_t* u, int rows, int d, int F, int Fs, int E, int k,
                        const int32_t* perm, const int32_t* cnt, const int32_t* off, const float* wts,
                        const int32_t* widx, int32_t* items, const void* wg, const void* wu, const void* wd,
                        const void* sg, const void* su, const void* sd, const ExpertScales* fp8, bf16_t* hid,
                        bf16_t* hid_s, bf16_t* y, float* ys) {
  MoeArgs p{u,  rows, d,  F,  Fs, E,  perm, cnt, off, wts, widx, items, wg, wu, wd, sg,
            su, sd,   fp8 ? *fp8 : ExpertScales{}, hid, hid_s, y, ys};
  const int ch = moe_rows_per_chunk(rows, E, k);
  if (fp8)
    launch_experts_fmt<true>(s, p, ch);
  else
    launch_experts_fmt<false>(s, p, ch);
}

void launch_moe_combine(hipStream_t s, float* h, const float* ys, const bf16_t* y, const int32_t* slot,
                        int rows, int d, int k, const bf16_t* next_gain, float eps, bf16_t* u) {
  if (d <= 2048)
    hipLaunchKernelGGL(moe_combine_kernel<2>, dim3(rows), dim3(256), 0, s, h, ys, y, slot, d, k, next_gain, eps, u);
  else
    hipLaunchKernelGGL(moe_combine_kernel<4>, dim3(rows), dim3(256), 0, s, h, ys, y, slot, d, k, next_gain, eps, u);
}
