// MoE routing: top-k experts per token with a softmax over the selected
// logits, then the token -> expert permutation (counting sort by expert,
// tokens ascending inside an expert) built with wave ballots and a
// wave-level prefix sum.
#include <type_traits>

#include <algorithm>

#include "common.h"
#include "kernels.h"

size_t permute_lds_bytes(int rows, int E, int k);

namespace {

// For a work-group that leaves a launch early while others still run (HBM
// mostly idle): copy its stripe of up to three equal-sized byte ranges that
// the next launch reads first into scratch LDS (1 KB a wave) with the
// load-to-LDS path, so that those lines sit in the memory-side cache when
// the next launch asks. Best effort: stripes of work-groups that do not leave
// early are skipped. Waits for its copies before returning (the LDS is the
// work-group's own until it exits).
__device__ __forceinline__ void prefetch_stripe(const char* r0, const char* r1, const char* r2, int64_t bytes,
                                                char* lds_scratch) {
  if (bytes < 16) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const char* rs[3] = {r0, r1, r2};
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    if (!rs[r]) continue;
    for (int64_t o = ((int64_t)blockIdx.x * nw + wave) * 1024; o < bytes; o += (int64_t)gridDim.x * nw * 1024)
      __builtin_amdgcn_global_load_lds(rs[r] + min(o + lane * 16, bytes - 16),
                                       (__attribute__((address_space(3))) void*)(lds_scratch + wave * 1024), 16, 0,
                                       0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Top-k (k <= 8) of E <= 128 logits for each of RB = 16 rows: every 16-lane
// group of the work-group's four waves takes one row, lane l16 holding the
// logits of experts l16 + 16m (m < 8; experts past E read as -inf). Each
// round takes the group's arg-max (lane-local over the 8 values, then four
// DPP steps inside the group; on equal values the lower expert id wins) and
// retires it. The selection comes out in descending order; lane j of the
// group then writes choice j and its softmax weight over the selected logits,
// w_j = exp(z_(j) - z_(0)) / sum_i exp(z_(i) - z_(0)), summed in that order.
// zl: LDS tile [16][E + 1]; rows at or past `rows` are skipped.
constexpr int RB = 16;  // rows per block

// With `coherent`, the expert ids are stored at agent scope (written through
// to memory), for a reader on another XCD within the same launch.
__device__ __forceinline__ void block_topk16(const float* zl, int E, int k, int t0, int rows, int32_t* __restrict__ idx,
                             float* __restrict__ w, bool coherent = false) {
  const int tid = threadIdx.x, r = tid >> 4, l16 = tid & 15;
  const float* zr = zl + r * (E + 1);
  float v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = l16 + 16 * m;
    v[m] = e < E ? zr[e] : -INFINITY;
  }
  // Always eight rounds (k <= 8 <= E; rounds past k are not used), written
  // with selects so that the rounds stay free of branches.
  float sel[8];
  int sid[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // lane-local: experts ascend with m, so a strict '>' keeps the lower id
    float bv = v[0];
    int bi = l16;
#pragma unroll
    for (int m = 1; m < 8; ++m) {
      const bool gt = v[m] > bv;
      bv = gt ? v[m] : bv;
      bi = gt ? l16 + 16 * m : bi;
    }
    // across the 16 lanes of the row on the DPP network; the merge is a
    // maximum under a total order, so every lane ends with the row's winner
    auto merge = [&](float ov, int oi) {
      const bool better = ov > bv || (ov == bv && oi < bi);
      bv = better ? ov : bv;
      bi = better ? oi : bi;
    };
    merge(dpp_movf<DPP_XOR1>(bv), dpp_mov<DPP_XOR1>(bi));
    merge(dpp_movf<DPP_XOR2>(bv), dpp_mov<DPP_XOR2>(bi));
    merge(dpp_movf<DPP_HALF_MIRROR>(bv), dpp_mov<DPP_HALF_MIRROR>(bi));
    merge(dpp_movf<DPP_MIRROR>(bv), dpp_mov<DPP_MIRROR>(bi));
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = bi == l16 + 16 * m ? -INFINITY : v[m];
    sel[j] = bv;
    sid[j] = bi;
  }
  // softmax over the selection, summed in selection order (every lane of the
  // row forms the same sum); lane j of the row then writes choice j
  float ex[8], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = j < k ? expf(sel[j] - sel[0]) : 0.f;
    sum += ex[j];
  }
  const int t = t0 + r;
  if (l16 < k && t < rows) {
    int my_id = sid[0];
    float my_ex = ex[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      my_id = j == l16 ? sid[j] : my_id;
      my_ex = j == l16 ? ex[j] : my_ex;
    }
    if (coherent)
      __hip_atomic_store(idx + (int64_t)t * k + l16, my_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      idx[(int64_t)t * k + l16] = my_id;
    w[(int64_t)t * k + l16] = my_ex / sum;
  }
}

// Top-k from given router logits: 16 rows per work-group.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int rows, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ float zl[RB * 129];
  const int t0 = blockIdx.x * RB;
  for (int i = threadIdx.x; i < RB * E; i += 256) {
    const int r = i / E, t = min(t0 + r, rows - 1);
    zl[r * (E + 1) + i % E] = z[(int64_t)t * E + i % E];
  }
  __syncthreads();
  block_topk16(zl, E, k, t0, rows, idx, w);
}

// Exclusive prefix sum of n <= 320 ints by one wave (5 consecutive per lane);
// out[n] receives the total.
__device__ __forceinline__ void wave_exclusive_scan(const int32_t* in, int32_t* out, int n, int lane) {
  int local[5], acc = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = lane * 5 + i;
    local[i] = e < n ? in[e] : 0;
    acc += local[i];
  }
  const int inc = wave_inclusive_scan(acc);
  int run = inc - acc;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = lane * 5 + i;
    if (e < n) out[e] = run;
    run += local[i];
  }
  if (lane == 63) out[n] = inc;
}

// Token -> expert permutation and the expert kernel's work list, by one
// work-group of any size that is a multiple of 256 threads (at least 4
// waves); nb = ceil(rows / 64) token blocks. When the (expert, block) tables
// of all rows fit the LDS budget (permute_max_blocks), in one pass:
//  1. mask[e][b] = bit set of the tokens of block b that chose expert e
//     (64-bit LDS atomic OR per (token, choice) pair);
//  2. one thread per expert: popcounts of its masks, running sum over the
//     blocks -> cnt[e] and the tokens of e in earlier blocks;
//  3. off = exclusive prefix sum of cnt; base[e][b] = off[e] + earlier
//     tokens; the work list of the expert kernel (groups: 0 = shared expert,
//     1 + e = routed e) as exclusive item and row-chunk offsets;
//  4. every pair (t, j) with expert e = idx[t][j] takes slot
//     base[e][t/64] + popcount(mask[e][t/64] below t): tokens ascending
//     inside an expert, three stores per pair (slot[t][j] coalesced).
// Otherwise (large batches) the counts come from LDS atomics over all pairs
// first, and steps 1, 2 and 4 run over consecutive chunks of
// permute_max_blocks token blocks, each chunk's bases starting after the
// tokens of the same expert in earlier chunks.
// With `coherent`, idx is read at agent scope (it was written in the same
// launch, possibly on another XCD). lds: permute_lds_bytes(rows, E, k).
struct PermuteArgs {
  const int32_t* idx;
  int rows, E, k, ch, ft_routed, ft_shared, dt;
  int32_t *cnt, *off, *perm, *slot, *widx, *items;
};

// LDS budget of the (expert, token block) tables: 8-byte mask + 4-byte base.
constexpr int PERMUTE_LDS_BUDGET = 57344;
__host__ __device__ __forceinline__ int permute_max_blocks(int E) { return PERMUTE_LDS_BUDGET / (12 * E); }

__device__ __forceinline__ void permute_block(const PermuteArgs& a, char* lds, bool coherent) {
  const int rows = a.rows, E = a.E, k = a.k;
  const int nb_all = (rows + 63) / 64;
  const bool chunked = nb_all > permute_max_blocks(E);
  const int nb = chunked ? permute_max_blocks(E) : nb_all;  // blocks held in the tables at a time
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(lds);  // [E][nb]
  int32_t* base = reinterpret_cast<int32_t*>(mask + (size_t)E * nb);     // [E][nb]
  __shared__ int32_t s_cnt[257];
  __shared__ int32_t s_run[257];
  __shared__ int32_t s_off[258];
  __shared__ int32_t s_ngu[MOE_MAX_GROUPS], s_ndn[MOE_MAX_GROUPS], s_nch[MOE_MAX_GROUPS];
  __shared__ int32_t s_igu[MOE_MAX_GROUPS + 1], s_idn[MOE_MAX_GROUPS + 1], s_ich[MOE_MAX_GROUPS + 1];
  const int nt = blockDim.x, nw = nt >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pairs = rows * k;
  auto load_idx = [&](int i) {
    return i >= pairs ? 0
                      : coherent ? __hip_atomic_load(a.idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : a.idx[i];
  };
  // expert ids are loaded PB per thread at a time, all issued before any use;
  // when one batch covers every pair, they stay in registers for step 4
  constexpr int PB = 8;
  const bool one_batch = !chunked && pairs <= PB * nt;
  int evc[PB];
  if (!chunked) {
    // with one batch, the ids are loaded before the tables are cleared
    if (one_batch) {
#pragma unroll
      for (int j = 0; j < PB; ++j) evc[j] = load_idx(tid + j * nt);
    }
    for (int i = tid; i < E * nb; i += nt) mask[i] = 0ull;
    __syncthreads();
    for (int i0 = tid; i0 < pairs; i0 += PB * nt) {
      int ev[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) ev[j] = one_batch ? evc[j] : load_idx(i0 + j * nt);
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        evc[j] = ev[j];
        const int i = i0 + j * nt, t = i / k;
        if (i < pairs) atomicOr(&mask[ev[j] * nb + (t >> 6)], 1ull << (t & 63));
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += nt) {  // one thread per expert, over its nb masks
      int run = 0;
      for (int b = 0; b < nb; ++b) {
        base[e * nb + b] = run;  // tokens of e in earlier blocks
        run += __popcll(mask[e * nb + b]);
      }
      s_cnt[e] = run;
    }
  } else {
    // counts over all pairs (the order of the atomics does not matter)
    for (int e = tid; e < E; e += nt) {
      s_cnt[e] = 0;
      s_run[e] = 0;
    }
    __syncthreads();
    for (int i0 = tid; i0 < pairs; i0 += PB * nt) {
      int ev[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) ev[j] = load_idx(i0 + j * nt);
#pragma unroll
      for (int j = 0; j < PB; ++j)
        if (i0 + j * nt < pairs) atomicAdd(&s_cnt[ev[j]], 1);
    }
  }
  __syncthreads();
  // groups: 0 = shared expert (all rows), 1 + e = routed expert e
  for (int g = tid; g <= E; g += nt) {
    const int n = g == 0 ? rows : s_cnt[g - 1];
    const int nmc = (n + a.ch - 1) / a.ch;
    s_nch[g] = nmc;
    s_ngu[g] = nmc * (g == 0 ? a.ft_shared : a.ft_routed);
    s_ndn[g] = nmc * a.dt;
  }
  __syncthreads();
  if (wave == 0) wave_exclusive_scan(s_cnt, s_off, E, lane);
  if (wave == 1) wave_exclusive_scan(s_ngu, s_igu, E + 1, lane);
  if (wave == 2) wave_exclusive_scan(s_ndn, s_idn, E + 1, lane);
  if (wave == 3) wave_exclusive_scan(s_nch, s_ich, E + 1, lane);
  __syncthreads();
  if (!chunked)
    for (int i = tid; i < E * nb; i += nt) base[i] += s_off[i / nb];
  for (int e = tid; e < E; e += nt) {
    a.cnt[e] = s_cnt[e];
    a.off[e] = s_off[e];
  }
  if (tid == 0) {
    a.off[E] = s_off[E];
    a.items[MOE_QUEUE] = 0;
  }
  if (wave == 4 % nw) {  // running statistics: experts touched per call
    int touched = 0;
    for (int e0 = 0; e0 < E; e0 += 64) touched += __popcll(__ballot(e0 + lane < E && s_cnt[e0 + lane] > 0));
    if (lane == 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(a.items + MOE_TOUCHED_TOTAL), (unsigned long long)touched);
      atomicAdd(reinterpret_cast<unsigned long long*>(a.items + MOE_PERMUTE_CALLS), 1ull);
    }
  }
  for (int g = tid; g <= E + 1; g += nt) {
    a.items[MOE_ITEMS_GU + g] = s_igu[g];
    a.items[MOE_ITEMS_DN + g] = s_idn[g];
    a.items[MOE_CHUNKS + g] = s_ich[g];
  }
  for (int c = tid; c < s_ich[E + 1]; c += nt) a.items[MOE_DONE + c] = 0;
  __syncthreads();  // base is final
  if (chunked) {
    // chunks of nb token blocks in order; s_run[e] = tokens of e in earlier chunks
    for (int c0 = 0; c0 < rows; c0 += 64 * nb) {
      const int cr = min(64 * nb, rows - c0), cnb = (cr + 63) / 64;
      for (int i = tid; i < E * cnb; i += nt) mask[i] = 0ull;
      __syncthreads();
      const int p0 = c0 * k, p1 = (c0 + cr) * k;
      for (int i0 = p0 + tid; i0 < p1; i0 += PB * nt) {
        int ev[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) ev[j] = i0 + j * nt < p1 ? load_idx(i0 + j * nt) : 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int i = i0 + j * nt, t = i / k - c0;
          if (i < p1) atomicOr(&mask[ev[j] * cnb + (t >> 6)], 1ull << (t & 63));
        }
      }
      __syncthreads();
      for (int e = tid; e < E; e += nt) {
        int run = s_off[e] + s_run[e];
        for (int b = 0; b < cnb; ++b) {
          base[e * cnb + b] = run;
          run += __popcll(mask[e * cnb + b]);
        }
        s_run[e] = run - s_off[e];
      }
      __syncthreads();
      for (int i0 = p0 + tid; i0 < p1; i0 += PB * nt) {
        int ev[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) ev[j] = i0 + j * nt < p1 ? load_idx(i0 + j * nt) : 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int i = i0 + j * nt;
          if (i >= p1) break;
          const int t = i / k, e = ev[j], tl = t - c0, b = tl >> 6, l = tl & 63;
          const unsigned long long below = l == 0 ? 0ull : (mask[e * cnb + b] << (64 - l));
          const int pos = base[e * cnb + b] + __popcll(below);
          a.slot[i] = pos;
          a.perm[pos] = t;
          a.widx[pos] = i;
        }
      }
      __syncthreads();  // the tables are reused by the next chunk
    }
    return;
  }
  for (int i0 = tid; i0 < pairs; i0 += PB * nt) {
    int ev[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) ev[j] = one_batch ? evc[j] : load_idx(i0 + j * nt);
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int i = i0 + j * nt;
      if (i >= pairs) break;
      const int t = i / k, e = ev[j], b = t >> 6, l = t & 63;
      const unsigned long long below = l == 0 ? 0ull : (mask[e * nb + b] << (64 - l));
      const int pos = base[e * nb + b] + __popcll(below);
      a.slot[i] = pos;
      a.perm[pos] = t;
      a.widx[pos] = i;
    }
  }
}

// The permutation as a launch of its own (1024 threads), from top-k results
// of an earlier launch.
__global__ __launch_bounds__(1024) void permute_kernel(PermuteArgs a) {
  extern __shared__ __align__(8) char pm_lds[];
  permute_block(a, pm_lds, false);
}

// MoE pre-norm, router logits and top-k. Work-group (row block rb of RB = 16
// rows, K part ks) of a grid of ceil(rows/16) x RKS, d split into RKS parts:
// eighths for calls of up to 512 rows (each work-group's first loads, which
// set the pace of such a launch, halve against quarters, ~1 us faster),
// quarters above (the extra partial lines and the last arrival's longer sum
// cost more than the shorter first loads save once the launch holds several
// waves of work-groups):
//  1. issues every load that depends on nothing at once, in order of use:
//     the sums of squares of its rows, its part of the hidden-state rows
//     and norm gains, and its router weight fragments (expert rows
//     16*(2w+n) + l16 of wave w, clamped to E-1, over its part of d);
//  2. 1/rms of its rows from the output projection's per-64-column sums of
//     squares (summed in a fixed order);
//  3. u = bf16(h / rms * gain) on its part of d -> workspace (the experts'
//     input rows) and an LDS tile;
//  4. partial logits of its part on the matrix cores, written through to
//     device-coherent memory, then counts itself in for the row block;
//  5. the last of the RKS to arrive adds the partials in part order
//     (deterministic whatever the arrival order), stores z, resets the
//     counter, and selects each row's experts (block_topk16);
//  6. (with the permutation) the last row block to finish runs it.
constexpr int ROUTER_EIGHTHS_MAX_ROWS = 512;

__device__ __forceinline__ void store16_coherent(void* dst, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

template <int RKS>
__global__ __launch_bounds__(256) void router_kernel(
    const float* __restrict__ h, const float* __restrict__ ss, const bf16_t* __restrict__ gain, int rows, int d,
    float eps, const bf16_t* __restrict__ wr, int E, int k, bf16_t* __restrict__ u, float* __restrict__ z,
    float* __restrict__ zpart, int32_t* __restrict__ sync, int32_t* __restrict__ idx, float* __restrict__ w,
    PermuteArgs pa, int do_permute, const char* pf0, const char* pf1, const char* pf2, int64_t pfn) {
  // 32-wide K steps whose weight fragments are loaded at once: a whole part
  // when d = 2048
  constexpr int RSTEPS = 64 / RKS;
  extern __shared__ __align__(16) char rt_lds[];
  const int kq = d / RKS, LDA = kq + 8, nct = d / 64;
  bf16_t* As = reinterpret_cast<bf16_t*>(rt_lds);                    // [RB][LDA]
  float* zt = reinterpret_cast<float*>(rt_lds + RB * LDA * 2);       // [RB][E + 1]
  float* sq = zt + RB * (E + 1);                                     // [RB][nct]
  __shared__ float s_inv[RB];
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int rb = blockIdx.x / RKS, ks = blockIdx.x % RKS;
  const int t0 = rb * RB, kb = ks * kq, nk = kq / 32;
  // part stride in rows, a multiple of RB: every row block's partials
  // fill whole 128-byte lines (E % 8 == 0), shared with no other block
  const int zs = div_up(rows, RB) * RB;

  // 1. every load that depends on nothing is issued first, in the order of
  // use (completion is in order): the output projection's sums of squares of
  // the block's rows, its first batch of hidden-state values and norm gains,
  // then the router weight fragments of the first RSTEPS steps
  float sqv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 256 * j, r = i / nct, ct = i % nct, t = t0 + r;
    sqv[j] = (i < RB * nct && t < rows) ? ss[(int64_t)ct * rows + t] : 0.f;
  }
  float4 hv[8];
  u32x2 gv[8];
  auto load_h = [&](int i0) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = i0 + b * 1024, r = i / kq, c = i % kq, t = min(t0 + r, rows - 1);
      const bool ok = i < RB * kq;
      hv[b] = *reinterpret_cast<const float4*>(h + (int64_t)t * d + kb + (ok ? c : 0));
      gv[b] = *reinterpret_cast<const u32x2*>(gain + kb + (ok ? c : 0));
    }
  };
  load_h(tid * 4);
  const bf16_t* brow[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) brow[n] = wr + (int64_t)min(16 * (2 * wave + n) + l16, E - 1) * d + kb + 8 * grp;
  u32x4 bf[RSTEPS][2];
#pragma unroll
  for (int st = 0; st < RSTEPS; ++st)
#pragma unroll
    for (int n = 0; n < 2; ++n) bf[st][n] = ld16(brow[n] + min(st, nk - 1) * 32);

  // 2. 1/rms per row: the partial sums added in tile order
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (tid + 256 * j < RB * nct) sq[tid + 256 * j] = sqv[j];
  for (int i = tid + 512; i < RB * nct; i += 256) {  // d > 2048: the remaining sums
    const int r = i / nct, ct = i % nct, t = t0 + r;
    sq[i] = t < rows ? ss[(int64_t)ct * rows + t] : 0.f;
  }
  __syncthreads();
  if (tid < RB) {
    float acc = 0.f;
    for (int ct = 0; ct < nct; ++ct) acc += sq[tid * nct + ct];
    s_inv[tid] = 1.0f / sqrtf(acc / (float)d + eps);
  }
  __syncthreads();

  // 3. normalised rows on this part (rows past the end are zero), in
  // batches of 8 float4 per thread (the first already loaded)
  for (int i0 = tid * 4; i0 < RB * kq; i0 += 8 * 1024) {
    if (i0 != tid * 4) load_h(i0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = i0 + b * 1024, r = i / kq, c = i % kq, t = t0 + r;
      if (i >= RB * kq) break;
      u32x2 pk = {0u, 0u};
      if (t < rows) {
        const float inv = s_inv[r];
        const float4 v = hv[b];
        pk = u32x2{pack_bf16x2(v.x * inv * __uint_as_float(gv[b].x << 16),
                               v.y * inv * __uint_as_float(gv[b].x & 0xffff0000u)),
                   pack_bf16x2(v.z * inv * __uint_as_float(gv[b].y << 16),
                               v.w * inv * __uint_as_float(gv[b].y & 0xffff0000u))};
        *reinterpret_cast<u32x2*>(u + (int64_t)t * d + kb + c) = pk;
      }
      *reinterpret_cast<u32x2*>(As + r * LDA + c) = pk;
    }
  }
  __syncthreads();

  // 4. partial logits: 16 rows x 32 experts per wave over the part
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = 0; s0 < nk; s0 += RSTEPS) {
    if (s0 > 0) {
#pragma unroll
      for (int st = 0; st < RSTEPS; ++st)
#pragma unroll
        for (int n = 0; n < 2; ++n) bf[st][n] = ld16(brow[n] + min(s0 + st, nk - 1) * 32);
    }
#pragma unroll
    for (int st = 0; st < RSTEPS; ++st) {
      const u32x4 a0 = ld16(As + l16 * LDA + min(s0 + st, nk - 1) * 32 + 8 * grp);
      const u32x4 a = s0 + st < nk ? a0 : zero;  // steps past the end add nothing
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[n] = mfma_bf16(a, bf[st][n], acc[n]);
    }
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = 16 * (2 * wave + n) + l16;
    if (e < E)
#pragma unroll
      for (int r = 0; r < 4; ++r) zt[(4 * grp + r) * E + e] = acc[n][r];  // dense [RB][E] here
  }
  __syncthreads();
  for (int i = tid * 4; i < RB * E; i += 1024) {
    const int t = t0 + i / E;
    if (t < rows)
      store16_coherent(zpart + ((int64_t)ks * zs + t) * E + i % E, *reinterpret_cast<const u32x4*>(zt + i));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(sync + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == RKS - 1;
    if (s_last) __hip_atomic_store(sync + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) {
    // leaving early (all but one of the RKS work-groups, ~13 us before the
    // launch ends at 256 rows): the
    // shared expert's weights, which the expert launch streams first, are
    // brought towards the caches meanwhile
    prefetch_stripe(pf0, pf1, pf2, pfn, rt_lds);
    return;
  }

  // 5. the last arrival: z = p0 + p1 + ... + p(RKS-1) in that order, then top-k per
  // row. The block's partial lines are read only here, after all were written,
  // and caches start the kernel invalidated: no cache holds a stale copy.
  // (E <= 128: at most 8 entries per thread, every load issued before the sums)
  // The loads are unconditional (indices clamped into the block's rows) and
  // every sum is formed before any store: gfx950 counts stores in the same
  // in-order counter as loads, so a store placed between a load and its use
  // would make that use wait for the store's round trip too.
  // Each thread takes two runs of four consecutive experts of one row (E is a
  // multiple of 8), 16-byte loads.
  float4 pv[2][RKS];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int i = min((tid + 256 * b) * 4, RB * E - 4), t = min(t0 + i / E, rows - 1), e = i % E;
#pragma unroll
    for (int q = 0; q < RKS; ++q) pv[b][q] = *reinterpret_cast<const float4*>(zpart + ((int64_t)q * zs + t) * E + e);
  }
  float4 zv[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    zv[b] = pv[b][0];
#pragma unroll
    for (int q = 1; q < RKS; ++q) {
      zv[b].x += pv[b][q].x;
      zv[b].y += pv[b][q].y;
      zv[b].z += pv[b][q].z;
      zv[b].w += pv[b][q].w;
    }
  }
  __syncthreads();  // the dense staging view of zt is no longer read
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int i = (tid + 256 * b) * 4, r = i / E, t = t0 + r, e = i % E;
    if (i < RB * E) {
      const bool live = t < rows;
      if (live) *reinterpret_cast<float4*>(z + (int64_t)t * E + e) = zv[b];
      float* zr = zt + r * (E + 1) + e;
      zr[0] = live ? zv[b].x : 0.f;
      zr[1] = live ? zv[b].y : 0.f;
      zr[2] = live ? zv[b].z : 0.f;
      zr[3] = live ? zv[b].w : 0.f;
    }
  }
  __syncthreads();
  block_topk16(zt, E, k, t0, rows, idx, w, do_permute != 0);
  if (!do_permute) return;

  // 6. the last row block to finish runs the permutation over all rows: its
  // expert ids were written through to memory and waited for before the
  // block counted itself in, and the permutation reads them at agent scope
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int nrb = div_up(rows, RB);
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(sync + nrb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nrb - 1;
    if (s_last) __hip_atomic_store(sync + nrb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  permute_block(pa, rt_lds, true);
}

}  // namespace

void launch_topk(hipStream_t s, const float* z, int rows, int E, int k, int32_t* idx, float* w) {
  hipLaunchKernelGGL(topk_kernel, dim3(div_up(rows, RB)), dim3(256), 0, s, z, rows, E, k, idx, w);
}

void launch_router(hipStream_t s, const float* h, const float* ss, const bf16_t* gain, int rows, int d, float eps,
                   const bf16_t* wr, int E, int k, bf16_t* u, float* z, float* zpart, int32_t* sync, int32_t* idx,
                   float* w, const RouterPermute* perm, const void* const* pf, int64_t pfn) {
  const int rks = rows <= ROUTER_EIGHTHS_MAX_ROWS ? 8 : 4;
  const int kq = d / rks;
  size_t lds = (size_t)RB * (kq + 8) * 2 + (size_t)RB * (E + 1) * 4 + (size_t)RB * (d / 64) * 4;
  PermuteArgs pa{idx, rows, E, k, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (perm) {
    pa = PermuteArgs{idx, rows, E, k, perm->ch, perm->ft_routed, perm->ft_shared, perm->dt, perm->cnt, perm->off,
                     perm->perm, perm->slot, perm->widx, perm->items};
    lds = std::max(lds, permute_lds_bytes(rows, E, k));
  }
  if (pf) lds = std::max(lds, (size_t)4096);  // prefetch_stripe's scratch: 1 KB a wave
  const char* p0 = pf ? (const char*)pf[0] : nullptr;
  const char* p1 = pf ? (const char*)pf[1] : nullptr;
  const char* p2 = pf ? (const char*)pf[2] : nullptr;
  const int64_t pn = pf ? pfn : 0;
  const dim3 grid(div_up(rows, RB) * rks);
  if (rks == 8)
    hipLaunchKernelGGL(router_kernel<8>, grid, dim3(256), lds, s, h, ss, gain, rows, d, eps, wr, E, k, u, z, zpart,
                       sync, idx, w, pa, perm ? 1 : 0, p0, p1, p2, pn);
  else
    hipLaunchKernelGGL(router_kernel<4>, grid, dim3(256), lds, s, h, ss, gain, rows, d, eps, wr, E, k, u, z, zpart,
                       sync, idx, w, pa, perm ? 1 : 0, p0, p1, p2, pn);
}

void launch_permute(hipStream_t s, const int32_t* idx, int rows, int E, int k, const RouterPermute& p) {
  const size_t lds = permute_lds_bytes(rows, E, k);
  const PermuteArgs pa{idx, rows, E, k, p.ch, p.ft_routed, p.ft_shared, p.dt, p.cnt, p.off, p.perm, p.slot,
                       p.widx, p.items};
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, pa);
}

// Dynamic LDS of the permutation kernel: mask (8 B) and base (4 B) per
// (expert, 64-token block), for at most permute_max_blocks(E) blocks at a time.
size_t permute_lds_bytes(int rows, int E, int k) {
  (void)k;
  return (size_t)E * std::min((rows + 63) / 64, permute_max_blocks(E)) * 12;
}
