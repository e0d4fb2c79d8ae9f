// Canvas attention: every canvas (or block) position of a request attends to
// the request's cached prefix and to the block itself, with GQA (q heads
// h = g*rep .. g*rep+rep-1 read kv head g). Denoising uses no mask inside the
// block; the causal encoder (commit / prefill) masks keys after the query.
//
// A work-group takes 64*QB query vectors of one (request, kv head), QB
// blocks of 16 per wave, and one contiguous range of 64-key tiles (a split of
// the keys), keeping an online softmax per query. Each K/V fragment a wave
// reads from LDS feeds the products of all of its query blocks. (QB = 2
// halves the LDS traffic per query but measured slower here: it halves the
// work-groups, and their registers allow one per compute unit.) Operands come straight from the KV cache:
//   S^T = K Q^T: the A operand is 16 keys x 32 dims of K, row-major in the
//     cache (16 contiguous bytes per lane), the B operand the wave's queries.
//   O^T = V^T P^T: the score accumulators already sit in the B-operand layout
//     (the lane holding query q has keys {4g+r} and {16+4g+r} of each 32-key
//     step); the cache stores V in that same key grouping (see v_index), so
//     the A operand is again 16 contiguous bytes per lane.
// A tile's 32 operand fragments (1 KB each) are copied global -> LDS by the
// asynchronous load-to-LDS path into one of two distinct LDS buffers: lane L
// of a copy lands at byte 16*L of its fragment, so each wave later reads a
// fragment with one linear, conflict-free LDS load, and the four waves share
// one copy of the tile. The next tile's copy is issued as soon as the current
// tile is in place; because the two buffers are distinct objects, reading one
// never waits for the copy into the other. (A deeper ring of copies measured
// no faster: the tile's LDS reads and softmax, not the copy, set the pace,
// and 64 KB of LDS leaves room for two work-groups per compute unit.)
// Softmax work is kept off the common path: keys are masked only on tiles
// that reach past the cache length or (causal) past a query's position, the
// running output is rescaled only when some query's maximum moved, and the
// denominator comes from the matrix cores (see lacc).
// With several splits, each work-group writes its unnormalised output and
// (max, sum) through to device-coherent memory and counts itself in; the last
// of the (request, kv head, query block) to arrive merges the splits in split
// order (deterministic), writes the bf16 output and resets the counter.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int KT = 64;  // keys per tile
constexpr int QB = 1;   // 16-query blocks per wave
constexpr int ATTN_QWG = 64 * QB;  // query vectors per work-group


__device__ __forceinline__ void store16_coherent(void* dst, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}
__device__ __forceinline__ void store8_coherent(void* dst, u32x2 v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

template <int DH>
__global__ __launch_bounds__(256) void attn_kernel(const bf16_t* __restrict__ q, KvGeom kv, int layer, ReqTable rt,
                                                   int Hq, int Hkv, int causal, int nsplit, float scale_log2,
                                                   float* __restrict__ opart, float2* __restrict__ ml,
                                                   int32_t* __restrict__ sync, bf16_t* __restrict__ out) {
  constexpr int NS = DH / 32;  // 32-dim steps of QK^T
  constexpr int ND = DH / 16;  // 16-dim output subtiles
  constexpr int CHUNKS = 4 * NS + 2 * ND;
  constexpr int QPW = 16 * QB;  // query vectors per wave
  // two distinct buffers: a copy into one never delays reads of the other
  __shared__ __align__(16) u32x4 tbA[CHUNKS][64];
  __shared__ __align__(16) u32x4 tbB[CHUNKS][64];
  __shared__ int s_last;
  const int rep = Hq / Hkv;
  const int n = rt.rows_per_req;
  const int rows_total = rt.n_req * n;
  const int nqv = n * rep;
  const int qblocks = div_up(nqv, ATTN_QWG);
  // Work-group id -> (request r, kv head g, query block qb, key split).
  // Dispatch is round-robin over the 8 XCDs (ids equal modulo 8 share an
  // XCD and its L2). When the (request, kv head) pairs come in multiples of
  // 8, every work-group of one pair gets ids equal modulo 8: the pair's K/V
  // tiles are fetched into that XCD's L2 once, and the split merge reads the
  // partial outputs its own XCD wrote. Otherwise the query blocks of one key
  // range (r, g, split) get ids equal modulo 8, in runs of 8 ranges ordered
  // query block major, so they still share one L2 copy of the tiles.
  const int npairs = rt.n_req * Hkv;
  int r, g, qb, split;
  if ((npairs & 7) == 0) {
    const int per = qblocks * nsplit, x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int pair = x + 8 * (i / per), local = i % per;
    qb = local / nsplit;
    split = local % nsplit;
    r = pair / Hkv;
    g = pair % Hkv;
  } else {
    const int C = npairs * nsplit;
    const int b = blockIdx.x, run = 8 * qblocks;
    const int cb = b / run, rem = b % run, width = min(8, C - 8 * cb);
    qb = rem / width;
    const int c = 8 * cb + rem % width;
    split = c % nsplit;
    g = (c / nsplit) % Hkv;
    r = c / (nsplit * Hkv);
  }
  const int group = (r * Hkv + g) * qblocks + qb;  // (request, kv head, query block)

  const int P = rt.pos0[r];
  const int nk = P + n;
  const int tiles = div_up(nk, KT);
  const int per = div_up(tiles, nsplit);
  const int t0 = split * per;
  const int t1 = min(tiles, t0 + per);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  // query block j of the wave: query vectors qb*QWG + wave*QPW + 16j + l16
  bool qvalid[QB];
  int qh[QB], row[QB], qlimit[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int qv = qb * ATTN_QWG + wave * QPW + 16 * j + l16;
    qvalid[j] = qv < nqv;
    const int qi = qvalid[j] ? qv / rep : 0;
    qh[j] = g * rep + (qvalid[j] ? qv % rep : 0);
    row[j] = r * n + qi;
    qlimit[j] = P + qi;  // causal: keys at positions <= P + qi
  }

  u32x4 qf[QB][NS];
  f32x4 oacc[QB][ND];
  f32x4 lacc[QB];
  float m_run[QB];  // running maximum of scale_log2 * score
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) oacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    lacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
  }

  const int slot = rt.slot[r];
  const bf16_t* Kp = kv.k_plane(slot, layer, g);
  const bf16_t* Vp = kv.v_plane(slot, layer, g);

  // Fragments of a tile: K subtile ks (16 keys) x dim step st at ks*NS + st,
  // then V block kk (32 keys) x dim subtile dt at 4*NS + kk*ND + dt. Wave w
  // copies chunks w + 4j. Both planes advance by KT*DH elements per tile, so
  // interior tiles only offset the addresses of the first tile; the tile that
  // reaches past nk clamps: K rows to the last key (finite; their scores are
  // masked), V blocks to the last block holding keys (entries past nk are
  // zeroed before use).
  constexpr int CPW = CHUNKS / 4;  // chunks per wave
  const bf16_t* cbase[CPW];
#pragma unroll
  for (int jc = 0; jc < CPW; ++jc) {
    const int ch = wave + 4 * jc;
    if (ch < 4 * NS) {
      cbase[jc] = Kp + (int64_t)(16 * (ch / NS) + l16) * DH + 32 * (ch % NS) + 8 * grp;
    } else {
      const int kk = (ch - 4 * NS) / ND, dt = (ch - 4 * NS) % ND;
      cbase[jc] = Vp + ((int64_t)(kk * 4 + grp) * DH + 16 * dt + l16) * 8;
    }
  }
  auto copy_tile = [&](int tile, u32x4 (&tb)[CHUNKS][64]) {
    const int k0 = tile * KT;
    const bool edge = k0 + KT > nk;
#pragma unroll
    for (int jc = 0; jc < CPW; ++jc) {
      const int ch = wave + 4 * jc;
      const bf16_t* src = cbase[jc] + (int64_t)k0 * DH;
      if (edge) {
        if (ch < 4 * NS) {
          const int key = min(k0 + 16 * (ch / NS) + l16, nk - 1);
          src = Kp + (int64_t)key * DH + 32 * (ch % NS) + 8 * grp;
        } else {
          const int kk = (ch - 4 * NS) / ND, dt = (ch - 4 * NS) % ND;
          const int blk = min((k0 + 32 * kk) >> 5, (nk - 1) >> 5);
          src = Vp + (((int64_t)blk * 4 + grp) * DH + 16 * dt + l16) * 8;
        }
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tb[ch][0], 16, 0, 0);
    }
  };
  // smallest query position of the wave: causal masking is needed only on
  // tiles reaching past it
  const int qi_lo = min((qb * ATTN_QWG + wave * QPW) / rep, n - 1);
  // the denominator runs on the matrix cores: an all-ones A operand turns the
  // probabilities of the PV product into their column sums
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  auto compute_tile = [&](int tile, const u32x4 (&tb)[CHUNKS][64]) {
    const int k0 = tile * KT;
    // All of the tile's K fragments are read from LDS at once, in the order
    // the products use them (dimension step major), so the first products
    // wait only for the first reads; the products then run dimension step by
    // dimension step over the four 16-key subtiles, so consecutive products
    // never depend on each other. The scheduling barrier keeps the reads
    // together: left to itself the compiler issued them in pairs, each pair
    // followed by a wait for all outstanding LDS reads.
    f32x4 s[QB][4];
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s[j][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 kf[4][NS];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks][st] = tb[ks * NS + st][lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < QB; ++j) s[j][ks] = mfma_bf16(kf[ks][st], qf[j][st], s[j][ks]);
    // the V fragments of both 32-key blocks are read right behind the
    // products, so they arrive while the softmax is formed
    u32x4 vf[2][ND];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) vf[kk][dt] = tb[4 * NS + kk * ND + dt][lane];
    __builtin_amdgcn_sched_barrier(0);
    const bool v_edge = k0 + KT > nk;
    const bool mask = v_edge || (causal && k0 + KT - 1 > P + qi_lo);
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (mask) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int key = k0 + 16 * ks + 4 * grp + rr;
            if (key >= nk || (causal && key > qlimit[j])) s[j][ks][rr] = -INFINITY;
          }
      }
      float tmax = fmaxf(fmaxf(fmaxf(s[j][0][0], s[j][0][1]), fmaxf(s[j][0][2], s[j][0][3])),
                         fmaxf(fmaxf(s[j][1][0], s[j][1][1]), fmaxf(s[j][1][2], s[j][1][3])));
      tmax = fmaxf(tmax, fmaxf(fmaxf(fmaxf(s[j][2][0], s[j][2][1]), fmaxf(s[j][2][2], s[j][2][3])),
                               fmaxf(fmaxf(s[j][3][0], s[j][3][1]), fmaxf(s[j][3][2], s[j][3][3]))));
      tmax = xrow_max(tmax);  // the other key groups of the query
      // running maximum in the scaled log2 domain (scale > 0 keeps the order)
      const float m_new = fmaxf(m_run[j], tmax * scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      // alpha == 1 exactly when the maximum did not move: skip the rescale
      // when that holds for every query of the block
      if (__ballot(m_new != m_run[j]) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_use);
        lacc[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) oacc[j][dt] *= alpha;
      }
      m_run[j] = m_new;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          s[j][ks][rr] = __builtin_amdgcn_exp2f(fmaf(s[j][ks][rr], scale_log2, -m_use));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 pf = {pack_bf16x2(s[j][2 * kk][0], s[j][2 * kk][1]),
                          pack_bf16x2(s[j][2 * kk][2], s[j][2 * kk][3]),
                          pack_bf16x2(s[j][2 * kk + 1][0], s[j][2 * kk + 1][1]),
                          pack_bf16x2(s[j][2 * kk + 1][2], s[j][2 * kk + 1][3])};
        if (v_edge) {
          // keys past nk: V entries may be unwritten cache rows (any bit
          // pattern); zero them so that 0 * V stays 0
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = k0 + 32 * kk + (e >> 2) * 16 + 4 * grp + (e & 3);
            const uint32_t keep = key < nk ? 0xffffffffu : ((e & 1) ? 0x0000ffffu : 0xffff0000u);
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) vf[kk][dt][e >> 1] &= keep;
          }
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) oacc[j][dt] = mfma_bf16(vf[kk][dt], pf, oacc[j][dt]);
        lacc[j] = mfma_bf16(ones, pf, lacc[j]);
      }
    }
  };

  // Tiles alternate between the two buffers: the copy of tile t + 1 is
  // issued as soon as tile t is in place (every wave waited for its own
  // copies, then the barrier) and overlaps the products of tile t.
  if (t0 < t1) copy_tile(t0, tbA);
  // the query fragments load while the first tile is in flight
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int st = 0; st < NS; ++st)
      qf[j][st] = qvalid[j] ? ld16(q + ((int64_t)row[j] * Hq + qh[j]) * DH + 32 * st + 8 * grp) : zero;
  for (int tile = t0; tile < t1; tile += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the tile have landed
    __syncthreads();                // ... and every other wave's; buffer B is free
    if (tile + 1 < t1) copy_tile(tile + 1, tbB);
    compute_tile(tile, tbA);
    if (tile + 1 >= t1) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tile + 2 < t1) copy_tile(tile + 2, tbA);
    compute_tile(tile + 1, tbB);
  }

  // lane (grp, l16) holds output dims 16dt + 4grp + 0..3 of query column l16
  // of each block; every row of the ones-product holds the column sum
  if (nsplit == 1) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (!qvalid[j]) continue;
      const float inv = 1.0f / lacc[j][0];
      bf16_t* op = out + ((int64_t)row[j] * Hq + qh[j]) * DH;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * grp) =
            u32x2{pack_bf16x2(oacc[j][dt][0] * inv, oacc[j][dt][1] * inv),
                  pack_bf16x2(oacc[j][dt][2] * inv, oacc[j][dt][3] * inv)};
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (!qvalid[j]) continue;
    float* op = opart + (((int64_t)split * rows_total + row[j]) * Hq + qh[j]) * DH;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) store16_coherent(op + 16 * dt + 4 * grp, __builtin_bit_cast(u32x4, oacc[j][dt]));
    // (max, sum) group-major, [group][split][ATTN_QWG queries]: a group's
    // entries fill whole lines that no other group touches
    if (grp == 0)
      store8_coherent(ml + ((int64_t)group * nsplit + split) * ATTN_QWG + wave * QPW + 16 * j + l16,
                      u32x2{__float_as_uint(m_run[j]), __float_as_uint(lacc[j][0])});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(sync + group, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nsplit - 1;
    if (s_last) __hip_atomic_store(sync + group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // merge: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, split order.
  // The group's partial lines are read only here, after every split wrote
  // them, and caches start the kernel invalidated: no stale copies. Every
  // load of a batch of four splits is issued before any is used (indices
  // past the last split are clamped and their terms skipped), so the merge
  // costs one or two memory round trips instead of one per split.
  constexpr int MAXS = DG_ATTN_SPLITS;
  static_assert(MAXS == 8, "two batches of four splits");
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (!qvalid[j]) continue;
    const int qcol = wave * QPW + 16 * j + l16;
    float2 mls[MAXS];
#pragma unroll
    for (int sp = 0; sp < MAXS; ++sp) mls[sp] = ml[((int64_t)group * nsplit + min(sp, nsplit - 1)) * ATTN_QWG + qcol];
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < MAXS; ++sp)
      if (sp < nsplit) M = fmaxf(M, mls[sp].x);
    float num[ND][4], den = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) num[dt][rr] = 0.f;
    auto batch = [&](int s0) {
      float4 v[4][ND];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* op = opart + (((int64_t)min(s0 + u, nsplit - 1) * rows_total + row[j]) * Hq + qh[j]) * DH;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) v[u][dt] = *reinterpret_cast<const float4*>(op + 16 * dt + 4 * grp);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = s0 + u;
        if (sp >= nsplit || mls[sp].x == -INFINITY) continue;
        const float wgt = exp2f(mls[sp].x - M);
        den += wgt * mls[sp].y;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          num[dt][0] += wgt * v[u][dt].x;
          num[dt][1] += wgt * v[u][dt].y;
          num[dt][2] += wgt * v[u][dt].z;
          num[dt][3] += wgt * v[u][dt].w;
        }
      }
    };
    batch(0);
    if (nsplit > 4) batch(4);
    const float inv = 1.0f / den;
    bf16_t* op = out + ((int64_t)row[j] * Hq + qh[j]) * DH;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * grp) =
          u32x2{pack_bf16x2(num[dt][0] * inv, num[dt][1] * inv), pack_bf16x2(num[dt][2] * inv, num[dt][3] * inv)};
  }
}

}  // namespace

// Splits of the key range: enough work-groups to cover the GPU about once
// (256 compute units, one work-group each); when the key ranges are long
// (at least 32 tiles per split at two work-groups per CU), enough for two
// per CU, whose per-tile softmax chains then interleave (measured 160 ->
// 120 us at a 32,768-key prefix; at 2,304 keys two per CU are slower). At
// most DG_ATTN_SPLITS, at least one tile per split.
int attn_splits(const ReqTable& rt, int Hq, int Hkv, int max_rows) {
  (void)max_rows;
  const int rep = Hq / Hkv;
  const int base = rt.n_req * Hkv * div_up(rt.rows_per_req * rep, ATTN_QWG);
  int max_pos = 0;
  for (int r = 0; r < rt.n_req; ++r) max_pos = max(max_pos, rt.pos0[r]);
  const int tiles = div_up(max_pos + rt.rows_per_req, KT);
  const int target = tiles >= 32 * div_up(512, base) ? 512 : 256;
  int ns = div_up(target, base);
  ns = min(ns, DG_ATTN_SPLITS);
  ns = min(ns, tiles);
  return max(ns, 1);
}

// (request, kv head, query block) groups of a call of at most max_rows rows:
// sum_r Hkv * ceil(n_r * rep / QWG) <= max_rows * Hq / QWG + DG_MAX_REQ * Hkv.
int attn_groups_bound(int max_rows, int Hq, int Hkv) { return div_up(max_rows * Hq, ATTN_QWG) + DG_MAX_REQ * Hkv; }

int attn_group_queries() { return ATTN_QWG; }

void launch_attention(hipStream_t s, const bf16_t* q, const KvGeom& kv, int layer, const ReqTable& rt, int Hq,
                      int Hkv, int dh, int causal, int nsplit, float* opart, float2* ml, int32_t* sync, bf16_t* out) {
  const int rep = Hq / Hkv;
  const int blocks = rt.n_req * Hkv * div_up(rt.rows_per_req * rep, ATTN_QWG) * nsplit;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  if (dh == 128)
    hipLaunchKernelGGL(attn_kernel<128>, dim3(blocks), dim3(256), 0, s, q, kv, layer, rt, Hq, Hkv, causal, nsplit,
                       scale_log2, opart, ml, sync, out);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(blocks), dim3(256), 0, s, q, kv, layer, rt, Hq, Hkv, causal, nsplit,
                       scale_log2, opart, ml, sync, out);
}
