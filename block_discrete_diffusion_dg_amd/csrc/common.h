// Device-side helpers shared by the gfx950 kernels: bf16 storage, MFMA
// fragments, wave-level reductions, and the per-call request table.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DG_MAX_REQ 32       // requests batched into one call

// Expert work list (int32 words in the workspace "items" buffer), written by
// the permutation kernel and consumed by the expert kernel. Groups: 0 = the
// shared expert, 1 + e = routed expert e.
constexpr int MOE_MAX_GROUPS = 129;       // E <= 128, plus the shared expert
constexpr int MOE_ITEMS_GU = 0;           // [G+1] exclusive gate/up item offsets
constexpr int MOE_ITEMS_DN = 136;         // [G+1] exclusive down item offsets
constexpr int MOE_CHUNKS = 272;           // [G+1] exclusive row-chunk offsets
constexpr int MOE_QUEUE = 408;            // work-queue head
constexpr int MOE_SPIN_TIMEOUTS = 409;    // waits that ran out (never reset)
constexpr int MOE_TOUCHED_TOTAL = 410;    // uint64: experts with >= 1 row, summed over calls
constexpr int MOE_PERMUTE_CALLS = 412;    // uint64: permutation calls (both never reset)
constexpr int MOE_DONE = 416;             // per-chunk count of finished 32-column gate/up units
#define DG_ATTN_SPLITS 8    // maximum key splits of the attention kernel
#define WAVE 64

// Per-call request table, passed by value to the kernels that need positions
// or KV-cache addresses. Row r*rows_per_req + i belongs to request r, at
// sequence position pos0[r] + i.
struct ReqTable {
  int32_t n_req;
  int32_t rows_per_req;
  int32_t slot[DG_MAX_REQ];
  int32_t pos0[DG_MAX_REQ];
};

// KV-cache geometry: [slot][layer][K|V][kv_head][max_ctx][head_dim] bf16.
struct KvGeom {
  bf16_t* base;
  int64_t slot_stride;   // elements per request slot
  int64_t layer_stride;  // elements per layer
  int64_t head_stride;   // elements per (K|V, kv_head) plane = max_ctx * dh
  int32_t n_kv_heads;
  int32_t head_dim;
  __device__ __forceinline__ bf16_t* k_plane(int slot, int layer, int g) const {
    return base + slot * slot_stride + layer * layer_stride + (int64_t)g * head_stride;
  }
  __device__ __forceinline__ bf16_t* v_plane(int slot, int layer, int g) const {
    return base + slot * slot_stride + layer * layer_stride +
           (int64_t)(n_kv_heads + g) * head_stride;
  }
};

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even: the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32), two values per instruction in pack_bf16x2.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// D = A(16x32) * B(32x16) + C on the gfx950 bf16 matrix core.
// Lane l supplies A row (l % 16) and B column (l % 16), eight consecutive
// reduction indices of group l / 16 (any fixed assignment of reduction
// indices works as long as A and B use the same one). The result holds
// D[4*(l/16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Reductions over the 16 lanes of each DPP row (lanes 16j .. 16j+15) on
// the DPP network, with no LDS round trip: butterflies inside each quad
// (lane ^ 1, lane ^ 2), then the half-row mirror (lane i <-> 7 - i within 8)
// and the row mirror (i <-> 15 - i). Every lane of the row ends with the same
// result: each step combines two equal-sized partial results, and the
// operation is commutative.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_movf(float v) {
  return __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_movf<DPP_XOR1>(v));
  v = fmaxf(v, dpp_movf<DPP_XOR2>(v));
  v = fmaxf(v, dpp_movf<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_movf<DPP_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_movf<DPP_XOR1>(v);
  v += dpp_movf<DPP_XOR2>(v);
  v += dpp_movf<DPP_HALF_MIRROR>(v);
  return v + dpp_movf<DPP_MIRROR>(v);
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_mov<DPP_XOR1>(v));
  v = min(v, dpp_mov<DPP_XOR2>(v));
  v = min(v, dpp_mov<DPP_HALF_MIRROR>(v));
  return min(v, dpp_mov<DPP_MIRROR>(v));
}

// Combine the four rows (lanes l, l ^ 16, l ^ 32, l ^ 48) with the gfx950
// row-swap instructions (VALU, no LDS round trip): with both operands the
// same register, v_permlane32_swap leaves each lane holding its own value
// and that of lane l ^ 32 (in some order), v_permlane16_swap the same for
// l ^ 16. The operation must be commutative; every lane ends with the same
// result.
__device__ __forceinline__ float xrow_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_sum(float v) { return xrow_sum(row16_sum(v)); }
__device__ __forceinline__ float wave_max(float v) { return xrow_max(row16_max(v)); }

// Inclusive prefix sum over the wave on the DPP network: shifts by 1, 2, 4, 8
// inside each 16-lane row (lanes shifted in from before the row start read
// 0), then the last lane of row 0 / row 2 is added to row 1 / row 3 and the
// last lane of row 1 to rows 2 and 3.
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118, DPP_BCAST15 = 0x142,
              DPP_BCAST31 = 0x143;
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, DPP_SHR1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_SHR2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_SHR4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_SHR8, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_BCAST15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, DPP_BCAST31, 0xc, 0xf, false);
  return v;
}

// (value, index) reduction: larger value wins, ties go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__host__ __device__ __forceinline__ int div_up(int a, int b) { return (a + b - 1) / b; }

// Work-group id -> (column tile nt, row chunk mc) for a grid of NT * MC
// work-groups. When NT is a multiple of 8, the row chunks of one column tile
// get ids 8 apart: dispatch is round-robin over the 8 XCDs, so they run on
// the same XCD and share its L2 copy of the tile's weights.
__device__ __forceinline__ void xcd_tile_coords(int NT, int MC, int& nt, int& mc) {
  const int b = blockIdx.x;
  if ((NT & 7) == 0) {
    mc = (b >> 3) % MC;
    nt = (b & 7) + 8 * (b / (8 * MC));
  } else {
    mc = b % MC;
    nt = b / MC;
  }
}
