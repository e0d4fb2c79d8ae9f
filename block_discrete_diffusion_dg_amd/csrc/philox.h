// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), written from that definition: each
// round multiplies counter words 0 and 2 by two fixed 32-bit multipliers,
// mixes the high halves with the other counter words and the key, and the key
// advances by two Weyl constants between rounds.
//
// The step draws one word per canvas position: counter = (position, step,
// block, request slot), key = (low, high 32 bits of the request's seed).
#pragma once

#include <stdint.h>

#include "common.h"

struct SampleTable {
  int32_t n_req;
  uint32_t key_lo[DG_MAX_REQ], key_hi[DG_MAX_REQ];
  int32_t block[DG_MAX_REQ];
  int32_t slot[DG_MAX_REQ];
};

inline SampleTable make_sample_table(int n_req, const uint64_t* seeds, const int32_t* blocks,
                                     const int32_t* slots) {
  SampleTable st{};
  st.n_req = n_req;
  for (int r = 0; r < n_req && r < DG_MAX_REQ; ++r) {
    st.key_lo[r] = (uint32_t)(seeds[r] & 0xffffffffu);
    st.key_hi[r] = (uint32_t)(seeds[r] >> 32);
    st.block[r] = blocks[r];
    st.slot[r] = slots[r];
  }
  return st;
}

// All four output words.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return u32x4{c0, c1, c2, c3};
}

// Gumbel noise for sampling (see the sampled-candidate mapping in dg.h): the
// uniform of vocabulary id v at canvas position i is word (v >> 4) & 3 of
// Philox at counter (v with bits 4-5 cleared, i, (block << 16) | step,
// 0x80000000 | slot), taken as ((word >> 9) + 1/2) * 2^-23 (exact in fp32).
__device__ __forceinline__ float gumbel_of_word(uint32_t w) {
  const float u = ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-07f;
  return -logf(-logf(u));
}

__device__ __forceinline__ uint32_t philox4x32_10_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                         uint32_t c3, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}
