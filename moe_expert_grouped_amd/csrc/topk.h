// topk.h -- one token's top-k selection and softmax on a 64-lane wavefront,
// shared by the routing kernel (logits from memory) and the router kernel
// (logits it computed itself).  gfx950 only; nothing here is shared with
// the oracle.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

// A candidate as one unsigned 64-bit key whose order is the selection order:
// the high half maps the fp32 logit to an unsigned integer of the same order
// (negative values bit-inverted, the others with the sign bit set), the low
// half is the inverted expert id, so equal logits go to the lower id (-0
// counts as +0, its equal).  Key 0 is below every real candidate.
__device__ __forceinline__ uint64_t cand_key(float v, int e) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

// The largest key of the wavefront, in every lane: DPP moves combine each
// quad (lane ^ 1, lane ^ 2) and then each row of 16 (rotations by 4 and 8),
// and the four row maxima are read out as scalars.  All 64 lanes must be
// active.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
  auto step = [&](auto CTRL) {
    constexpr int ctrl = decltype(CTRL)::value;
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)key, ctrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(key >> 32), ctrl, 0xf, 0xf, false);
    const uint64_t o = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    key = o > key ? o : key;
  };
  step(std::integral_constant<int, 0xb1>{});  // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4e>{});  // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x124>{}); // row_ror:4
  step(std::integral_constant<int, 0x128>{}); // row_ror:8
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    best = o > best ? o : best;
  }
  return best;
}

// The wavefront holds logit v[i] of expert lane + 64 i (i < EPL); experts at
// or past E never compete.  Each of the k rounds takes each lane's best
// untaken key and the wavefront's largest of them: the order is exact (larger
// fp32 logit, then lower id), so the selection matches any correct
// implementation bit for bit.  Slot 0 holds the largest logit; the weights
// are the fp32 softmax over the k selected logits, their exponentials summed
// in slot order.  Lane j < k writes slot j of idx_row / w_row, and returns
// the expert it wrote (other lanes return 0).
template <int EPL>
__device__ __forceinline__ int topk_softmax(const float (&v)[EPL], int E, int k, int lane,
                                             int32_t *__restrict__ idx_row,
                                             float *__restrict__ w_row) {
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i < E ? cand_key(v[i], lane + 64 * i) : 0;

  float top = 0.0f, sum = 0.0f;
  float sel_ex = 0.0f; // lane j keeps the j-th selected id and exponential
  int sel_e = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t c = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) c = key[i] > c ? key[i] : c;
    const uint64_t best = wave_max_key(c); // the same in every lane
    const float bv = key_value(best);
    const int be = key_expert(best);
    if (j == 0) top = bv;
    const float ex = expf(bv - top);
    sum += ex;
    if (lane == j) {
      sel_e = be;
      sel_ex = ex;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == best) key[i] = 0; // taken (keys are unique: one per expert)
  }
  if (lane < k) {
    idx_row[lane] = sel_e;
    w_row[lane] = sel_ex / sum;
  }
  return sel_e;
}

} // namespace moe
