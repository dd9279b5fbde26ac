// topk.h -- one token's top-k selection and softmax on a 64-lane wavefront,
// shared by the routing kernel (logits from memory) and the router kernel
// (logits it computed itself).  gfx950 only; nothing here is shared with
// the oracle.
#pragma once

#include "common.h"

namespace moe {

struct Cand {
  float v;
  int e;
};

// larger logit first; equal logits to the lower expert id
__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
  return a.v > b.v || (a.v == b.v && a.e < b.e);
}

// The wavefront holds logit v[i] of expert lane + 64 i (i < EPL); experts at
// or past E never compete.  Each of the k rounds finds each lane's best
// untaken (value, id), then a butterfly reduction picks the wavefront's best
// with the lower-id tie-break: comparisons are exact fp32, so the selection
// matches any correct implementation bit for bit.  Slot 0 holds the largest
// logit; the weights are the fp32 softmax over the k selected logits.  Lane
// j < k writes slot j of idx_row / w_row.
template <int EPL>
__device__ __forceinline__ void topk_softmax(const float (&v)[EPL], int E, int k, int lane,
                                             int32_t *__restrict__ idx_row,
                                             float *__restrict__ w_row) {
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) taken[i] = lane + 64 * i >= E;

  float sel_v = 0.0f; // lane j keeps the j-th selected logit / id
  int sel_e = 0;
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    Cand c{0.0f, 0x7fffffff};
    bool have = false;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (!taken[i]) {
        Cand d{v[i], lane + 64 * i};
        if (!have || better(d, c)) c = d;
        have = true;
      }
    }
    // a lane with nothing left offers an id that loses every comparison
    if (!have) c.v = -__builtin_inff();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Cand o;
      o.v = __shfl_xor(c.v, off, 64);
      o.e = __shfl_xor(c.e, off, 64);
      if (better(o, c)) c = o;
    }
    // c is now the same (value, id) in every lane
    if (j == 0) top = c.v;
    if (lane == j) {
      sel_v = c.v;
      sel_e = c.e;
    }
    const int owner_slot = c.e >> 6;
    if ((c.e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i == owner_slot) taken[i] = true;
    }
  }

  const float ex = lane < k ? expf(sel_v - top) : 0.0f;
  float s = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane < k) {
    idx_row[lane] = sel_e;
    w_row[lane] = ex / s;
  }
}

} // namespace moe
