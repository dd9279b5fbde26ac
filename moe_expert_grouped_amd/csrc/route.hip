// route.hip -- top-k routing with a softmax over the k selected logits.
//
// The MoE layer of "Comm-compute fusion (1)" (section 4, the MoE layer0 /
// layer1 rows: reorder by route, then a top-k weighted reduction) needs, for
// every token, its k experts and their weights.  The pages do not define the
// router; the reading taken: select on the fp32 logits (descending, equal
// logits to the lower expert id, slot 0 the largest) and weight by the
// softmax over the k selected logits.
//
// Design: one 64-lane wavefront per token.  Each lane holds ceil(E/64)
// logits in registers (E <= 1024).  Each of the k rounds finds the lane-local
// best untaken (value, id), then a cross-lane butterfly reduction picks the
// global best with the lower-id tie-break; comparisons are exact fp32, so the
// selection matches any correct implementation bit for bit.  The softmax is
// fp32 on the k selected values.  Memory traffic is 4*T*E + 8*T*k bytes with
// coalesced row loads; the kernel is latency-bound at the shapes of interest.
#include "common.h"

namespace moe {

struct Cand {
  float v;
  int e;
};

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
  return a.v > b.v || (a.v == b.v && a.e < b.e);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T,
                                                    int E, int k,
                                                    int32_t *__restrict__ topk_idx,
                                                    float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return; // whole wave exits together (t is wave-uniform)

  const float *row = logits + (size_t)t * E;
  float v[EPL];
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    taken[i] = e >= E; // slots past E never compete
    v[i] = e < E ? row[e] : 0.0f;
  }

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
    topk_idx[(size_t)t * k + lane] = sel_e;
    topk_w[(size_t)t * k + lane] = ex / s;
  }
}

hipError_t launch_route(const float *logits, int T, int E, int k, int32_t *topk_idx,
                        float *topk_w, hipStream_t stream) {
  const int tokens_per_block = 4;
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
  const int epl = (E + 63) / 64;
  if (epl <= 1)
    route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (epl <= 2)
    route_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (epl <= 4)
    route_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (epl <= 8)
    route_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else
    route_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

} // namespace moe
