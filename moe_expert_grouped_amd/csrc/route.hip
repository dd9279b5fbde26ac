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
// logits in registers (E <= 1024); the selection and the softmax are
// topk_softmax (topk.h).  Memory traffic is 4*T*E + 8*T*k bytes with
// coalesced row loads; the kernel is latency-bound at the shapes of interest.
#include "topk.h"

namespace moe {

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
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  topk_softmax<EPL>(v, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
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
