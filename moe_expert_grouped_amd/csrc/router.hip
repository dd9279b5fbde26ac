// router.hip -- the router front end: logits = x . W^T and the routing of
// those logits in one launch.
//
// The pages take the router logits as given (the route that the reorder of
// "Comm-compute fusion (1)", section 4 follows); the step before them is the
// linear router, logits[t][e] = x[t] . W[e] with W stored [E][H], fp32
// accumulation of bf16 products.  The selection and the weights are exactly
// those of moe_route (topk_softmax in topk.h), taken on the fp32 logits
// computed here.
//
// Design (gfx950): one 4-wavefront workgroup per (32 tokens, hidden slice),
// each wavefront a quarter of the slice with 32x32x16 bf16 matrix
// instructions.  A routing of few tokens cuts H into up to 16 slices
// so the launch still covers the chip (a CU streams only a few tens of GB/s
// of these row pieces, so the bandwidth must come from all of them).  The A
// operand (32 token rows x 16 hidden) and the B operand (16 hidden x 32
// experts, i.e. 32 rows of W) are both 16 contiguous bytes per lane, so
// both are loaded straight from global memory into registers, a batch of k
// steps ahead of the matrix instructions that use them; the k order within
// groups of four steps is permuted so that each lane reads 64 contiguous
// bytes of its row per group.  The four wavefronts' [32 x E] tiles meet in
// LDS and are summed in wavefront order; with one slice each wavefront then
// routes 8 of the tokens, with several the slices' partial logits go to a
// workspace and a second launch adds them in slice order and routes (one
// fixed rounding order either way).  (128-token workgroups, which read half
// the W bytes per token, need 16 slices at T = 2048, and their partials
// then cost as much as x: 20.9 against 14.5 us.)
// Traffic: 2 T H (x, once) + 2 E H per workgroup (W, from L2) + 8 S T E
// (partials, S > 1) + 4 T E (logits, if written) + 8 T k bytes.
#include "topk.h"

namespace moe {

constexpr int kRouterTok = 32;                 // tokens per workgroup (one MFMA row tile)
constexpr int kRouterWaves = 4;

// The hidden dimension is cut into S slices so that a routing of few tokens
// still spreads over the whole chip (one workgroup per (32 tokens, slice)).
// S depends only on T and H: the smallest power of two, at most 16, with at
// least 256 workgroups, such that each slice is a multiple of 64.
int router_splits(int T, int H) {
  const int nblk = (T + kRouterTok - 1) / kRouterTok;
  int s = 1;
  while (s < 16 && (long)nblk * s < 256 && H % (64 * 2 * s) == 0) s *= 2;
  return s;
}

size_t router_workspace_bytes(int T, int H, int E) {
  const int s = router_splits(T, H);
  return s > 1 ? (size_t)s * T * E * sizeof(float) : 0;
}

// Workgroup (b, s): tokens 32 b .. 32 b + 31, hidden slice s (of S), a
// quarter of the slice per wavefront; with S == 1 it also routes its
// tokens, else it writes its [32 x E] partial logits to part_out[s] for
// router_select_kernel.
// NT 32-expert column tiles: E <= 32 NT
template <int NT>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ w, int T, int H,
                                                     int E, int k, int S, float *__restrict__ part_out,
                                                     float *__restrict__ logits,
                                                     int32_t *__restrict__ topk_idx,
                                                     float *__restrict__ topk_w) {
  constexpr int EP = 32 * NT;     // expert columns computed
  constexpr int LD = EP + 1;      // LDS row stride in floats
  constexpr int U = NT <= 2 ? 8 : 4; // k steps per load batch
  __shared__ float part[kRouterWaves][kRouterTok][LD];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kRouterTok;
  const int hs = H / S;             // this workgroup's hidden slice
  const int hq = hs / kRouterWaves; // this wavefront's part of it, a multiple of 16
  const int hoff = blockIdx.y * hs + wave * hq;
  const int q = lane >> 5;          // which 8 of a k step's 16 hidden values this lane holds

  // A: lane l holds 8 hidden values of token row t0 + l % 32, B the same 8 of
  // W row 32 n + l % 32 (the operand layouts of the 32x32x16 instruction).
  // Which 8: the k steps go in groups of four over 64 hidden values, and
  // lane half q takes the 32 values [32 q, 32 q + 32) of the group, 8 per
  // step -- each lane reads 64 contiguous bytes of its row over a group (the
  // sum over k is the same; its order is fixed).  Steps past the last whole
  // group take 16 consecutive values, 8 per lane half.
  const int steps = hq / 16;
  const int steps4 = steps & ~3;
  auto vec = [&](int st) { return st < steps4 ? 8 * (st >> 2) + 4 * q + (st & 3) : 2 * st + q; };
  // rows past T and experts past E read row 0 instead (loads stay unconditional,
  // so the compiler can keep the next batch in flight): their logits are
  // never written or selected
  const int ti = t0 + (lane & 31);
  const bool tv = ti < T;
  const bf16x8 *xa = reinterpret_cast<const bf16x8 *>(x + (size_t)(tv ? ti : 0) * H + hoff);
  const bf16x8 *wb[NT];
  bool ev[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = 32 * n + (lane & 31);
    ev[n] = e < E;
    wb[n] = reinterpret_cast<const bf16x8 *>(w + (size_t)(ev[n] ? e : 0) * H + hoff);
  }
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};

  // Batches of U k steps alternate between two register sets, so the next
  // batch's loads are in flight while the matrix instructions use this one.
  bf16x8 a0[U], b0[U][NT], a1[U], b1[U][NT];
  auto load = [&](bf16x8(&a)[U], bf16x8(&b)[U][NT], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = vec(s0 + u);
      a[u] = xa[v];
#pragma unroll
      for (int n = 0; n < NT; ++n) b[u][n] = wb[n][v];
    }
  };
  auto mma = [&](const bf16x8(&a)[U], const bf16x8(&b)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u][n], acc[n], 0, 0, 0);
  };
  const int nb = steps / U; // whole batches
  if (nb > 0) load(a0, b0, 0);
  int bi = 0;
  for (; bi + 1 < nb; bi += 2) {
    load(a1, b1, (bi + 1) * U);
    mma(a0, b0);
    if (bi + 2 < nb) load(a0, b0, (bi + 2) * U);
    mma(a1, b1);
  }
  if (bi < nb) mma(a0, b0); // an odd batch count ends in the first set
  for (int s = nb * U; s < steps; ++s) {
    const int v = vec(s);
    const bf16x8 a = xa[v];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = wb[n][v];
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
    }
  }

  // accumulator r of lane l: token 8 (r / 4) + 4 (l / 32) + r % 4, expert 32 n + l % 32
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      part[wave][8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][32 * n + (lane & 31)] = acc[n][r];
  __syncthreads();
  // the four wavefronts' parts, summed in wavefront order
  float *dst = S > 1 ? part_out + (size_t)blockIdx.y * T * E : logits;
  for (int i = threadIdx.x; i < kRouterTok * EP; i += blockDim.x) {
    const int tr = i / EP, e = i - tr * EP;
    float s = part[0][tr][e] + part[1][tr][e];
    s += part[2][tr][e];
    s += part[3][tr][e];
    part[0][tr][e] = s;
    if (dst && e < E && t0 + tr < T) dst[(size_t)(t0 + tr) * E + e] = s;
  }
  if (S > 1) return; // router_select_kernel adds the slices and routes
  __syncthreads();

  constexpr int EPL = (EP + 63) / 64;
  for (int j = 0; j < kRouterTok / kRouterWaves; ++j) {
    const int tr = wave * (kRouterTok / kRouterWaves) + j;
    const int t = t0 + tr;
    if (t >= T) break; // wavefront-uniform
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? part[0][tr][e] : 0.0f;
    }
    topk_softmax<EPL>(v, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
  }
}

// One wavefront per token: the S slices' partial logits added in slice
// order, written to logits if asked, then routed.
template <int EPL>
__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ part, int T,
                                                            int E, int k, int S,
                                                            float *__restrict__ logits,
                                                            int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return; // wavefront-uniform
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float s = 0.0f;
    if (e < E) {
      s = part[(size_t)t * E + e];
      for (int j = 1; j < S; ++j) s += part[((size_t)j * T + t) * E + e];
      if (logits) logits[(size_t)t * E + e] = s;
    }
    v[i] = s;
  }
  topk_softmax<EPL>(v, E, k, lane, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

bool router_fits(int H, int E) { return H % 64 == 0 && E >= 1 && E <= 128; }

hipError_t launch_router(const uint16_t *x, const uint16_t *w, int T, int H, int E, int k,
                         float *logits, int32_t *topk_idx, float *topk_w, void *ws,
                         hipStream_t stream) {
  const int S = router_splits(T, H);
  float *part = S > 1 ? static_cast<float *>(ws) : nullptr;
  const dim3 grid((T + kRouterTok - 1) / kRouterTok, S), block(64 * kRouterWaves);
  const int nt = (E + 31) / 32;
  if (nt <= 1)
    router_kernel<1><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w);
  else if (nt == 2)
    router_kernel<2><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w);
  else if (nt == 3)
    router_kernel<3><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w);
  else
    router_kernel<4><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w);
  if (S > 1) {
    const dim3 g2((T + 3) / 4);
    if (E <= 64)
      router_select_kernel<1><<<g2, 256, 0, stream>>>(part, T, E, k, S, logits, topk_idx, topk_w);
    else
      router_select_kernel<2><<<g2, 256, 0, stream>>>(part, T, E, k, S, logits, topk_idx, topk_w);
  }
  return hipGetLastError();
}

} // namespace moe
