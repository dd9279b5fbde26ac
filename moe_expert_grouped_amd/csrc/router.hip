// router.hip -- the router front end: logits = x . W^T and the routing of
// those logits (one launch, or two when the hidden dimension is sliced).
//
// The pages take the router logits as given (the route that the reorder of
// "Comm-compute fusion (1)", section 4 follows); the step before them is the
// linear router, logits[t][e] = x[t] . W[e] with W stored [E][H], fp32
// accumulation of bf16 products.  The selection and the weights are exactly
// those of moe_route (topk_softmax in topk.h), taken on the fp32 logits
// computed here.
//
// Design (gfx950): one 4-wavefront workgroup per (32 tokens, hidden slice).
// A routing of few tokens cuts H into up to 16 slices so the launch still
// covers the chip.  The slice streams through a 4-stage LDS ring in chunks of
// 64 hidden values -- 128 bytes of every x row and W row, one whole cache
// line -- by direct global->LDS DMA, 8 rows per instruction: loading the
// 32x32x16 operands straight into registers touches 32 rows per instruction
// and is bound by the request rate, not by bytes.  In each chunk wavefront w
// takes k step w (16 of the 64 values) for every 32-expert column tile:
// its A fragment (32 token rows x 16) and B fragments (32 W rows x 16) are
// one 16-byte LDS read per lane each, the 16-byte granules of a row XOR-
// swizzled by row / 2 so that 16 consecutive rows hit 16 distinct bank
// groups.  The four wavefronts' [32 x E] tiles meet in LDS (in the ring,
// once the last chunk is consumed) and are summed in wavefront order; with
// one slice each wavefront then routes 8 of the tokens, with several the
// slices' partial logits go to a workspace and a second launch adds them in
// slice order and routes (one fixed rounding order either way).  (128-token
// workgroups, which read half the W bytes per token, need 16 slices at
// T = 2048, and their partials then cost as much as x.)  The kernel
// boundary is the grid-wide step here: a one-launch form in which the last
// of a token block's slices to arrive (a compare-and-swap on a per-block
// word) adds the slices ran 24.0 us against 10.1 us for the two launches at
// T = 2048, and a grid-wide last arriver for the histogram 67 us -- each
// device-scope atomic round trip costs microseconds on this part.
//
// The routing kernel also counts the chosen experts (the histogram the
// permutation starts from): a per-workgroup LDS histogram, then one
// device-scope add per expert into expert_counts, issued without waiting
// for a result.  The counts are cleared by the first launch when the hidden
// dimension is sliced, else by a one-workgroup clearing launch before it.
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

constexpr int kRouterChunk = 64; // hidden values per ring stage (128 bytes of a row)
constexpr int kRouterStages = 4;

// LDS position of 16-byte granule g of ring row r (8 granules per row)
__device__ __forceinline__ int router_swz(int g, int r) { return g ^ ((r >> 1) & 7); }

// Workgroup (b, s): tokens 32 b .. 32 b + 31, hidden slice s (of S); with
// S == 1 it also routes its tokens, else it writes its [32 x E] partial
// logits to part_out[s] for router_select_kernel.
// NT 32-expert column tiles: E <= 32 NT
template <int NT>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ w, int T, int H,
                                                     int E, int k, int S, float *__restrict__ part_out,
                                                     float *__restrict__ logits,
                                                     int32_t *__restrict__ topk_idx,
                                                     float *__restrict__ topk_w,
                                                     int32_t *__restrict__ counts) {
  constexpr int EP = 32 * NT;                // expert columns computed
  constexpr int LD = EP + 1;                 // LDS row stride of the partial tiles, in floats
  constexpr int XB = kRouterTok * 128;       // x bytes of a stage: 32 rows x 128 bytes
  constexpr int SB = XB + EP * 128;          // stage bytes: then EP rows of W
  constexpr int NI = 1 + NT;                 // DMA instructions per wavefront per chunk
  static_assert(kRouterTok == 8 * kRouterWaves, "one x instruction per wavefront");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRouterStages * SB];
  __shared__ int32_t s_hist[32 * NT];
  // after the last chunk the ring holds the wavefronts' partial tiles
  static_assert(sizeof(float) * kRouterWaves * kRouterTok * LD <= kRouterStages * SB, "fits");
  float(*part)[kRouterTok][LD] = reinterpret_cast<float(*)[kRouterTok][LD]>(ring);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kRouterTok;
  const int hs = H / S; // this workgroup's hidden slice, a multiple of 64
  const int h0 = blockIdx.y * hs;
  const int nchunk = hs / kRouterChunk;

  // DMA instruction j of a chunk fills ring rows 8 j .. 8 j + 7 (x rows for
  // j < 4, then W rows); wavefront w issues j = w and j = 4 + w + 4 m.  Lane
  // l writes granule l % 8 of row 8 j + l / 8, so it fetches the row's
  // granule router_swz(l % 8, row).  Rows past T and experts past E read the
  // last valid row: their products are never written or selected.
  const int rr = lane >> 3; // row within the instruction
  const int xrow = 8 * wave + rr;
  const int tok = min(t0 + xrow, T - 1);
  const uint16_t *xs = x + (size_t)tok * H + h0 + 8 * router_swz(lane & 7, xrow);
  const uint16_t *wsrc[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const int wr = 8 * (wave + 4 * m) + rr;
    wsrc[m] = w + (size_t)min(wr, E - 1) * H + h0 + 8 * router_swz(lane & 7, wr);
  }
  const uint32_t ring_lds = lds_addr_of(ring);
  auto issue = [&](int c) {
    const uint32_t st = ring_lds + (c % kRouterStages) * SB;
    dma16(xs + c * kRouterChunk, st + wave * 1024);
#pragma unroll
    for (int m = 0; m < NT; ++m) dma16(wsrc[m] + c * kRouterChunk, st + XB + (wave + 4 * m) * 1024);
  };

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};
  // operand rows of this lane (token row, and W row 32 n + row of tile n)
  // and the granule of this wavefront's k step: lane half q holds hidden
  // values 8 q .. 8 q + 7 of the step (the 32x32x16 operand layouts)
  const int row = lane & 31;
  const int gpos = router_swz(2 * wave + (lane >> 5), row) * 16;

  const int pre = min(kRouterStages - 1, nchunk);
  for (int c = 0; c < pre; ++c) issue(c);
  for (int c = 0; c < nchunk; ++c) {
    // chunk c has landed for this wavefront once only the chunks issued
    // after it (at most kRouterStages - 2) are in flight; the barrier makes
    // it so for every wavefront, and frees the stage of chunk c - 1
    const int after = min(kRouterStages - 2, nchunk - 1 - c);
    if (after >= 2)
      wait_vmcnt<2 * NI>();
    else if (after == 1)
      wait_vmcnt<NI>();
    else
      wait_vmcnt<0>();
    block_barrier();
    if (c + kRouterStages - 1 < nchunk) issue(c + kRouterStages - 1);
    const MOE_LDS unsigned char *sb =
        (const MOE_LDS unsigned char *)ring + (c % kRouterStages) * SB;
    const bf16x8 a = *(const MOE_LDS bf16x8 *)(sb + row * 128 + gpos);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 b = *(const MOE_LDS bf16x8 *)(sb + XB + (32 * n + row) * 128 + gpos);
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
    }
  }

  // every wavefront is done reading the ring (the last wait was for all DMA)
  __syncthreads();
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
  if (S > 1) {
    // router_select_kernel adds the slices, routes and counts; the counts
    // start from zero (that launch follows this one)
    if (counts && blockIdx.x == 0 && blockIdx.y == 0)
      for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
    return;
  }
  for (int e = threadIdx.x; e < EP; e += blockDim.x) s_hist[e] = 0;
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
    const int chosen = topk_softmax<EPL>(v, E, k, lane, topk_idx + (size_t)t * k,
                                         topk_w + (size_t)t * k);
    if (counts && lane < k) atomicAdd(&s_hist[chosen], 1);
  }
  if (!counts) return;
  __syncthreads();
  // cleared by the launch before this one
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (s_hist[e]) atomicAdd(&counts[e], s_hist[e]);
}

// One wavefront per token: the S slices' partial logits added in slice
// order, written to logits if asked, then routed.
// Token t of router_select_kernel (one wavefront): the S slices' partial
// logits added in slice order, written to logits if asked, then routed;
// with hist, its choices counted there.
template <int EPL>
__device__ __forceinline__ void select_one(const float *__restrict__ part, int T, int E, int k,
                                           int S, float *__restrict__ logits,
                                           int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, int t, int lane,
                                           int32_t *hist) {
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
  const int chosen = topk_softmax<EPL>(v, E, k, lane, topk_idx + (size_t)t * k,
                                       topk_w + (size_t)t * k);
  if (hist && lane < k) atomicAdd(&hist[chosen], 1);
}

// 16 tokens per 1024-thread workgroup, whose choices are counted in LDS and
// added into counts (cleared by router_kernel).
template <int EPL>
__global__ __launch_bounds__(1024) void router_select_kernel(const float *__restrict__ part, int T,
                                                             int E, int k, int S,
                                                             float *__restrict__ logits,
                                                             int32_t *__restrict__ topk_idx,
                                                             float *__restrict__ topk_w,
                                                             int32_t *__restrict__ counts) {
  __shared__ int32_t s_hist[64 * EPL];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (int e = threadIdx.x; e < 64 * EPL; e += blockDim.x) s_hist[e] = 0;
  __syncthreads();
  if (t < T) select_one<EPL>(part, T, E, k, S, logits, topk_idx, topk_w, t, lane,
                             counts ? s_hist : nullptr);
  if (!counts) return;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (s_hist[e]) atomicAdd(&counts[e], s_hist[e]);
}

bool router_fits(int H, int E) { return H % 64 == 0 && E >= 1 && E <= 128; }

// Clears expert_counts before a routing kernel that adds into it.
__global__ void router_clear_counts(int32_t *__restrict__ counts, int E) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
}

hipError_t launch_router(const uint16_t *x, const uint16_t *w, int T, int H, int E, int k,
                         float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts,
                         void *ws, hipStream_t stream) {
  const int S = router_splits(T, H);
  float *part = S > 1 ? static_cast<float *>(ws) : nullptr;
  if (counts && S == 1) router_clear_counts<<<1, 256, 0, stream>>>(counts, E);
  const dim3 grid((T + kRouterTok - 1) / kRouterTok, S), block(64 * kRouterWaves);
  const int nt = (E + 31) / 32;
  if (nt <= 1)
    router_kernel<1><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w, counts);
  else if (nt == 2)
    router_kernel<2><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w, counts);
  else if (nt == 3)
    router_kernel<3><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w, counts);
  else
    router_kernel<4><<<grid, block, 0, stream>>>(x, w, T, H, E, k, S, part, logits, topk_idx,
                                                 topk_w, counts);
  if (S > 1) {
    const dim3 g2((T + 15) / 16);
    if (E <= 64)
      router_select_kernel<1><<<g2, 1024, 0, stream>>>(part, T, E, k, S, logits, topk_idx, topk_w,
                                                       counts);
    else
      router_select_kernel<2><<<g2, 1024, 0, stream>>>(part, T, E, k, S, logits, topk_idx, topk_w,
                                                       counts);
  }
  return hipGetLastError();
}

} // namespace moe
