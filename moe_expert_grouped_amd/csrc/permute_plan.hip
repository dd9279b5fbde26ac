// permute_plan.hip -- the reorder by route and the grouped GEMM's row-task
// plan in one launch, for routings of up to 16384 (token, slot) pairs (the
// MoE layer0 row of "Comm-compute fusion (1)", section 4: reorder the rows by
// expert into the 128-row-aligned groups of the grouped GEMM template,
// "Comm-compute fusion (3)", section 4).
//
// The same results as the counting-sort passes of permute.hip followed by
// the plan kernel of the grouped GEMM, without the grid-wide steps between
// them: every workgroup loads the whole routing (16 ids per thread at most)
// and builds the histogram, the padded offsets and the plan offsets in LDS;
// then workgroup g places the pairs of experts g, g + G, ...: a thread's
// pairs are consecutive, so one block-wide prefix sum of per-thread matches
// gives every pair its rank (stable: ascending pair index within an
// expert).  The redundant loads are G times 4 T k bytes of L2 reads, small
// at these sizes; one launch instead of four (histogram, scan, scatter,
// plan) saves their latencies, which is what these steps are bound by.
// Expert ids outside [0, E) are skipped (the pair gets row -1).
#include "common.h"

namespace moe {

constexpr int kRPThreads = 1024;
constexpr int kRPMaxExperts = 1024;
constexpr int kRPWaves = kRPThreads / 64;
constexpr int kRPMaxPairs = 16384; // pairs per routing on this path

// Histogram copies: one per wavefront while they fit in 16 KiB.
__host__ __device__ inline int hist_copies(int E) {
  const int c = 4096 / E;
  return c >= kRPWaves ? kRPWaves : (c < 1 ? 1 : c);
}

struct PPArgs {
  const int32_t *idx;       // [T*k] expert of each pair
  const int32_t *counts_in; // [E] pairs per expert, if already counted (the router's), or NULL
  int T, E, k, cap;
  int32_t *counts, *offsets, *pair_to_row, *row_to_pair, *block_expert, *num_padded_rows;
  int32_t *plan; // optional: the row-task plan
};

// Thread tid holds pairs tid * NS .. tid * NS + NS - 1.
template <int NS>
__global__ __launch_bounds__(kRPThreads) void permute_plan_kernel(PPArgs a) {
  extern __shared__ int hist[]; // [hist_copies(E)][E]
  __shared__ int cnt[kRPMaxExperts];
  __shared__ int off[kRPMaxExperts + 1];
  __shared__ int toff[kRPMaxExperts + 1];
  __shared__ int wtot[kRPWaves];
  __shared__ int wtot2[kRPWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = gridDim.x;
  const int T = a.T, E = a.E, k = a.k;
  const long R = (long)T * k;
  const bool owner = tid % G == (int)blockIdx.x; // writes the rows of this thread's skipped pairs

  // up to one histogram per wavefront (wavefront w counts into copy w %
  // copies; no contention between the wavefronts of different copies),
  // cleared while the routing loads are in flight
  const int copies = hist_copies(E);
  for (int i = tid; i < copies * E; i += kRPThreads) hist[i] = 0;
  int key[NS];
  auto pair_of = [&](int u) -> long { return (long)tid * NS + u; };
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const long p = pair_of(u);
    const int e = p < R ? a.idx[p] : -1;
    key[u] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  if (a.counts_in) {
    // counted by the router front end in its launch
    for (int e = tid; e < E; e += kRPThreads) cnt[e] = a.counts_in[e];
  } else {
    int *my_hist = hist + __builtin_amdgcn_readfirstlane(wave % copies) * E;
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (key[u] >= 0) atomicAdd(&my_hist[key[u]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kRPThreads) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < copies; ++w) c += hist[w * E + e];
      cnt[e] = c;
    }
  }
  __syncthreads();

  // padded offsets and first row task of every expert (one thread per expert)
  const int padded = tid < E ? (cnt[tid] + kRowBlock - 1) / kRowBlock * kRowBlock : 0;
  const int tasks = (padded / kRowBlock + 1) / 2;
  const int incl = wave_incl_scan(padded);
  const int incl2 = wave_incl_scan(tasks);
  if (lane == 63) {
    wtot[wave] = incl;
    wtot2[wave] = incl2;
  }
  __syncthreads();
  int before = 0, before2 = 0;
  for (int w = 0; w < wave; ++w) {
    before += wtot[w];
    before2 += wtot2[w];
  }
  if (tid < E) {
    off[tid] = before + incl - padded;
    toff[tid] = before2 + incl2 - tasks;
  }
  if (tid == E - 1) {
    off[E] = before + incl;
    toff[E] = before2 + incl2;
  }
  __syncthreads();
  const int m_pad = off[E];
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kRPThreads) {
      if (a.counts != a.counts_in) a.counts[e] = cnt[e];
      a.offsets[e] = off[e];
    }
    if (tid == 0) {
      a.offsets[E] = m_pad;
      a.num_padded_rows[0] = m_pad;
      if (a.plan) {
        a.plan[0] = toff[E];
        a.plan[1] = m_pad / kRowBlock;
      }
    }
  }

  // the experts of this workgroup
  for (int e = blockIdx.x; e < E; e += G) {
    int m = 0;
#pragma unroll
    for (int u = 0; u < NS; ++u) m += key[u] == e;
    const int mi = wave_incl_scan(m);
    __syncthreads(); // every thread is done reading wtot
    if (lane == 63) wtot[wave] = mi;
    __syncthreads();
    int row = off[e] + mi - m;
    for (int w = 0; w < wave; ++w) row += wtot[w];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (key[u] == e) {
        const long p = pair_of(u);
        a.pair_to_row[p] = row;
        a.row_to_pair[row] = (int32_t)p;
        ++row;
      }
    }
    const int r0 = off[e], r1 = off[e + 1];
    for (int r = r0 + cnt[e] + tid; r < r1; r += kRPThreads) a.row_to_pair[r] = -1;
    const int b0 = r0 / kRowBlock, nb = (r1 - r0) / kRowBlock;
    for (int b = tid; b < nb; b += kRPThreads) a.block_expert[b0 + b] = e;
    if (a.plan) {
      for (int q = tid; 2 * q < nb; q += kRPThreads) {
        const int i = toff[e] + q;
        a.plan[kPlanHead + 2 * i] = (b0 + 2 * q) | (2 * q + 1 < nb ? kPlanTwo : 0);
        a.plan[kPlanHead + 2 * i + 1] = e;
      }
    }
  }

  // rows and blocks past M_pad, shared out over the workgroups
  for (int r = m_pad + (int)blockIdx.x * kRPThreads + tid; r < a.cap; r += G * kRPThreads)
    a.row_to_pair[r] = -1;
  for (int b = m_pad / kRowBlock + (int)blockIdx.x * kRPThreads + tid; b < a.cap / kRowBlock;
       b += G * kRPThreads)
    a.block_expert[b] = -1;
  // pairs without a valid expert
  if (owner) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (key[u] < 0 && pair_of(u) < R) a.pair_to_row[pair_of(u)] = -1;
  }
}

// Whether the one-launch path takes this shape.  The callers check cap >=
// the padded capacity.
bool permute_plan_fits(int T, int E, int k) {
  const long R = (long)T * k;
  return R <= kRPMaxPairs && E >= 1 && E <= kRPMaxExperts && k >= 1;
}

// The permutation maps, block experts and, with plan non-NULL, the row-task
// plan of the routing idx.
// counts_in: the pairs per expert if counted already (the router front end's
// histogram; every id then lies in [0, E)), else NULL.
hipError_t launch_permute_plan(const int32_t *idx, int T, int E, int k, int cap, int32_t *counts,
                               int32_t *offsets, int32_t *pair_to_row, int32_t *row_to_pair,
                               int32_t *block_expert, int32_t *num_padded_rows, int32_t *plan,
                               hipStream_t stream, const int32_t *counts_in) {
  if (!permute_plan_fits(T, E, k)) return hipErrorInvalidValue;
  PPArgs a{idx, counts_in, T, E, k, cap, counts, offsets, pair_to_row, row_to_pair, block_expert,
           num_padded_rows, plan};
  const int G = E; // one workgroup per expert
  const size_t hist_bytes = (size_t)hist_copies(E) * E * sizeof(int); // <= 16 KiB
  const long R = (long)T * k;
  const int ns = (int)((R + kRPThreads - 1) / kRPThreads);
#define MOE_PP(NSV)                                                                           \
  if (ns <= NSV) {                                                                            \
    permute_plan_kernel<NSV><<<G, kRPThreads, hist_bytes, stream>>>(a);                       \
    return hipGetLastError();                                                                 \
  }
  MOE_PP(1) MOE_PP(2) MOE_PP(4) MOE_PP(8) MOE_PP(16)
#undef MOE_PP
  return hipErrorInvalidValue;
}

} // namespace moe
