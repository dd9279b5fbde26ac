// permute.hip -- reorder (token, slot) pairs into expert-contiguous,
// 128-row-aligned blocks (the "reorder by route" of the MoE layer0 row in
// "Comm-compute fusion (1)", section 4; 128 rows is the task and expert
// alignment unit of the grouped GEMM template in "Comm-compute fusion (3)",
// section 4).
//
// The order is a stable counting sort by expert: within an expert, rows
// follow ascending pair index p = t*k + j.  No atomic operation decides a
// position, so every run produces the same bits.
//
//   pass 1  permute_hist     one workgroup per chunk of 1024 pairs: per-expert
//                            counts of the chunk (LDS counters; counting is
//                            order-free), written expert-major [E][chunks]
//   pass 2  permute_scan     one workgroup: per-expert totals, padded
//                            exclusive offsets, M_pad, per-(expert, chunk)
//                            first rows, and the expert of every row block
//   pass 3  permute_scatter  one workgroup per chunk: the stable rank of each
//                            pair inside its chunk (64-lane ballots match
//                            equal experts inside a wavefront; per-wave counts
//                            in LDS order the wavefronts), then the row maps;
//                            the same grid marks padding rows with -1
//   pass 4  permute_gather   optional: x_perm[row] = x[token of row] below
//                            M_pad (each x row read once, stored to its k
//                            rows), zero rows for padding (16-byte vectors)
// Routings of at most 16384 pairs take passes 1-3 in a single launch
// instead (permute_plan.hip).  On both paths a pair whose expert id lies
// outside [0, E) gets no row (pair_to_row = -1) and counts for no expert.
#include "common.h"

#include <algorithm>

namespace moe {

constexpr int kPermChunk = 1024;  // pairs per chunk
constexpr int kPermThreads = 256; // threads of the chunk kernels
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kPermThreads) void permute_hist(const int32_t *__restrict__ idx,
                                                             long R, int E, int nchunks,
                                                             int32_t *__restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const long p0 = (long)c * kPermChunk;
  const long p1 = min(p0 + kPermChunk, R);
  for (long p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1); // ids outside [0, E) get no row
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)e * nchunks + c] = cnt[e];
}

__global__ __launch_bounds__(1024) void permute_scan(
    const int32_t *__restrict__ hist, int E, int nchunks, int cap, int32_t *__restrict__ base,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ block_expert, int32_t *__restrict__ num_padded_rows) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int wave_tot[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;

  // per-expert totals
  for (int e = wave; e < E; e += nwaves) {
    int s = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int c = c0 + lane;
      s += c < nchunks ? hist[(size_t)e * nchunks + c] : 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) cnt[e] = s;
  }
  __syncthreads();

  // exclusive scan of the padded counts over experts (one thread per expert)
  const int e = threadIdx.x;
  const int padded = e < E ? (cnt[e] + kRowBlock - 1) / kRowBlock * kRowBlock : 0;
  const int incl = wave_incl_scan(padded);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  if (e < E) {
    off[e] = before + incl - padded;
    counts[e] = cnt[e];
    offsets[e] = before + incl - padded;
  }
  if (e == E - 1) {
    off[E] = before + incl;
    offsets[E] = before + incl;
    num_padded_rows[0] = before + incl;
  }
  __syncthreads();
  const int m_pad = off[E];

  // first row of every (expert, chunk): the expert's offset plus the pairs of
  // the same expert in earlier chunks
  for (int ee = wave; ee < E; ee += nwaves) {
    int carry = off[ee];
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < nchunks ? hist[(size_t)ee * nchunks + c] : 0;
      const int in = wave_incl_scan(v);
      if (c < nchunks) base[(size_t)ee * nchunks + c] = carry + in - v;
      carry += __shfl(in, 63, 64);
    }
  }

  // expert of each 128-row block: the largest e with off[e] <= row
  // (empty experts have off[e] == off[e+1] and own no block)
  const int nblk = cap / kRowBlock;
  for (int b = threadIdx.x; b < nblk; b += blockDim.x) {
    const int r = b * kRowBlock;
    int ex = -1;
    if (r < m_pad) {
      int lo = 0, hi = E - 1; // invariant: off[lo] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r)
          lo = mid;
        else
          hi = mid - 1;
      }
      ex = lo;
    }
    block_expert[b] = ex;
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter(
    const int32_t *__restrict__ idx, long R, int E, int nchunks, int cap,
    const int32_t *__restrict__ base, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ block_expert,
    int32_t *__restrict__ pair_to_row, int32_t *__restrict__ row_to_pair) {
  constexpr int kWaves = kPermThreads / 64;
  __shared__ int next_row[kMaxExperts];
  __shared__ int wcount[kWaves][kMaxExperts];
  const int c = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    next_row[e] = base[(size_t)e * nchunks + c];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcount[w][e] = 0;
  }
  int nbits = 1; // bits to tell apart ids 0..E (E = "no pair")
  while ((1 << nbits) <= E) ++nbits;
  __syncthreads();

  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  const long p0 = (long)c * kPermChunk;
  for (int sub = 0; sub < kPermChunk; sub += kPermThreads) {
    const long p = p0 + sub + threadIdx.x;
    const bool in = p < R;
    const int raw = in ? idx[p] : E;
    // a pair routed outside [0, E) takes the "no pair" key E and gets no row
    const bool valid = in && (unsigned)raw < (unsigned)E;
    const int key = valid ? raw : E;
    if (in && !valid) pair_to_row[p] = -1;
    // lanes of this wavefront holding the same key
    unsigned long long same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    const bool leader = rank == 0;
    const bool last = (same >> lane) == 1ull;
    if (valid && leader) wcount[wave][key] = __popcll(same);
    __syncthreads();
    int row = 0;
    bool last_overall = false;
    if (valid) {
      int before = 0, after = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int n = wcount[w][key];
        if (w < wave) before += n;
        if (w > wave) after += n;
      }
      row = next_row[key] + before + rank;
      last_overall = last && after == 0;
      pair_to_row[p] = row;
      row_to_pair[row] = (int32_t)p;
    }
    __syncthreads();
    if (valid && last_overall) next_row[key] = row + 1;
    if (valid && leader) wcount[wave][key] = 0;
    __syncthreads();
  }

  // padding rows (and rows beyond M_pad) of this workgroup's share get -1;
  // real rows are written above by exactly one pair, so the sets are disjoint
  const int share = (cap + nchunks - 1) / nchunks;
  const int r0 = c * share;
  const int r1 = min(r0 + share, cap);
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const int ex = block_expert[r / kRowBlock];
    if (ex < 0 || r - offsets[ex] >= counts[ex]) row_to_pair[r] = -1;
  }
}

// The row gather, token by token: one wavefront per (token, 512-column
// chunk) loads the chunk of x[t] once (64 lanes x 16 bytes) and stores it
// to the rows of the token's k pairs (pairs without a row are skipped);
// then the same grid zero-fills the chunks of the padding rows below M_pad
// (read on the device).  Rows at or past M_pad are not written.  The stores
// are non-temporal: x_perm is written once and not read back here.
__global__ __launch_bounds__(256) void permute_gather(const uint16_t *__restrict__ x, int H,
                                                      const int32_t *__restrict__ pair_to_row,
                                                      const int32_t *__restrict__ row_to_pair,
                                                      const int32_t *__restrict__ num_padded_rows,
                                                      int T, int k, int cap,
                                                      uint16_t *__restrict__ x_perm) {
  // H % 8 == 0, 16-byte vectors
  const int lane = threadIdx.x & 63;
  const long wid = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long nw = ((long)gridDim.x * blockDim.x) >> 6;
  const int chunks = (H + 511) / 512;
  const long tok_chunks = (long)T * chunks;
  for (long q = wid; q < tok_chunks; q += nw) {
    const int t = (int)(q / chunks);
    const int col = (int)(q - (long)t * chunks) * 512 + lane * 8;
    if (col >= H) continue;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(x + (size_t)t * H + col);
    for (int j = 0; j < k; ++j) {
      const int r = pair_to_row[(size_t)t * k + j];
      if (r < 0) continue;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(x_perm + (size_t)r * H + col));
    }
  }
  const int rows = min(num_padded_rows[0], cap);
  const long row_chunks = (long)rows * chunks;
  for (long q = wid; q < row_chunks; q += nw) {
    const int r = (int)(q / chunks);
    const int col = (int)(q - (long)r * chunks) * 512 + lane * 8;
    if (col >= H || row_to_pair[r] >= 0) continue;
    __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                reinterpret_cast<u32x4 *>(x_perm + (size_t)r * H + col));
  }
}

bool permute_plan_fits(int T, int E, int k);
hipError_t launch_permute_plan(const int32_t *idx, int T, int E, int k, int cap, int32_t *counts,
                               int32_t *offsets, int32_t *pair_to_row, int32_t *row_to_pair,
                               int32_t *block_expert, int32_t *num_padded_rows, int32_t *plan,
                               hipStream_t stream, const int32_t *counts_in);

size_t permute_workspace_bytes(long R, int E) {
  const long nchunks = (R + kPermChunk - 1) / kPermChunk;
  return (size_t)2 * E * nchunks * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t *idx, int T, int k, int E, const uint16_t *x, int H,
                          int32_t *counts, int32_t *offsets, int32_t *pair_to_row,
                          int32_t *row_to_pair, int32_t *block_expert,
                          int32_t *num_padded_rows, uint16_t *x_perm, int cap, void *ws,
                          hipStream_t stream) {
  if (permute_plan_fits(T, E, k)) {
    // up to 16384 pairs: one launch (permute_plan.hip)
    const hipError_t e = launch_permute_plan(idx, T, E, k, cap, counts, offsets, pair_to_row,
                                             row_to_pair, block_expert, num_padded_rows, nullptr,
                                             stream, nullptr);
    if (e != hipSuccess) return e;
  } else {
    const long R = (long)T * k;
    const int nchunks = (int)((R + kPermChunk - 1) / kPermChunk);
    int32_t *hist = reinterpret_cast<int32_t *>(ws);
    int32_t *base = hist + (size_t)E * nchunks;
    permute_hist<<<nchunks, kPermThreads, 0, stream>>>(idx, R, E, nchunks, hist);
    permute_scan<<<1, 1024, 0, stream>>>(hist, E, nchunks, cap, base, counts, offsets,
                                         block_expert, num_padded_rows);
    permute_scatter<<<nchunks, kPermThreads, 0, stream>>>(idx, R, E, nchunks, cap, base, counts,
                                                          offsets, block_expert, pair_to_row,
                                                          row_to_pair);
  }
  if (x && x_perm) {
    // four wavefronts per workgroup, one (token, chunk) each per pass
    const long waves = (long)T * ((H + 511) / 512);
    const int grid = (int)std::min<long>((waves + 3) / 4, 8192);
    permute_gather<<<grid, 256, 0, stream>>>(x, H, pair_to_row, row_to_pair, num_padded_rows, T,
                                             k, cap, x_perm);
  }
  return hipGetLastError();
}

} // namespace moe
