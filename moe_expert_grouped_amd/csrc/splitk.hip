// splitk.hip -- the reductions after a split-K grouped GEMM.
//
// When a layer share's routing leaves most compute units without a (row
// task, column block) task -- the wave rule of "Comm-compute fusion (1)",
// section 5: with less than one wave of tasks the machine is not filled --
// the grouped GEMM cuts each task's k range into S equal parts and runs the
// parts as tasks of their own (S = splitk_parts_for(tasks, grid, max_parts)
// on the task count in the plan, 1 when the tasks fill the CUs: the GEMM and
// these kernels decide it alike, on the device).  Each part writes its raw
// fp32 sums, for the rows that carry a (token, slot) pair p, to P[s][p][m][n]
// (m: the B matrix).  These kernels add the S parts in part order, so every
// output is one deterministic sum, and apply what the GEMM's epilogue would
// have:
//   * after gate/up: h[row(p)][n] = round_bf16(SiLU(g) * u), g and u the
//     summed gate and up values, SiLU(z) = z / (1 + e^-z) through the
//     hardware reciprocal, as the GEMM's own epilogue computes it;
//   * after down, also the top-k weighted combine that section 4 of the same
//     page places after the down GEMM (its MoE layer1 row):
//     out[t][n] = round_bf16(sum_j w[t][j] * y_j[n]) with
//     y_j = round_bf16(summed parts of pair t*k+j) -- the rounding of y the
//     store epilogue and the combine kernel apply, in the same slot order;
//     y itself is never stored.
// Both are HBM-light (they touch only the pairs' rows) and latency-bound.
#include "common.h"

namespace moe {

// One thread per (pair, 4 columns).
__global__ __launch_bounds__(256) void splitk_silu_kernel(const float *__restrict__ P,
                                                          const int32_t *__restrict__ plan,
                                                          int ncol, int grid, int max_parts,
                                                          int R, int N,
                                                          const int32_t *__restrict__ pair_to_row,
                                                          uint16_t *__restrict__ h) {
  const int S = splitk_parts_for(plan[0] * ncol, grid, max_parts);
  if (S == 1) return; // not split: the GEMM's own epilogue wrote h
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = N / 4;
  const long p = i / n4;
  if (p >= R) return;
  const int c = (int)(i - p * n4) * 4;
  const int r = pair_to_row[p];
  if (r < 0) return; // routed to no valid expert: no row
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float *base = P + ((size_t)s * R + p) * 2 * N + c;
    const float4 a = *reinterpret_cast<const float4 *>(base);
    const float4 b = *reinterpret_cast<const float4 *>(base + N);
    g[0] += a.x, g[1] += a.y, g[2] += a.z, g[3] += a.w;
    u[0] += b.x, u[1] += b.y, u[2] += b.z, u[3] += b.w;
  }
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])) * u[e];
  *reinterpret_cast<uint2 *>(h + (size_t)r * N + c) =
      uint2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
}

// One thread per (token, 8 columns).  Not split (S == 1), the GEMM's own
// epilogue stored y ([rows][H] bf16 at Y, the same region), which is then
// read as the combine kernel reads it.
__global__ __launch_bounds__(256) void splitk_combine_kernel(
    const float *__restrict__ P, const uint16_t *__restrict__ Y, const int32_t *__restrict__ plan,
    int ncol, int grid, int max_parts, int T, int k, int H,
    const int32_t *__restrict__ pair_to_row, const float *__restrict__ w,
    uint16_t *__restrict__ out) {
  const int S = splitk_parts_for(plan[0] * ncol, grid, max_parts);
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int h8 = H / 8;
  const long t = i / h8;
  if (t >= T) return;
  const int c = (int)(i - t * h8) * 8;
  const size_t R = (size_t)T * k;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const size_t p = (size_t)t * k + j;
    const int r = pair_to_row[p];
    if (r < 0) continue; // a pair without a row adds nothing
    u32x4 q; // y of the pair, 8 bf16 values
    if (S == 1) {
      q = *reinterpret_cast<const u32x4 *>(Y + (size_t)r * H + c);
    } else {
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < S; ++s) {
        const float *base = P + ((size_t)s * R + p) * H + c;
        const float4 a = *reinterpret_cast<const float4 *>(base);
        const float4 b = *reinterpret_cast<const float4 *>(base + 4);
        y[0] += a.x, y[1] += a.y, y[2] += a.z, y[3] += a.w;
        y[4] += b.x, y[5] += b.y, y[6] += b.z, y[7] += b.w;
      }
      // rounded to bf16 as the store epilogue rounds y
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = pack2_bf16(y[2 * e], y[2 * e + 1]);
    }
    const float wj = w[p];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(wj, __uint_as_float(q[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(wj, __uint_as_float(q[e] & 0xffff0000u), acc[2 * e + 1]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(acc[2 * e], acc[2 * e + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + (size_t)t * H + c));
}

// P: the partials; plan: the GEMM's row-task plan; ncol: its column blocks;
// grid: its workgroups; max_parts: the part bound it was launched with.
hipError_t launch_splitk_silu(const float *P, const int32_t *plan, int ncol, int grid,
                              int max_parts, int R, int N, const int32_t *pair_to_row,
                              uint16_t *h, hipStream_t stream) {
  const long n = (long)R * (N / 4);
  splitk_silu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      P, plan, ncol, grid, max_parts, R, N, pair_to_row, h);
  return hipGetLastError();
}

hipError_t launch_splitk_combine(const float *P, const uint16_t *Y, const int32_t *plan,
                                 int ncol, int grid, int max_parts, int T, int k, int H,
                                 const int32_t *pair_to_row, const float *w, uint16_t *out,
                                 hipStream_t stream) {
  const long n = (long)T * (H / 8);
  splitk_combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      P, Y, plan, ncol, grid, max_parts, T, k, H, pair_to_row, w, out);
  return hipGetLastError();
}

} // namespace moe
