// combine.hip -- the top-k weighted reduction back to token order (the step
// after the down GEMM in the MoE layer1 row of the dataflow table in
// "Comm-compute fusion (1)", section 4):
//   out[t][n] = round_bf16( sum_{j<k} w[t][j] * y[pair_to_row[t*k+j]][n] ).
//
// HBM-bound: it reads k rows of y and writes one row of out per token
// (2*T*k*H + 2*T*H bytes), 16-byte vectors (8 bf16 per lane), accumulating
// in fp32 in slot order, so each output element is one deterministic sum.
#include "common.h"

namespace moe {

// One wavefront per (token, 512-column chunk): 64 lanes x 8 bf16.  A token
// row of H = 4096 is 8 wavefronts, so a T = 2048 combine runs 16K wavefronts
// (64 per CU) with k 16-byte loads in flight each.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ y, int H,
                                                      const int32_t *__restrict__ pair_to_row,
                                                      const float *__restrict__ w, int T,
                                                      int k, uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int chunks = (H + 511) / 512;
  const long wid = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int t = (int)(wid / chunks);
  if (t >= T) return;
  const int col = (int)(wid - (long)t * chunks) * 512 + lane * 8;
  if (col >= H) return;
  u32x4 q[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      // a pair without a row (routed to no valid expert) adds nothing
      const int row = pair_to_row[(size_t)t * k + j];
      wt[j] = row >= 0 ? w[(size_t)t * k + j] : 0.0f;
      q[j] = row >= 0 ? *reinterpret_cast<const u32x4 *>(y + (size_t)row * H + col)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[2 * h] = fmaf(wt[j], __uint_as_float(q[j][h] << 16), acc[2 * h]);
        acc[2 * h + 1] = fmaf(wt[j], __uint_as_float(q[j][h] & 0xffff0000u), acc[2 * h + 1]);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 4; ++h)
    o[h] = pack2_bf16(acc[2 * h], acc[2 * h + 1]);
  // non-temporal: the output is written once and not read here
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + (size_t)t * H + col));
}

hipError_t launch_combine(const uint16_t *y, int H, const int32_t *pair_to_row, const float *w,
                          int T, int k, uint16_t *out, hipStream_t stream) {
  const long waves = (long)T * ((H + 511) / 512);
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (k <= 1)
    combine_kernel<1><<<grid, block, 0, stream>>>(y, H, pair_to_row, w, T, k, out);
  else if (k <= 2)
    combine_kernel<2><<<grid, block, 0, stream>>>(y, H, pair_to_row, w, T, k, out);
  else if (k <= 4)
    combine_kernel<4><<<grid, block, 0, stream>>>(y, H, pair_to_row, w, T, k, out);
  else if (k <= 8)
    combine_kernel<8><<<grid, block, 0, stream>>>(y, H, pair_to_row, w, T, k, out);
  else
    combine_kernel<16><<<grid, block, 0, stream>>>(y, H, pair_to_row, w, T, k, out);
  return hipGetLastError();
}

// Finalize of the weighted-scatter variant: out[i] = round_bf16(acc[i]),
// 8 elements (32 bytes in, 16 bytes out) per thread; the scalar tail covers
// n % 8.  HBM-bound: 6 bytes per element.
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ acc, long n,
                                                       uint16_t *__restrict__ out) {
  const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i + 8 <= n) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(acc + i);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(acc + i + 4);
    u32x4 o;
    o[0] = pack2_bf16(a[0], a[1]);
    o[1] = pack2_bf16(a[2], a[3]);
    o[2] = pack2_bf16(b[0], b[1]);
    o[3] = pack2_bf16(b[2], b[3]);
    *reinterpret_cast<u32x4 *>(out + i) = o;
  } else {
    for (long j = i; j < n; ++j) out[j] = f32_to_bf16(acc[j]);
  }
}

// Clears n floats (16 bytes per thread, scalar tail).  A kernel rather than
// a memset node, so the layer stays capturable in a HIP graph.
__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ p, long n) {
  const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 4 <= n)
    *reinterpret_cast<f32x4 *>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  else
    for (long j = i; j < n; ++j) p[j] = 0.f;
}

hipError_t launch_finalize(const float *acc, long n, uint16_t *out, hipStream_t stream) {
  const long threads = (n + 7) / 8;
  finalize_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(acc, n, out);
  return hipGetLastError();
}

hipError_t launch_zero(float *p, long n, hipStream_t stream) {
  const long threads = (n + 3) / 4;
  zero_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

} // namespace moe
