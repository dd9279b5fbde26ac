// combine.hip -- the top-k weighted reduction back to token order (the
// "epilogue + top-k weighted reduction" of the MoE layer1 row in
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
      const int row = pair_to_row[(size_t)t * k + j];
      wt[j] = w[(size_t)t * k + j];
      q[j] = *reinterpret_cast<const u32x4 *>(y + (size_t)row * H + col);
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
    o[h] = (uint32_t)f32_to_bf16(acc[2 * h]) | ((uint32_t)f32_to_bf16(acc[2 * h + 1]) << 16);
  *reinterpret_cast<u32x4 *>(out + (size_t)t * H + col) = o;
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

} // namespace moe
