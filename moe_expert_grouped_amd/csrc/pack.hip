// pack.hip -- the interleaved gate/up weight layout (MOE_B_KN_GATE_UP of
// include/moe.h) from separate gate and up weights [E][K][N]: row k of
// expert e becomes, for each block b of 128 output columns, 128 gate columns
// then the same 128 up columns.  A copy of 16 bytes per thread (HBM-bound:
// 2 x 2 E K N bytes read and written), done once when the weights are
// loaded; the gate/up GEMM then streams each k row of a weight tile as one
// contiguous 512-byte piece.
#include "common.h"

namespace moe {

// one thread per 16-byte output vector: rows = E K, n16 = N / 8 vectors per
// source row, 2 n16 per output row
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const u32x4 *__restrict__ gate,
                                                           const u32x4 *__restrict__ up,
                                                           long rows, int n16,
                                                           u32x4 *__restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * 2 * n16) return;
  const long r = i / (2 * n16);
  const int v = (int)(i - r * 2 * n16); // output vector inside the row
  const int blk = v >> 5;               // 256 output columns = 32 vectors per 128-column block
  const int w = v & 31;
  const u32x4 *src = (w >> 4) ? up : gate;
  out[i] = src[r * n16 + blk * 16 + (w & 15)];
}

hipError_t launch_pack_gate_up(const uint16_t *gate, const uint16_t *up, int E, int K, int N,
                               uint16_t *out, hipStream_t stream) {
  const long rows = (long)E * K;
  const int n16 = N / 8;
  const long total = rows * 2 * n16;
  pack_gate_up_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const u32x4 *>(gate), reinterpret_cast<const u32x4 *>(up), rows, n16,
      reinterpret_cast<u32x4 *>(out));
  return hipGetLastError();
}

} // namespace moe
