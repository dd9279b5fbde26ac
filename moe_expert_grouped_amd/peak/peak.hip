// peak.hip -- measured peaks of the part, reported next to the published
// ones: an MFMA-only loop (bf16 v_mfma_f32_32x32x16, no memory traffic) and a
// read-only HBM stream (16-byte loads, one contiguous part per
// workgroup).  Measurement only: the
// MoE path never calls these; they live in their own library,
// libmoe_peak_gfx950.so (include/moe_peak.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_peak.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8; // independent accumulators per wavefront

// Every wavefront issues iters * kChains MFMAs; the chains are independent so
// the matrix core never waits on a previous result.  The operands depend on
// the thread id so nothing folds; one value per thread is written only if it
// equals an impossible sentinel, so the loop cannot be removed and no memory
// traffic is generated.
__global__ __launch_bounds__(256) void mfma_loop(int iters, float *sink) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 1e-3f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(1.0f - 1e-3f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 c[kChains];
  for (int j = 0; j < kChains; ++j)
    for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < kChains; ++j)
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == -1.2345f) sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each workgroup reads its own contiguous part of the n16 16-byte vectors
// (n16 / gridDim.x of them; the last one also takes the remainder), 4 KiB per
// step across its 256 threads, 8 steps in flight per thread -- the pattern
// that streamed fastest among grid-stride, per-workgroup and LDS-DMA forms;
// the XOR of everything read is written only if it equals a sentinel.
__global__ __launch_bounds__(256) void read_stream(const u32x4 *__restrict__ p, size_t n16,
                                                   unsigned *sink) {
  const size_t per = n16 / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = blockIdx.x + 1 == gridDim.x ? n16 : b0 + per;
  size_t i = b0 + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < b1; i += 256) acc ^= p[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[blockIdx.x] = acc[0];
}

} // namespace

extern "C" {

long long moe_peak_mfma_flops(int workgroups, int iters) {
  if (workgroups <= 0 || iters <= 0) return -1;
  // 4 wavefronts per workgroup, kChains MFMAs of 32 x 32 x 16 (2 flop each)
  return (long long)workgroups * 4 * iters * kChains * (2LL * 32 * 32 * 16);
}

int moe_peak_mfma(int workgroups, int iters, float *sink, void *stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return 1;
  mfma_loop<<<workgroups, 256, 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int moe_peak_read(const void *buf, size_t bytes, int workgroups, unsigned *sink, void *stream) {
  if (!buf || !sink || bytes < 16 || workgroups <= 0) return 1;
  if (((uintptr_t)buf & 15u) != 0) return 1;
  read_stream<<<workgroups, 256, 0, (hipStream_t)stream>>>((const u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

} // extern "C"
