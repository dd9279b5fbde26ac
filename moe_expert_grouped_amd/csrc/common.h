// common.h -- device helpers shared by the HIP kernels of the MoE library
// (gfx950 / CDNA4 only).  Nothing here is shared with the oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_LDS __attribute__((address_space(3)))

namespace moe {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kRowBlock = 128; // rows per task / expert alignment unit

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Direct global->LDS DMA.  Issued through inline asm so that the compiler
// neither tracks these loads nor inserts its own (conservative) waits for
// them: lane i of the wavefront writes bytes [16 i, 16 i + 16) (or [4 i, 4 i
// + 4) for the dword form) after the wave-uniform LDS byte address in M0
// (one wait state between the M0 write and its use).  Completion is awaited
// explicitly with wait_vmcnt; loads complete in issue order.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(lds_addr)
               : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (SGPR pair) and a 32-bit per-lane
// byte offset: the per-lane state is one register instead of a pointer.
// NT: the non-temporal (streaming) cache policy, for data read about once.
template <bool NT>
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff),
                 "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
                 "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g),
               "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
  return (uint32_t)(uintptr_t)(const MOE_LDS void *)p;
}

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// LDS wait through the builtin, so the compiler's own wait insertion knows
// the reads issued before it have completed (encoding: vmcnt and expcnt at
// their maximum, lgkmcnt 0)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Two fp32 values -> a packed pair (a in the low half), round-to-nearest-
// even: one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// fp32 -> bf16, round-to-nearest-even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Inclusive prefix sum across the 64 lanes of a wavefront, with DPP lane
// moves (no LDS permutes): shifts right by 1, 2, 4, 8 inside each row of 16
// lanes (lanes shifted in from outside the row add 0), then row r adds the
// last lane of row r - 1 (rows 1 and 3) and rows 2 and 3 add lane 31.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31
  return v;
}

// Inclusive max-scan across the 64 lanes of a wavefront, the same lane moves
// (lanes shifted in from outside a row, or masked off, contribute -1: every
// value scanned is >= -1).
__device__ __forceinline__ int wave_incl_max_scan(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x111, 0xf, 0xf, false)); // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x112, 0xf, 0xf, false)); // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x114, 0xf, 0xf, false)); // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x118, 0xf, 0xf, false)); // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x142, 0xa, 0xf, false)); // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x143, 0xc, 0xf, false)); // row_bcast:31
  return v;
}

// Row-task plan of the grouped GEMM, built on the device from the block
// groups and the padded row count: plan[0] = number of row tasks, plan[1] =
// number of blocks, then per row task i (one or two consecutive 128-row
// blocks of one group, paired from the first block of each run of equal
// groups):  plan[2 + 2 i] = first block | (blocks - 1) << 30,
//           plan[3 + 2 i] = group.
constexpr int kPlanHead = 2;
constexpr int kPlanTwo = 1 << 30;
inline size_t plan_ints(int cap) { return kPlanHead + 2 * (size_t)(cap / kRowBlock); }

// Split K (the grouped GEMM's SK form and the reductions after it): the k
// parts, at most `max_parts` (1, 2 or 4), of a GEMM of `tasks` (row task,
// column block) tasks on `grid` persistent workgroups, decided from the
// task count the routing gave (the plan), so the GEMM and its reduction agree
// without the host.  1 unless the tasks leave at least a quarter of the
// workgroups idle (with 3/4 of them busy the weight stream already draws
// about all the HBM bandwidth it gets: measured); otherwise the part count
// that gives the busiest workgroup the least work -- items of 1/p of the
// k range, ceil(ceil(tasks p / XCDs) / workgroups per XCD) of them, as the
// persistent schedule deals them out -- the fewer parts on a tie.
__host__ __device__ inline int splitk_parts_for(int tasks, int grid, int max_parts) {
  if (tasks <= 0 || 4L * tasks > 3L * grid - 1) return 1;
  const int nx = grid % 8 == 0 ? 8 : 1, S = grid / nx;
  int best = 1;
  long best_items = ((long)tasks + nx - 1) / nx;
  best_items = (best_items + S - 1) / S;
  for (int p = 2; p <= max_parts; p *= 2) {
    long items = ((long)tasks * p + nx - 1) / nx;
    items = (items + S - 1) / S;
    if (items * best < best_items * p) { // items / p < best_items / best
      best = p;
      best_items = items;
    }
  }
  return best;
}

} // namespace moe
