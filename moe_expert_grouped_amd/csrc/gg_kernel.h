// gg_kernel.h -- the grouped GEMM of the MoE layer on CDNA4 (gfx950): kernel
// templates, instantiated per (epilogue, B layout, dtype, B cache policy) by
// gg_inst.hip.
//
// What it computes ("Comm-compute fusion (3)", section 4, the grouped GEMM
// template): output rows come in 128-row blocks; block b belongs to group
// g = block_group[b] and every row r of it is  D[r] = A[a(r)] . B[g], where
// a(r) is r itself or the token row named by the permutation (the
// reorder-by-route prologue of the MoE layer0 row, "Comm-compute fusion (1)",
// section 4).  The SiLU*up epilogue fuses the activation of the serial layer
// (gate/up GEMM -> SiLU -> down GEMM, part (1), section 1) into the gate/up
// GEMM: B holds the gate weights, B2 the up weights, and each workgroup
// accumulates matching gate and up column tiles side by side.  The weighted
// scatter epilogue folds the top-k weighted reduction (the MoE layer1 row,
// part (1), section 4) into the down GEMM: each row adds its routing weight
// times its product into the fp32 row of its token.
//
// How (the pages' SM120 template -- TMA producer warp, mbarrier ring, 8
// consumer warps, 128-row tasks -- is prior art; this is the CDNA4 form):
//   * a task is one or two 128-row blocks of the SAME group (a "row task",
//     up to 256 rows) times one BN-column block: the weight tile is streamed
//     once for up to 256 rows, halving weight traffic per row against
//     128-row tasks.  A plan kernel pairs consecutive blocks of each group
//     (gg_plan_kernel) so the task list is dense;
//   * persistent grid of one workgroup per CU, 8 wavefronts (two per SIMD:
//     one's matrix instructions run while the other issues its fragment
//     reads and DMA) for the full-size store and SiLU*up tiles, 4 (one per
//     SIMD) otherwise; the task list is cut into 8 contiguous ranges, one per
//     XCD (workgroup w runs on XCD w % 8), so the column tasks of one row
//     task share its A rows in that XCD's L2, walking k in the same order;
//   * 32-deep K slices stream through LDS rings with direct global->LDS DMA
//     (global_load_lds_dwordx4), no registers spent on staging: a shallow
//     ring for A tiles (mostly L2 hits) and a deeper one for the weight
//     tiles (HBM, whose latency under load needs ~80 KiB in flight per CU),
//     both running across task boundaries;
//   * the kernel body issues no ordinary global load: the per-task plan
//     entry, the A-row and epilogue index tables and the scatter weights are
//     DMA'd into small LDS rings one or two tasks ahead, so every wait is an
//     explicit s_waitcnt vmcnt(n) on DMA that completes in issue order, and
//     no compiler-inserted vmcnt(0) ever drains the ring;
//   * one s_barrier per slice publishes the slice to the workgroup and
//     frees the oldest stage (the roles of the pages' arrived / finished
//     barriers); fragment reads of the next k step are issued before the
//     matrix instructions of the current one, across slice boundaries too;
//   * LDS rows are XOR-swizzled in 16-byte granules by permuting the source
//     address each lane fetches (the DMA writes lane-contiguously);
//   * A tiles (and B tiles stored [N][K]) are read with ds_read_b128; weight
//     tiles stored [K][N] with the gfx950 transpose read ds_read_b64_tr_b16,
//     which hands each lane 4 consecutive k of one column -- the MFMA B
//     operand layout;
//   * v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulators; with WV
//     wavefronts, wavefront (wm, wn) owns rows [128 wm, 128 wm + 128) and
//     columns [WC wn, WC wn + WC) of each B matrix, WC = BN / (WV / 2).  A
//     one-block task loads its 128 rows twice (one fixed register layout);
//     the second copy's products are not stored, and in the streamed-weight
//     form neither they nor those of all-padding 32-row groups are computed;
//   * the store epilogues convert pairs with one packed instruction and go
//     through LDS (the stages of the slice just consumed) so each store
//     writes whole row pieces; the weighted scatter adds with fp32 atomics.
#pragma once
#include <utility>

#include "common.h"

namespace moe {

// Compile-time loops: f(I_<0>{}), ..., f(I_<N-1>{}), so register arrays are
// indexed with constants.
template <int V> using I_ = std::integral_constant<int, V>;
template <class F, int... Is>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, Is...>) {
  (f(I_<Is>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int kBM = 128;     // rows per block: alignment unit and plan granule
constexpr int kTM = 256;     // rows per task: one or two blocks of one group
// Ring slots of the per-task tables.  The tables of task i are fetched when
// the B stream starts task i-1 and read until task i's epilogue; those of
// task i+4 (same slot) are fetched when the B stream -- NBR-1 slices ahead
// of the consumer -- starts task i+3, which it reaches after task i's
// epilogue as long as 2 KT >= NBR - 1 (KT slices per task; the host only
// picks ring depths that satisfy this).  Plan entries are fetched two tasks
// ahead of the B stream into a ring of 8, and read at the start of each
// task, before the slot can be refetched.
constexpr int kTabSlots = 4;
constexpr int kPlanSlots = 8;

// Epilogues: plain store, SiLU(gate) * up of two B matrices, weighted scatter.
enum { kEpiStore = 0, kEpiSiluMul = 1, kEpiScatter = 2 };

struct GGArgs {
  const uint16_t *A;
  const int32_t *a_src_row; // A row of output row r: a_src_row[r] / a_src_div (NULL: r)
  int a_src_div;
  const uint16_t *B;
  const uint16_t *B2;
  const int32_t *plan;
  uint16_t *D;                 // STORE / SILU_MUL output [cap][N]
  float *Dacc;                 // WEIGHTED_SCATTER output [T][N] (fp32, accumulated into)
  const int32_t *epi_row_pair; // scatter: pair of each row; store: rows with p < 0 are skipped
  const float *pair_w;         // scatter: weight of each pair
  int topk;                    // scatter: token of pair p is p / topk
  int N, K;
  int group_rows; // row tasks per super-block of the task order (>= 1)
  int ldb;        // [K][N] weights: elements per k row (N, or 2N interleaved)
  int b_il;       // gate/up interleaved in 128-column blocks in B (B2 unused)
  // The fused form (LP): the kernel computes the permutation itself from
  // the routing, builds its own row-task plan and A-row tables in LDS, and
  // writes the permutation for the steps after it.
  const int32_t *route_idx = nullptr; // [R] expert of each (token, slot) pair
  int lp_R = 0, lp_E = 0, lp_cap = 0; // pairs, experts, row capacity
  int32_t *o_counts = nullptr, *o_offsets = nullptr, *o_p2r = nullptr, *o_r2p = nullptr,
          *o_bexp = nullptr, *o_mpad = nullptr, *o_plan = nullptr;
  // Split K (store and SiLU*up epilogues, not the fused form): each task's k
  // range in S equal parts, S = splitk_parts_for(row tasks x column blocks,
  // grid, ksplit), each part a task of its own whose fp32 accumulators go,
  // for the rows with a pair p >= 0 in the task's table, to
  // Dpart[(part * part_R + p) * NB * N + m * N + column] (m: the B matrix)
  // instead of the epilogue; a reduction kernel adds the parts in order and
  // applies the epilogue.  With S == 1 (the tasks fill the CUs) the epilogue
  // runs as without the split, into D.
  int ksplit = 1;
  float *Dpart = nullptr;
  int part_R = 0;
};

// Limits of the fused form: experts (one LDS scan over them) and pairs (the
// routing staged in the 48 KiB A ring, which the A stream fills only after
// the tables are built).
constexpr int kLpMaxExperts = 256;
constexpr int kLpMaxPairs = 12288;

// Exclusive prefix sum of v over the NTH threads of the workgroup, in
// thread order; `total` gets the sum.  wt: NTH / 64 ints of LDS.  Two
// barriers, so wt is free again on return.
template <int NTH>
__device__ __forceinline__ int block_excl_scan(int v, int32_t *wt, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wt[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const int t = wt[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// The routing staged in LDS: DMA of 64 ids per wavefront instruction (ids
// past the last pair re-read the last one and are never used), one wait.
template <int NTH>
__device__ __forceinline__ void lp_stage(const int32_t *idx, int R, int32_t *ids) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // the LDS address is scalar
  for (int c = wave * 64; c < R; c += NTH)
    dma4(idx + min(c + lane, R - 1), lds_addr_of(ids + c));
  wait_vmcnt<0>();
  __syncthreads();
}

// The permutation's stable order by its definition: thread t takes pairs
// t NS .. t NS + NS - 1 (NS = ceil(R / NTH) <= 32) as the bits of one mask
// of matches, so a prefix sum over the threads of their match counts gives
// each pair of expert e its rank among the pairs of e (ascending pair
// index).  The thread reads its pairs rotated by its index, so the lanes of
// a read spread over the banks.  f(p, rank) is called for every pair p of e.
template <int NTH, class F>
__device__ __forceinline__ void lp_each_of_expert(const int32_t *ids, int R, int e, int32_t *wt,
                                                  F &&f) {
  const int t = threadIdx.x;
  const int NS = (R + NTH - 1) / NTH;
  uint32_t mask = 0;
  for (int u = 0; u < NS; ++u) {
    const int j = (u + t) % NS, p = t * NS + j;
    if (p < R && ids[p] == e) mask |= 1u << j;
  }
  int tot;
  const int before = block_excl_scan<NTH>(__builtin_popcount(mask), wt, tot);
  for (uint32_t m = mask; m; m &= m - 1) {
    const int j = __builtin_ctz(m);
    f(t * NS + j, before + __builtin_popcount(mask & ((1u << j) - 1u)));
  }
}

// 16-byte-granule XOR swizzles of tiles stored with 64- or 128-byte rows
// (A tiles and [N][K] B tiles: BK = 32 or 64 k of one row).  Both make the
// ds_read_b128 of 16 consecutive rows at one logical granule conflict-free,
// for 64 banks (16 lanes per cycle) and for 32 banks (8 lanes per cycle).
__device__ __forceinline__ int swz64(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int BK> __device__ __forceinline__ int swz_rows(int r) {
  if constexpr (BK == 64)
    return swz128(r);
  else
    return swz64(r);
}

// Swizzle of a [K][N] weight tile with BN columns (rows of 2*BN bytes), read
// with ds_read_b64_tr_b16: one 16-lane group reads 4 consecutive k rows x 32
// bytes, two groups read neighbouring 32-byte column pairs.
template <int BN> __device__ __forceinline__ int swz_kn(int k) {
  if constexpr (BN >= 128)
    return 2 * (k & 3) + 8 * (k & 1);
  else
    return 2 * (k & 3);
}

template <bool FP16>
__device__ __forceinline__ f32x16 mfma32(const i16x4 a0, const i16x4 a1, const i16x4 b0,
                                         const i16x4 b1, f32x16 acc) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const i16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (FP16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Reads one accumulator out of its AGPR where the epilogue needs it.  Plain
// C++ uses make the compiler copy every accumulator into VGPRs at once after
// the k loop (hundreds of registers at the register peak); an asm operand
// constrained to an AGPR keeps them there until each piece is stored.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Task order: super-blocks of `GR` row tasks; inside one, the column block
// varies slowest, so the row tasks of a super-block (mostly one group) read
// each weight tile at about the same time and share it in L2, while with
// GR = 1 the column tasks of one row task run side by side and share its A
// rows.
__device__ __forceinline__ void task_coords(int task, int GR, int ncol, int nrt, int bn, int &rt,
                                            int &n0) {
  const int span = GR * ncol;
  const int sb = task / span;
  const int r = task - sb * span;
  const int rows = min(GR, nrt - sb * GR);
  const int n = r / rows;
  rt = sb * GR + (r - n * rows);
  n0 = n * bn;
}

// Epilogue of one wavefront's share of a tile for STORE and SILU_MUL.  These
// epilogues run the matrix instructions with the operands swapped (weights
// as the first operand), so each 32 x 32 accumulator tile is the transpose:
// register 4 q + e of lane l holds row l % 32, column 8 q + 4 (l / 32) + e.
// Stored straight from registers, each store instruction would write 16
// bytes to each of 32 rows (32 separate pieces), which the memory pipeline
// issues at about a tenth of its byte rate.  So each 32-row tile goes
// through `stg` (this wavefront's 32 x WC staging rows in LDS, 16-byte chunks
// XOR-swizzled by row, their 8-byte halves swapped in every other group of 8
// rows, so neither the writes nor the reads conflict on banks): lanes write their converted 8-byte pieces, then read
// back whole rows, CPR lanes per row, and store 16 contiguous bytes each --
// a store instruction covers 64 / CPR rows of WC columns.  Rows whose entry
// in `skip` (the task's pair table, if any) is negative are padding and are
// not written.
template <int NB, bool FP16, int MI, int NI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NB][MI][NI], uint16_t *Dt, int N,
                                           const MOE_LDS int32_t *skip, int lane, int row0,
                                           int col0, MOE_LDS unsigned char *stg) {
  constexpr int WC = NI * 32;  // columns of this wavefront
  constexpr int RB = WC * 2;   // bytes per staged row
  constexpr int CPR = RB / 16; // 16-byte chunks per row
  constexpr int RPI = 64 / CPR; // rows per store instruction
  // the chunk swizzle takes row bits from SH up: with 64-byte rows two rows
  // share a 128-byte line of banks, and the row's low bit already tells them apart
  constexpr int SH = CPR == 4 ? 1 : 0;
  static_assert(CPR >= 4 && (CPR & (CPR - 1)) == 0 && 64 % CPR == 0, "staging rows");
  const int r = lane & 31;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    // this lane's row r: 8-byte piece (j, q) is granule 8 j + 2 q + l / 32
#pragma unroll
    for (int j = 0; j < NI; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t pk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float o[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float v = acc_read(acc[0][i][j][4 * q + 2 * h + e]);
            if constexpr (NB == 2) {
              // SiLU(v) * u with the hardware reciprocal (about 1 ulp, far
              // below the bf16 rounding that follows) instead of a correctly
              // rounded division, which costs ~10 instructions per value
              const float u = acc_read(acc[1][i][j][4 * q + 2 * h + e]);
              v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
            }
            o[e] = v;
          }
          // one packed round-to-nearest-even conversion per two values
          pk[h] = FP16 ? pack2_f16(o[0], o[1]) : pack2_bf16(o[0], o[1]);
        }
        // chunk XOR row, and the two 8-byte halves swapped in rows with bit
        // 3 set: the 16 lanes of a quarter-wavefront hit distinct banks
        const int chunk = (4 * j + q) ^ ((r >> SH) & (CPR - 1));
        const int half = (lane >> 5) ^ ((r >> 3) & 1);
        *(MOE_LDS u32x2 *)(stg + r * RB + chunk * 16 + half * 8) = u32x2{pk[0], pk[1]};
      }
      // one 32 x 32 tile at a time: unrolled freely, the scheduler would
      // convert every tile at once and hold ~100 registers of temporaries
      __builtin_amdgcn_sched_barrier(0);
    }
    // whole rows back out: lane l stores chunk l % CPR of row l / CPR (+ RPI per step)
#pragma unroll
    for (int rr = 0; rr < 32 / RPI; ++rr) {
      const int row = rr * RPI + lane / CPR;
      const int ch = lane % CPR;
      u32x4 v = *(const MOE_LDS u32x4 *)(stg + row * RB + ((ch ^ ((row >> SH) & (CPR - 1))) * 16));
      if ((row >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]}; // halves back in column order
      const int trow = row0 + i * 32 + row; // row inside the task
      if (!skip || skip[trow] >= 0)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<unsigned char *>(Dt) +
                                   (uint32_t)((trow * N + col0 + ch * 8) * 2)) = v;
    }
  }
}

// Split-K epilogue of one wavefront's share of a tile (the transposed
// accumulator layout of the store epilogues: register 4 q + e of lane l
// holds row l % 32, column 8 q + 4 (l / 32) + e of each 32 x 32 tile): the
// raw fp32 sums of the rows whose pair is p >= 0, 16 bytes per lane and
// store, at Dp[(p * NB + m) * N + col] (Dp: this k part's block).
template <int NB, int MI, int NI>
__device__ __forceinline__ void partial_tile(const f32x16 (&acc)[NB][MI][NI], float *Dp, int N,
                                             const MOE_LDS int32_t *ptab, int lane, int row0,
                                             int col) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int p = ptab[row0 + i * 32 + (lane & 31)];
    if (p >= 0) {
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 v;
            v.x = acc_read(acc[m][i][j][4 * q + 0]);
            v.y = acc_read(acc[m][i][j][4 * q + 1]);
            v.z = acc_read(acc[m][i][j][4 * q + 2]);
            v.w = acc_read(acc[m][i][j][4 * q + 3]);
            *reinterpret_cast<float4 *>(Dp + ((size_t)p * NB + m) * N + col + j * 32 + 8 * q +
                                        4 * (lane >> 5)) = v;
          }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Weighted-scatter epilogue of one wavefront's share of a tile: task row r
// adds w_r * acc into the fp32 token row p_r / k of Dacc, with the pair p_r
// and its weight w_r taken from the task's LDS tables (padding rows, p < 0,
// add nothing).  fp32 device-scope atomics: the k contributions of a token
// meet in no fixed order.
template <int MI, int NI>
__device__ __forceinline__ void scatter_tile(const f32x16 (&acc)[1][MI][NI], float *Dacc, int N,
                                             const MOE_LDS int32_t *ptab,
                                             const MOE_LDS float *wtab, int k, int lane, int row0,
                                             int col) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int p = ptab[tr];
      if (p >= 0) {
        const float w = wtab[tr];
        float *o = Dacc + (size_t)(p / k) * N + col + (lane & 31);
#pragma unroll
        for (int j = 0; j < NI; ++j) unsafeAtomicAdd(o + j * 32, w * acc_read(acc[0][i][j][r]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// BN: output columns per task (per B matrix); BK: k per slice (32 or 64:
// A rows of 64 or 128 bytes per slice); EPI: kEpiStore, kEpiSiluMul (two B
// matrices) or kEpiScatter; KN: B stored [K][N] (else [N][K]); NA, NBR:
// depths of the A ring and of the B ring.
//
// Two rings: the B (weight) ring is deeper than the A ring.  Weights stream
// from HBM, whose latency under full load is several microseconds, so each
// CU needs most of its in-flight bytes to be weights; A tiles mostly hit in
// L2 and need a shorter lead.  At consumer slice c the wavefront issues A
// slice c + NA - 1 and then B slice c + NBR - 1 (each into the slot its
// ring freed at the previous barrier), so the B stream runs NBR - NA
// slices further ahead and may already be on a later task than the A
// stream; each stream keeps its own task cursor.
// WV: wavefronts per workgroup, 4 (one per SIMD, 256 accumulators each) or 8
// (two per SIMD, 128 accumulators each: while one issues its fragment reads
// and DMA, the other feeds the matrix pipe).  Each covers 128 rows and
// BN / (WV / 2) columns of the task.
// LP: the fused form -- the permutation is computed by the kernel from the
// routing instead of read from a plan and row map built before it (see
// GGArgs); SiLU*up on [K][N] weights with gathered A rows only.
// SK: the split-K form (see GGArgs::ksplit; store and SiLU*up only).
template <int BN, int BK, int EPI, bool KN, bool FP16, int NA, int NBR, bool BNT, int WV,
          bool LP = false, bool SK = false>
__global__ __launch_bounds__(64 * WV, 1) void grouped_gemm_kernel(GGArgs args) {
  constexpr int NB = EPI == kEpiSiluMul ? 2 : 1; // B matrices
  constexpr int ARP = BK * 2;                    // bytes per A row (and [N][K] B row) per slice
  constexpr int A_BYTES = kTM * ARP;             // one A stage
  constexpr int B_BYTES = BK * BN * 2;           // one B matrix of one B stage
  constexpr int BS_BYTES = NB * B_BYTES;         // one B stage
  constexpr int A_INSTR = A_BYTES / 1024 / WV;    // DMA instructions per wavefront per A slice
  constexpr int B_INSTR = B_BYTES / 1024 / WV;    // per B matrix per B slice
  constexpr int A_LOADS = A_INSTR;
  constexpr int B_LOADS = NB * B_INSTR;
  constexpr int LA = NA - 1;                          // A issue lead (slices)
  constexpr int LB = NBR - 1;                         // B issue lead (slices)
  // DMA instructions issued after the later of A slice 1 and B slice 1 by
  // the end of the prologue: A slice s is issued with B slice s + LB - LA,
  // so with LB > LA, A slice 1 is the later one and the B slice issued with
  // it plus LA - 2 whole pairs follow it; with LB == LA, B slice 1 is the
  // later one and LA - 2 pairs follow.  (The same count, with LA - 1 pairs,
  // holds for slice 0, the first wait.)
  constexpr int NQ = A_LOADS + B_LOADS; // DMA instructions per slice
  constexpr int AFTER0 = (LB > LA ? B_LOADS : 0) + (LA - 1) * NQ;
  static_assert(LA >= 2, "the A stream leads by at least two slices");
  constexpr int A_RPI = 1024 / ARP;                   // A rows per DMA instruction
  constexpr int A_GPR = ARP / 16;                     // 16-byte granules per A row
  constexpr int WCOL = WV / 2;                        // wavefronts across the columns
  constexpr int WC = BN / WCOL;                       // columns per wavefront per matrix
  constexpr int TR = kTM / WV;                        // table rows fetched per wavefront
  constexpr int NI = WC / 32;
  constexpr bool SCAT = EPI == kEpiScatter;
  static_assert(BK == 32, "two 16-deep k steps per slice");
  static_assert(WV == 4 || WV == 8, "wavefronts per workgroup");
  static_assert(NI >= 1 && B_INSTR >= 1 && A_INSTR * A_RPI * WV == kTM, "DMA split");
  static_assert(NA >= 2 && NBR >= NA, "ring depths");

  __shared__ __attribute__((aligned(1024))) unsigned char aring[NA * A_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char bring[NBR * BS_BYTES];
  // tab: the task's pair per row -- the A source pairs if A rows are
  // gathered, else the epilogue pairs; etab: scatter only, the epilogue pairs
  // when they differ from the A source pairs; wtab: scatter only, the weights
  __shared__ __attribute__((aligned(16))) int32_t tab[kTabSlots][kTM];
  __shared__ __attribute__((aligned(16))) int32_t etab[SCAT ? kTabSlots : 1][SCAT ? kTM : 1];
  __shared__ __attribute__((aligned(16))) float wtab[SCAT ? kTabSlots : 1][SCAT ? kTM : 1];
  __shared__ __attribute__((aligned(16))) int32_t ptab[WV][kPlanSlots][2]; // plan entries

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WCOL;
  const int wn = wave % WCOL;
  const int N = args.N, K = args.K;
  static_assert(!SK || (!LP && EPI != kEpiScatter), "split K: store and SiLU*up only");
  static_assert(!LP || (EPI == kEpiSiluMul && KN), "the fused form is the gate/up GEMM's");
  const bool has_a = LP || args.a_src_row != nullptr;
  // the pair table `tab` holds a_src_row if given, else epi_row_pair; the
  // scatter's own epilogue table is needed only when both differ
  const int32_t *tab_src = has_a ? args.a_src_row : args.epi_row_pair;
  const bool has_tab = LP || tab_src != nullptr;
  const bool own_e = SCAT && has_a && args.epi_row_pair != args.a_src_row;

  // ---------------- fused form: the permutation from the routing ----------------
  // The routing is staged in the A ring and counted in LDS; the expert
  // offsets and row-task offsets follow by two scans.  That fixes the task
  // list, so the weight stream can start; the A-row tables of this
  // workgroup's tasks are built while its first slices are in flight, and
  // the permutation the later steps read is written after the main loop.
  // (Compact loops throughout: this code runs once per workgroup, so its
  // instruction fetch, not its arithmetic, is what it costs.)
  constexpr int NTH = 64 * WV;
  __shared__ int32_t lp_s[LP ? 3 * (kLpMaxExperts + 1) + 16 : 1];
  int32_t *const lp_cnt = lp_s;
  int32_t *const lp_off = lp_s + (kLpMaxExperts + 1);
  int32_t *const lp_toff = lp_s + 2 * (kLpMaxExperts + 1);
  int32_t *const lp_wt = lp_s + 3 * (kLpMaxExperts + 1);
  int32_t *const lp_ids = reinterpret_cast<int32_t *>(aring);
  int nrt, m_pad = 0;
  if constexpr (LP) {
    static_assert(!LP || NA * A_BYTES >= 4 * kLpMaxPairs, "the routing fits the A ring");
    static_assert(!LP || kLpMaxPairs <= 32 * NTH, "a thread's pairs fit one mask");
    const int R = args.lp_R, E = args.lp_E;
    for (int e = tid; e < E; e += NTH) lp_cnt[e] = 0;
    lp_stage<NTH>(args.route_idx, R, lp_ids);
#pragma unroll 4
    for (int p = tid; p < R; p += NTH) {
      const int e = lp_ids[p];
      if (e >= 0 && e < E) atomicAdd(&lp_cnt[e], 1);
    }
    __syncthreads();
    // padded offsets and each expert's first row task (one thread per expert)
    const int c = tid < E ? lp_cnt[tid] : 0;
    const int padded = (c + kBM - 1) / kBM * kBM;
    const int tasks = (padded / kBM + 1) / 2;
    int mp, ntasks;
    const int o = block_excl_scan<NTH>(padded, lp_wt, mp);
    const int to = block_excl_scan<NTH>(tasks, lp_wt, ntasks);
    if (tid < E) {
      lp_off[tid] = o;
      lp_toff[tid] = to;
    }
    if (tid == 0) {
      lp_off[E] = mp;
      lp_toff[E] = ntasks;
    }
    __syncthreads();
    // the same in every lane (a value read from LDS is not known to be):
    // the task addresses derived from it are wave-uniform scalars
    nrt = __builtin_amdgcn_readfirstlane(ntasks);
    m_pad = __builtin_amdgcn_readfirstlane(mp);
  } else {
    nrt = args.plan[0]; // read before any DMA is in flight
  }

  // The permutation the later steps read, written by the fused form at its
  // end: the experts of this workgroup (their pairs' rows, padding rows,
  // block experts, plan entries); workgroup 0 the counts, offsets, M_pad,
  // the plan's head and the pairs routed outside [0, E); all of them,
  // shared out, the rows and blocks past M_pad.  The routing is staged in
  // the A ring again (every wavefront's DMA has landed and the rings are
  // read).
  auto lp_outputs = [&]() {
    if constexpr (LP) {
      const int R = args.lp_R, E = args.lp_E;
      __syncthreads();
      lp_stage<NTH>(args.route_idx, R, lp_ids);
      // (the lambdas capture plain pointers: a reference to the kernel's
      // argument block would move it to private memory, and every field read
      // from there would no longer be known to be wave-uniform)
      int32_t *const o_p2r = args.o_p2r, *const o_r2p = args.o_r2p;
      for (int e = blockIdx.x; e < E; e += gridDim.x) {
        const int r0 = lp_off[e], r1 = lp_off[e + 1];
        lp_each_of_expert<NTH>(lp_ids, R, e, lp_wt, [=](int p, int rank) {
          o_p2r[p] = r0 + rank;
          o_r2p[r0 + rank] = p;
        });
        for (int r = r0 + lp_cnt[e] + tid; r < r1; r += NTH) o_r2p[r] = -1;
        const int b0 = r0 / kBM, nbk = (r1 - r0) / kBM;
        for (int b = tid; b < nbk; b += NTH) args.o_bexp[b0 + b] = e;
        for (int q = tid; 2 * q < nbk; q += NTH) {
          const int i = lp_toff[e] + q;
          args.o_plan[kPlanHead + 2 * i] = (b0 + 2 * q) | (2 * q + 1 < nbk ? kPlanTwo : 0);
          args.o_plan[kPlanHead + 2 * i + 1] = e;
        }
      }
      if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += NTH) {
          args.o_counts[e] = lp_cnt[e];
          args.o_offsets[e] = lp_off[e];
        }
        if (tid == 0) {
          args.o_offsets[E] = m_pad;
          args.o_mpad[0] = m_pad;
          args.o_plan[0] = nrt;
          args.o_plan[1] = m_pad / kBM;
        }
      }
      // (loops with the same trip count in every lane)
      const int step = gridDim.x * NTH, cap = args.lp_cap;
      for (int r0 = m_pad + (int)blockIdx.x * NTH; r0 < cap; r0 += step)
        if (r0 + tid < cap) o_r2p[r0 + tid] = -1;
      for (int b0 = m_pad / kBM + (int)blockIdx.x * NTH; b0 < cap / kBM; b0 += step)
        if (b0 + tid < cap / kBM) args.o_bexp[b0 + tid] = -1;
      for (int p0 = (int)blockIdx.x * NTH; p0 < R; p0 += step)
        if (p0 + tid < R && (lp_ids[p0 + tid] < 0 || lp_ids[p0 + tid] >= E)) o_p2r[p0 + tid] = -1;
    }
  };

  // ---------------- schedule ----------------
  const int ncol = N / BN;
  // k parts per task (split K: from the task count, at most args.ksplit)
  // and slices per item
  const int KS = SK ? splitk_parts_for(nrt * ncol, gridDim.x, args.ksplit) : 1;
  const int KT = K / BK / KS;
  const int ntask = nrt * ncol * KS; // (row task, column block, k part)
  const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
  const int xcd = blockIdx.x % nx;
  const int S = gridDim.x / nx;
  const int slot = blockIdx.x / nx;
  const int tx0 = (int)(((long)ntask * xcd) / nx);
  const int tx1 = (int)(((long)ntask * (xcd + 1)) / nx);
  // the fused form builds the tables of at most kTabSlots items (the host
  // bounds the task count so; more would not be computed)
  const int n_items = min(tx1 - tx0 > slot ? (tx1 - tx0 - slot + S - 1) / S : 0,
                          LP ? kTabSlots : 1 << 30);
  if (n_items == 0) {
    lp_outputs();
    return;
  }
  const int total = n_items * KT; // slices of this workgroup
  auto coords = [&](int i, int &rt, int &n0) {
    const int t = tx0 + slot + i * S;
    task_coords(SK ? t / KS : t, args.group_rows, ncol, nrt, BN, rt, n0);
    // wave-uniform: the weight stream addresses are scalar operands
    rt = __builtin_amdgcn_readfirstlane(rt);
    n0 = __builtin_amdgcn_readfirstlane(n0);
  };
  // the k part of item i (the parts of one task are neighbouring items)
  auto kpart = [&](int i) -> int {
    if constexpr (!SK) return 0;
    return __builtin_amdgcn_readfirstlane((tx0 + slot + i * S) % KS);
  };
  if constexpr (LP) {
    // the plan entries of this workgroup's items, from the offsets: row task
    // rt is task rt - toff[e] of the expert e with toff[e] <= rt < toff[e+1]
    // (each wavefront writes its own copy, as the DMA'd entries would be)
    for (int i = 0; i < n_items; ++i) {
      int rt, n0;
      coords(i, rt, n0);
      const int E = args.lp_E;
      int lo = 0, hi = E - 1; // the last expert with toff <= rt (empty experts own no task)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (lp_toff[mid] <= rt)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int q = rt - lp_toff[lo];
      const int nbk = (lp_off[lo + 1] - lp_off[lo]) / kBM;
      if (lane == 0) {
        ptab[wave][i][0] = (lp_off[lo] / kBM + 2 * q) | (2 * q + 1 < nbk ? kPlanTwo : 0);
        ptab[wave][i][1] = lo;
      }
    }
  }
  // ---------------- per-task tables (DMA'd into small LDS rings) ----------------
  // DMA the plan entry of item i into this wavefront's slot (lanes 0, 1).
  auto fetch_plan = [&](int i) {
    if constexpr (LP) return; // built in LDS above
    int rt, n0;
    coords(i, rt, n0);
    if (lane < 2)
      dma4(args.plan + kPlanHead + 2 * rt + lane, lds_addr_of(&ptab[wave][i % kPlanSlots][0]));
  };
  auto plan_of = [&](int i, int &b, int &nb, int &g) {
    const int e = __builtin_amdgcn_readfirstlane(ptab[wave][i % kPlanSlots][0]);
    g = __builtin_amdgcn_readfirstlane(ptab[wave][i % kPlanSlots][1]);
    b = e & (kPlanTwo - 1);
    nb = (e & kPlanTwo) ? 2 : 1;
  };
  // DMA this wavefront's TR rows of the pair tables of item i (its plan
  // entry has landed).  Rows of the missing second block of a one-block
  // task repeat the first block's rows.
  auto fetch_tables = [&](int i) {
    if (LP || !has_tab) return; // LP: built in LDS above
    int b, nb, g;
    plan_of(i, b, nb, g);
    const int r = TR * wave + (lane % TR);
    const size_t src = (size_t)b * kBM + (nb == 2 ? r : (r & (kBM - 1)));
    const int s = i % kTabSlots;
    if (lane < TR) dma4(tab_src + src, lds_addr_of(&tab[s][TR * wave]));
    if constexpr (SCAT)
      if (own_e && lane < TR) dma4(args.epi_row_pair + src, lds_addr_of(&etab[s][TR * wave]));
  };
  // the epilogue's pair per row
  auto pair_table = [&](int s) -> const MOE_LDS int32_t * {
    if constexpr (SCAT)
      if (own_e) return (const MOE_LDS int32_t *)etab[s];
    return (const MOE_LDS int32_t *)tab[s];
  };
  // DMA the routing weights of this wavefront's TR rows of item i (its pair
  // table has landed).
  auto fetch_weights = [&](int i) {
    if constexpr (SCAT) {
      const int s = i % kTabSlots;
      const int p = pair_table(s)[TR * wave + (lane % TR)];
      if (lane < TR) dma4(args.pair_w + (p < 0 ? 0 : p), lds_addr_of(&wtab[s][TR * wave]));
    }
  };
  // The column tasks of one row task run side by side on neighbouring CUs
  // of one XCD and walk k in the same order, so each A slice is fetched into
  // that XCD's L2 once and served to all of them while it is still there.

  // ---------------- A stream ----------------
  int a_i = 0, a_k = KT; // item being issued, slices of it issued
  const unsigned char *a_src[A_INSTR];
  // Point the A sources at item i (its plan entry and tables have landed).
  // A one-block task loads its 128 rows twice (rows 128-255 repeat them,
  // served by the caches) so every slice has the same DMA count.
  auto a_begin = [&](int i) {
    // item i's tables were fetched when the B stream began item i-1, which
    // the consumer's waits have covered unless the A lead is long against
    // the task length; then wait for everything
    if (i > 0 && KT + LB <= 2 * LA) wait_vmcnt<0>();
    int b, nb, g;
    plan_of(i, b, nb, g);
    const MOE_LDS int32_t *ptbl = (const MOE_LDS int32_t *)tab[i % kTabSlots];
    const size_t kb = (size_t)kpart(i) * KT * BK; // the item's first k (split K)
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      // instruction q covers task rows (wave*A_INSTR+q)*A_RPI .. +A_RPI
      const int row = (wave * A_INSTR + q) * A_RPI + lane / A_GPR;
      long src = (long)b * kBM + (nb == 2 ? row : (row & (kBM - 1)));
      if (has_a) {
        const int p = ptbl[row];
        src = p < 0 ? 0 : p / args.a_src_div; // padding rows read a valid row
      }
      const int c = (lane % A_GPR) ^ swz_rows<BK>(row);
      a_src[q] = reinterpret_cast<const unsigned char *>(args.A) + ((size_t)src * K + kb + c * 8) * 2;
    }
    fetch_weights(i);
    a_i = i;
    a_k = 0;
  };
  // The DMA of one A slice: a_prep does the bookkeeping (task switch, k
  // offset, stage), a_emit(q) issues instruction q, so the consumer can
  // spread the instructions among its matrix instructions.  Past the end of
  // the stream the slices still go out, re-reading the last slice into the
  // stage they would use: that stage was released and is never read again
  // (the consumer ends first), and every slice keeps the same instruction
  // count, so the waits are exact and the issue sequence has no branches.
  int a_issued = 0; // A slices issued
  uint32_t a_koff = 0, a_stage = 0;
  auto a_prep = [&]() {
    if (a_issued < total) {
      if (a_k == KT) a_begin(a_i + 1);
      a_koff = (uint32_t)(a_k * BK * 2);
      ++a_k;
    }
    a_stage = lds_addr_of(aring) + (a_issued % NA) * A_BYTES + wave * A_INSTR * 1024;
    ++a_issued;
  };
  auto a_emit = [&](int q) { dma16(a_src[q] + a_koff, a_stage + q * 1024); };
  auto a_issue = [&]() {
    a_prep();
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) a_emit(q);
  };

  // ---------------- B stream ----------------
  constexpr int RPI = KN ? 512 / BN : A_RPI; // k rows ([K][N]) or n rows ([N][K]) per instruction
  // the swizzle depends on k mod 4 ([K][N]) or n mod 16 ([N][K]): distinct
  // per-lane offset patterns among the instructions
  constexpr int QV = KN ? (RPI < 4 ? 4 / RPI : 1) : (RPI < 16 ? 16 / RPI : 1);
  uint32_t b_off[QV];
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    if constexpr (KN) {
      constexpr int GPR = BN / 8; // 16-byte granules per k row
      const int k = v * RPI + lane / GPR;
      b_off[v] = (uint32_t)(((lane / GPR) * args.ldb + (((lane % GPR) ^ swz_kn<BN>(k)) * 8)) * 2);
    } else {
      const int n = v * RPI + lane / A_GPR;
      b_off[v] =
          (uint32_t)(((lane / A_GPR) * K + (((lane % A_GPR) ^ swz_rows<BK>(n)) * 8)) * 2);
    }
  }
  int b_i = 0, b_k = KT;
  const unsigned char *b_base[NB];
  // Start the B stream on item i: fetch the plan entry of item i+2 and the
  // tables of item i+1, then point the B bases at item i (its plan entry
  // has landed).
  auto b_begin = [&](int i) {
    // the plan entry of item i+1 (read by fetch_tables) was fetched when
    // item i-1 began, which the consumer's waits have covered once a task
    // has more than NA - 1 slices; below that, wait for everything
    if (i > 0 && KT < NA) wait_vmcnt<0>();
    if (i + 2 < n_items) fetch_plan(i + 2);
    if (i + 1 < n_items) fetch_tables(i + 1);
    int rt, n0, b, nb, g;
    coords(i, rt, n0);
    plan_of(i, b, nb, g);
    const int gg = g < 0 ? 0 : g;
    const size_t kb = (size_t)kpart(i) * KT * BK; // the item's first k (split K)
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      // interleaved gate/up: block b of 128 columns holds gate then up
      const unsigned char *Bm =
          reinterpret_cast<const unsigned char *>(m == 0 || args.b_il ? args.B : args.B2) +
          (size_t)gg * K * (KN ? args.ldb : N) * 2;
      const int col = args.b_il ? ((n0 >> 7) << 8) + (n0 & 127) + m * 128 : n0;
      // this wavefront's first k row (or n row) of every slice
      b_base[m] = KN ? Bm + ((size_t)(kb + wave * B_INSTR * RPI) * args.ldb + col) * 2
                     : Bm + ((size_t)(n0 + wave * B_INSTR * RPI) * K + kb) * 2;
    }
    b_i = i;
    b_k = 0;
  };
  // the B slice's DMA in the same two parts (instruction e: matrix e /
  // B_INSTR, piece e % B_INSTR), past the end of the stream likewise
  int b_issued = 0;
  size_t b_koff = 0;
  uint32_t b_stage = 0;
  auto b_prep = [&]() {
    if (b_issued < total) {
      if (b_k == KT) b_begin(b_i + 1);
      b_koff = KN ? (size_t)b_k * BK * args.ldb * 2 : (size_t)b_k * BK * 2;
      ++b_k;
    }
    b_stage = lds_addr_of(bring) + (b_issued % NBR) * BS_BYTES + wave * B_INSTR * 1024;
    ++b_issued;
  };
  auto b_emit = [&](int e) {
    const int m = e / B_INSTR, q = e % B_INSTR;
    const size_t qoff = KN ? (size_t)q * RPI * args.ldb * 2 : (size_t)q * RPI * K * 2;
    dma16s<BNT>(b_off[q % QV], b_base[m] + b_koff + qoff, b_stage + m * B_BYTES + q * 1024);
  };
  auto b_issue = [&]() {
    b_prep();
#pragma unroll
    for (int e = 0; e < B_LOADS; ++e) b_emit(e);
  };

  // prologue: the plan entries of items 0-3 and the tables of items 0-2 --
  // all the prologue's streams can reach (the B stream at most item 1, as
  // 2 KT >= NBR - 1) and what their task starts fetch for later ones.  The B
  // stream needs only plan entries, so it starts while the tables are in
  // flight: its first LB - LA slices go out, then the A stream (whose row
  // addresses come from the tables) joins, A slice s right before B slice
  // s + LB - LA, the order of the main loop.  The tables were issued before
  // at least (LB - LA) B_LOADS DMA instructions (task starts may add more,
  // which only makes the wait stricter).
  // The A-row tables of the fused form's items: table row r of item i is
  // the pair of rank j0 + r among the pairs of its expert g (a one-block task
  // repeats its 128 rows); ranks past the expert's count are padding (-1).
  auto lp_tables = [&]() {
    if constexpr (LP) {
      for (int i = 0; i < n_items; ++i) {
        int b, nb, g;
        plan_of(i, b, nb, g);
        const int j0 = b * kBM - lp_off[g];
        for (int r = tid; r < kTM; r += NTH) tab[i][r] = -1;
        __syncthreads();
        int32_t *const trow = tab[i];
        lp_each_of_expert<NTH>(lp_ids, args.lp_R, g, lp_wt, [=](int p, int rank) {
          const int r = rank - j0;
          if (r >= 0 && r < nb * kBM) {
            trow[r] = p;
            if (nb == 1) trow[r + kBM] = p;
          }
        });
        __syncthreads();
      }
    }
  };

  for (int j = 0; j < 4 && j < n_items; ++j) fetch_plan(j);
  wait_vmcnt<0>();
  for (int j = 0; j < 3 && j < n_items; ++j) fetch_tables(j);
  b_begin(0);
  for (int s = 0; s < LB - LA; ++s) b_issue();
  lp_tables(); // the fused form: while the first weight slices are in flight
  wait_vmcnt<(LB - LA) * B_LOADS>();
  a_begin(0);
  for (int s = 0; s < LA; ++s) {
    a_issue();
    b_issue();
  }

  // ---------------- compute (consumer) ----------------
  // The accumulators are carried across items and cleared right after each
  // epilogue has read them, so one register set serves every item.
  f32x16 acc[NB][4][NI];
  auto clear_acc = [&]() {
    // an opaque zero: a constant zero vector would be hoisted out of the
    // item loop and kept in 16 * NB * 4 * NI spare registers
    float z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][a][j][r] = z;
  };

  // Fragments of one 16-deep k step, double-buffered in registers.
  i16x4 fa[2][4][2];
  i16x4 fb[2][NB][NI][2];
  // LDS read d of the fragments of k step kk of slice c into buffer BUF:
  // d < 4 the A rows of 32-row group d; then the B columns, two transpose
  // reads per 32-column group and matrix ([K][N]) or one 16-byte read
  // ([N][K]).
  constexpr int ND = 4 + NB * NI * (KN ? 2 : 1); // LDS reads per k step
  auto frag = [&](auto D, auto BUF, int c, int kk) {
    constexpr int d = decltype(D)::value;
    constexpr int buf = decltype(BUF)::value;
    if constexpr (d < 4) {
      const MOE_LDS unsigned char *sA =
          (const MOE_LDS unsigned char *)(aring + (c % NA) * A_BYTES);
      const int row = wm * 128 + d * 32 + (lane & 31);
      const int c16 = (kk * 2 + (lane >> 5)) ^ swz_rows<BK>(row);
      const u32x4 v = *(const MOE_LDS u32x4 *)(sA + row * ARP + c16 * 16);
      fa[buf][d][0] = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
      fa[buf][d][1] = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
    } else if constexpr (KN) {
      constexpr int e = d - 4, m = e / (2 * NI), j = (e / 2) % NI, h = e % 2;
      const MOE_LDS unsigned char *sB =
          (const MOE_LDS unsigned char *)(bring + (c % NBR) * BS_BYTES + m * B_BYTES);
      // lane group G = lane/16 reads columns n0 + 16*(G&1) .. +16 at
      // k = 8*(G>>1) + 4*h + (lane%16)/4; each lane points at 4
      // consecutive columns, the transpose read returns 4 k of one column
      const int G = lane >> 4;
      const int q = lane & 15;
      const int n = wn * WC + j * 32 + 16 * (G & 1) + 4 * (q & 3);
      const int k = kk * 16 + 8 * (G >> 1) + (q >> 2) + 4 * h;
      const int o = k * (BN * 2) + (((n >> 3) ^ swz_kn<BN>(k)) << 4) + ((n & 7) << 1);
      fb[buf][m][j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4 *)(sB + o));
    } else {
      constexpr int e = d - 4, m = e / NI, j = e % NI;
      const MOE_LDS unsigned char *sB =
          (const MOE_LDS unsigned char *)(bring + (c % NBR) * BS_BYTES + m * B_BYTES);
      const int n = wn * WC + j * 32 + (lane & 31);
      const int c16 = (kk * 2 + (lane >> 5)) ^ swz_rows<BK>(n);
      const u32x4 v = *(const MOE_LDS u32x4 *)(sB + n * ARP + c16 * 16);
      fb[buf][m][j][0] = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
      fb[buf][m][j][1] = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
    }
  };
  // matrix instruction t of a k step on buffer BUF (row group fastest)
  constexpr int NM = NB * NI * 4;
  // Bit mi: this wavefront's 32-row group mi of the current item has a row
  // whose product is used (wave-uniform, set at each item's start).  Only
  // the streamed-weight form (BNT) skips the others: there each weight tile
  // is read about once, the kernel waits on HBM and the skipped matrix work
  // is pure saving (tp_share layer -4.6 %, ep_skew -5 %), while in the
  // MFMA-bound shapes the predicate on every matrix instruction costs more
  // than the little padding saves (dense +5 %, prefill +9 %).
  uint32_t live = 0xF;
  auto mma = [&](auto T, auto BUF) {
    constexpr int t = decltype(T)::value;
    constexpr int buf = decltype(BUF)::value;
    constexpr int m = t / (4 * NI), j = (t / 4) % NI, mi = t % 4;
    if constexpr (BNT)
      if (!(live & (1u << mi))) return;
    // the weighted scatter keeps the row-major accumulator layout (its fp32
    // atomics then cover 32 contiguous columns per row); the stores take the
    // transposed one (weights as the first operand)
    if constexpr (SCAT)
      acc[m][mi][j] = mfma32<FP16>(fa[buf][mi][0], fa[buf][mi][1], fb[buf][m][j][0],
                                   fb[buf][m][j][1], acc[m][mi][j]);
    else
      acc[m][mi][j] = mfma32<FP16>(fb[buf][m][j][0], fb[buf][m][j][1], fa[buf][mi][0],
                                   fa[buf][mi][1], acc[m][mi][j]);
  };
  // DMA instruction q of this slice's share (A first, then B)
  auto dma = [&](auto Q) {
    constexpr int q = decltype(Q)::value;
    if constexpr (q < A_LOADS)
      a_emit(q);
    else
      b_emit(q - A_LOADS);
  };
  // Interleave: after matrix instruction t of a k step come the fragment
  // reads FPS*t .. FPS*t+FPS-1 (of the next k step; in the last k step,
  // from matrix instruction BAR on, of the next slice, after the barrier);
  // the slice's DMA instructions are spread evenly over both k steps, DMA
  // q after matrix instruction dslot(q) of the slice's 2 NM.  A wavefront
  // whose DMA queue is full stalls at its next DMA instruction, so the
  // issue is kept steady: a burst would stall the matrix pipe and then
  // leave the memory pipeline idle for the rest of the slice.  A
  // scheduling fence after every group keeps the order.
  constexpr int FPS = 2;
  constexpr int FSLOTS = (ND + FPS - 1) / FPS;
  constexpr int BAR = NM >= 8 ? NM / 4 : 0;
  static_assert(BAR + FSLOTS <= NM, "fragment reads fit the last k step");
  constexpr auto dslot = [](int q) { return (2 * NM * q) / NQ + NM / NQ; };
  // DMA instructions of a slice issued before the wait of its last k step
  constexpr int D_PRE = [&] {
    int n = 0;
    for (int q = 0; q < NQ; ++q) n += dslot(q) < NM + BAR;
    return n;
  }();
  // The wait of slice c's last k step is for slice c+1: A slice c+1 came
  // with the DMA of slice c+1-LA, B slice c+1 earlier (LB > LA) or with it;
  // after the later of them come the rest of that slice's DMA (B_LOADS if
  // A was the later one), LA - 2 whole slices and the D_PRE instructions
  // of slice c issued so far.
  constexpr int AFTER = (LB > LA ? B_LOADS : 0) + (LA - 2) * NQ + D_PRE;
  static_assert(AFTER >= 0 && AFTER < 64 && AFTER0 < 64, "vmcnt range");
  auto dma_at = [&](auto S) {
    constexpr int slot = decltype(S)::value;
    static_for<NQ>([&](auto Q) {
      if constexpr (dslot(decltype(Q)::value) == slot) dma(Q);
    });
  };

  // Slice 0 (A and B) has landed for this wavefront once at most AFTER0
  // DMA instructions are still in flight (DMA completes in issue order;
  // every slice, past the end of the stream too, has the same count).
  wait_vmcnt<AFTER0>();
  block_barrier();
  static_for<ND>([&](auto D) { frag(D, I_<0>{}, 0, 0); });
  clear_acc();

  int c = 0; // slice being consumed (global count)
  for (int i = 0; i < n_items; ++i) {
    // this item's coordinates, read before later fetches may reuse its slot
    int rt, n0, b, nb, g;
    coords(i, rt, n0);
    plan_of(i, b, nb, g);
    // Matrix instructions whose products nobody reads (BNT only): all of
    // them for an item of no group, those of the second half of a one-block
    // task (a copy of the first), and a 32-row group whose rows are all
    // padding (pair < 0 in the item's table; the epilogues do not store or
    // add such rows).  Their accumulators stay zero.
    if (!BNT) {
      live = 0xF;
    } else if (g < 0 || (nb == 1 && wm == 1)) {
      live = 0;
    } else if (has_tab) {
      const MOE_LDS int32_t *trow = (const MOE_LDS int32_t *)tab[i % kTabSlots] + wm * 128;
      uint32_t lv = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        lv |= (__builtin_amdgcn_ballot_w64(lane < 32 && trow[mi * 32 + lane] >= 0) != 0) << mi;
      live = __builtin_amdgcn_readfirstlane(lv);
    } else {
      live = 0xF;
    }
    for (int kt = 0; kt < KT; ++kt, ++c) {
      // k step 0 on buffer 0: its fragments (read during the previous
      // matrix instructions) are in -- said explicitly, so no LDS wait lands
      // among the matrix instructions; among them, the fragment reads of k
      // step 1 and this wavefront's share of the next slices' DMA, into the
      // stages every wavefront released at the last barrier
      wait_lgkm0();
      static_for<NM>([&](auto T) {
        constexpr int t = decltype(T)::value;
        mma(T, I_<0>{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<FPS>([&](auto F) {
          constexpr int d = FPS * t + decltype(F)::value;
          if constexpr (d < ND) frag(I_<d>{}, I_<1>{}, c, 1);
        });
        if constexpr (t == 0) {
          a_prep();
          b_prep();
        }
        dma_at(T);
        __builtin_amdgcn_sched_barrier(0);
      });
      // k step 1 on buffer 1 (its fragments are in: this wavefront is done
      // reading stage c).  After the last slice the same sequence waits for
      // and reads the slice past the end of the stream, which was issued like
      // any other: one branch-free sequence for every slice.
      wait_lgkm0();
      static_for<NM>([&](auto T) {
        constexpr int t = decltype(T)::value;
        if constexpr (t == BAR) {
          // slice c+1 has landed for this wavefront ... and for every
          // wavefront; and every wavefront is done reading stage c, which
          // the next issues overwrite
          wait_vmcnt<AFTER>();
          block_barrier();
        }
        mma(T, I_<1>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (t >= BAR)
          static_for<FPS>([&](auto F) {
            constexpr int d = FPS * (t - BAR) + decltype(F)::value;
            if constexpr (d < ND) frag(I_<d>{}, I_<0>{}, c + 1, 0);
          });
        dma_at(I_<NM + t>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }

    // no group: no output; a one-block task has no rows 128-255
    if (g >= 0 && (nb == 2 || wm == 0)) {
      const int s = i % kTabSlots;
      if constexpr (SCAT) {
        scatter_tile<4, NI>(acc, args.Dacc, N, pair_table(s), (const MOE_LDS float *)wtab[s],
                            args.topk, lane, wm * 128, n0 + wn * WC);
      } else if (SK && KS > 1) {
        // split K: this part's raw sums of the rows with a pair (the host
        // requires a table)
        partial_tile<NB, 4, NI>(acc, args.Dpart + (size_t)kpart(i) * args.part_R * NB * N, N,
                                pair_table(s), lane, wm * 128, n0 + wn * WC);
      } else {
        // staging: the stages of the slice just consumed, which every
        // wavefront finished reading at its barrier and which the next DMA
        // issue (in the next slice) overwrites -- the first half of the
        // wavefronts in the A stage, the second in the B stage, 32 rows x WC
        // columns each
        constexpr int SW = 32 * WC * 2;
        static_assert((WV / 2) * SW <= A_BYTES && (WV / 2) * SW <= BS_BYTES, "staging space");
        MOE_LDS unsigned char *stg =
            wave < WV / 2
                ? (MOE_LDS unsigned char *)aring + ((c - 1) % NA) * A_BYTES + wave * SW
                : (MOE_LDS unsigned char *)bring + ((c - 1) % NBR) * BS_BYTES +
                      (wave - WV / 2) * SW;
        // (the split form, with both epilogues in its loop, has no registers
        // for the store offsets hoisted out of it: an opaque copy of N keeps
        // them inside)
        int Ns = N;
        if constexpr (SK) asm volatile("" : "+s"(Ns));
        store_tile<NB, FP16, 4, NI>(acc, args.D + (size_t)b * kBM * N + n0, Ns,
                                    has_tab ? pair_table(s) : nullptr, lane, wm * 128, wn * WC,
                                    stg);
      }
    }
    // every wavefront's staging is read back before any wavefront issues the
    // next slice's DMA into those stages (the other epilogues stage nothing)
    if (!SCAT && !(SK && KS > 1)) block_barrier();
    clear_acc();
  }
  // drain any DMA still in flight before the workgroup retires its LDS
  wait_vmcnt<0>();
  lp_outputs();
}

template <int BN, int BK, int EPI, bool KN, bool FP16, int NA, int NBR, bool BNT, int WV = 4,
          bool LP = false, bool SK = false>
static hipError_t launch_one(const GGArgs &a, int grid, hipStream_t stream) {
  grouped_gemm_kernel<BN, BK, EPI, KN, FP16, NA, NBR, BNT, WV, LP, SK>
      <<<grid, 64 * WV, 0, stream>>>(a);
  return hipGetLastError();
}

// Tile configuration of one launch: BN (columns per matrix), BK (k per
// slice), A and B ring depths, row tasks per super-block of the task order,
// wavefronts per workgroup.
struct TileCfg {
  int bn, bk, na, nb, group;
  int waves = 4;
};

// The instantiated (BN, BK, NA, NBR) per B-matrix count; the rings stay
// within 144 KiB so the tables and staging tiles fit in the 160 KiB of LDS.
// Every BN has the 4/4 rings, safe for any K (2 KT >= 3).
inline bool tile_supported(int nbm, int bn, int bk, int na, int nb, int waves = 4) {
  if (bk != 32) return false;
  // eight wavefronts: the full-size rings of the default tiles, no scatter
  if (waves == 8)
    return na == 3 && ((nbm == 1 && bn == 256 && nb == 6) || (nbm == 2 && bn == 128 && (nb == 6 || nb == 4)));
  if (waves != 4) return false;
  if (na == 4 && nb == 4) return bn == 64 || bn == 128 || (bn == 256 && nbm == 1);
  if (nbm == 2) return (bn == 128 && na == 3 && nb == 6) || (bn == 64 && na == 3 && nb == 10);
  return (bn == 256 && na == 3 && nb == 6) || (bn == 128 && na == 3 && nb == 10) ||
         (bn == 64 && na == 4 && nb == 8);
}

// Launch of one (epilogue, B layout, dtype, B cache policy) combination
// with the tile shape c.  Explicitly instantiated in gg_inst.hip, one object
// per combination; the dispatcher declares those instantiations extern.
// The fused gate/up form (LP): bf16 [K][N] weights, the eight-wavefront
// 128-column tile (shorter K, which takes the four-wavefront tiles, runs the
// permutation as its own launch).
inline bool lp_tile(const TileCfg &c) {
  return c.bn == 128 && c.bk == 32 && c.waves == 8 && c.na == 3 && c.nb == 4;
}
template <bool BNT>
hipError_t launch_lp(const GGArgs &a, const TileCfg &c, int grid, hipStream_t s) {
  if (!lp_tile(c)) return hipErrorInvalidValue;
  return launch_one<128, 32, kEpiSiluMul, true, false, 3, 4, BNT, 8, true>(a, grid, s);
}

// The split-K form exists for the streamed bf16 [K][N] store and SiLU*up
// tiles of eight wavefronts (the shapes with fewer tasks than workgroups).
inline bool splitk_tile(int epilogue, const TileCfg &c) {
  return c.waves == 8 && c.bk == 32 && c.group >= 1 &&
         ((epilogue == kEpiStore && c.bn == 256 && c.na == 3 && c.nb == 6) ||
          (epilogue == kEpiSiluMul && c.bn == 128 && c.na == 3 && c.nb == 4));
}

template <int EPI, bool KN, bool FP16, bool BNT>
hipError_t launch_bn(const GGArgs &a, const TileCfg &c, int grid, hipStream_t s) {
  if (a.ksplit > 1) {
    if constexpr (KN && !FP16 && BNT && EPI != kEpiScatter) {
      if (!splitk_tile(EPI, c)) return hipErrorInvalidValue;
      if constexpr (EPI == kEpiSiluMul)
        return launch_one<128, 32, EPI, KN, FP16, 3, 4, BNT, 8, false, true>(a, grid, s);
      else
        return launch_one<256, 32, EPI, KN, FP16, 3, 6, BNT, 8, false, true>(a, grid, s);
    }
    return hipErrorInvalidValue;
  }
#define MOE_GG_CASE(BNV, NAV, NBV)                                                            \
  if (c.waves == 4 && c.bn == BNV && c.bk == 32 && c.na == NAV && c.nb == NBV)                \
    return launch_one<BNV, 32, EPI, KN, FP16, NAV, NBV, BNT>(a, grid, s);
#define MOE_GG_CASE8(BNV, NAV, NBV)                                                           \
  if (c.waves == 8 && c.bn == BNV && c.bk == 32 && c.na == NAV && c.nb == NBV)                \
    return launch_one<BNV, 32, EPI, KN, FP16, NAV, NBV, BNT, 8>(a, grid, s);
  if constexpr (EPI == kEpiSiluMul) {
    MOE_GG_CASE(128, 3, 6) MOE_GG_CASE(128, 4, 4) MOE_GG_CASE(64, 3, 10) MOE_GG_CASE(64, 4, 4)
    MOE_GG_CASE8(128, 3, 6) MOE_GG_CASE8(128, 3, 4)
  } else {
    MOE_GG_CASE(256, 3, 6) MOE_GG_CASE(256, 4, 4) MOE_GG_CASE(128, 3, 10) MOE_GG_CASE(128, 4, 4)
    MOE_GG_CASE(64, 4, 8) MOE_GG_CASE(64, 4, 4)
    if constexpr (EPI == kEpiStore) { MOE_GG_CASE8(256, 3, 6) }
  }
#undef MOE_GG_CASE
#undef MOE_GG_CASE8
  return hipErrorInvalidValue;
}

} // namespace moe
