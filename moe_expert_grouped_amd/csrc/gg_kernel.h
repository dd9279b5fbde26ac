// gg_kernel.h -- the grouped GEMM of the MoE layer on CDNA4 (gfx950): kernel
// templates, instantiated per (epilogue, B layout, dtype) by gg_inst.hip.
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
// consumer warps -- is prior art; this is the CDNA4 form of the same ideas):
//   * persistent grid of one 256-thread workgroup (4 wavefronts) per CU;
//     tasks are (row block, column block) pairs, row-block-major, counted
//     from the device-resident padded row count so the host never waits;
//   * the task list is cut into 8 contiguous ranges, one per XCD (workgroup
//     w runs on XCD w % 8), so the row blocks of one expert -- which share
//     its weight tiles -- run side by side on one XCD and meet in its L2;
//   * every workgroup streams its tasks' 64-deep K slices through an
//     NSTAGE-deep ring of LDS stages with direct global->LDS DMA
//     (global_load_lds_dwordx4): no registers are spent on staging and the
//     ring keeps NSTAGE-1 slices in flight, across task boundaries too;
//     completion is tracked per wavefront with s_waitcnt vmcnt and made
//     visible to the workgroup with one s_barrier per slice (the roles of
//     the pages' "arrived"/"finished" barriers);
//   * LDS rows are XOR-swizzled in 16-byte granules by permuting the source
//     address each lane fetches (the DMA writes lane-contiguously);
//   * A tiles (and B tiles stored [N][K]) are read with ds_read_b128; weight
//     tiles stored [K][N] are read with the gfx950 transpose read
//     ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//     column -- exactly the MFMA B-operand layout;
//   * v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulators in registers; each
//     wavefront owns a 64 x (BN/2) quarter of the 128 x BN tile.
#pragma once
#include <stdio.h>
#include <stdlib.h>

#include "common.h"

namespace moe {

constexpr int kBM = 128;
constexpr int kBK = 64;

// Wavefront layout of a workgroup: WAVES = 4 (one per SIMD, a 2 x 2 grid of
// 64 x BN/2 wave tiles) or 8 (two per SIMD, so one wavefront's LDS and DMA
// waits hide behind the other's MFMAs: a 2 x 4 grid of 64 x BN/4 wave tiles,
// or 4 x 2 of 32 x BN/2 when BN = 64).
template <int BN, int WAVES> struct WaveGrid {
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int WMR = WAVES == 4 ? 2 : (BN >= 128 ? 2 : 4); // wave rows
  static constexpr int WNC = WAVES / WMR;                          // wave columns
  static constexpr int WR = kBM / WMR;                             // rows per wave
  static constexpr int WC = BN / WNC;                              // columns per wave (per matrix)
  static constexpr int MI = WR / 32;
  static constexpr int NI = WC / 32;
  static_assert(WC >= 32 && WR >= 32, "wave tile");
};

struct GGArgs {
  const uint16_t *A;
  const int32_t *a_src_row;
  int a_src_div;
  const uint16_t *B;
  const uint16_t *B2;
  const int32_t *block_group;
  const int32_t *num_rows;
  uint16_t *D;
  int N, K, cap;
  int group_rows;  // row blocks per super-block of the task order (>= 1)
  float *partials; // partial tiles of a split tail (NULL: no split)
  // weighted scatter only: row r adds pair_w[p] * product into Dacc[p / topk]
  // (p = epi_row_pair[r], skipped when negative)
  float *Dacc;
  const int32_t *epi_row_pair;
  const float *pair_w;
  int topk;
};

// Epilogues: plain store, SiLU(gate) * up of two B matrices, weighted scatter.
enum { kEpiStore = 0, kEpiSiluMul = 1, kEpiScatter = 2 };

// 16-byte-granule XOR swizzle of a tile stored with 128-byte rows (A tiles,
// [N][K] B tiles).  Conflict-free ds_read_b128 of 16 consecutive rows at one
// logical granule for both 32- and 64-bank LDS views.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Swizzle of a [K][N] weight tile with BN columns (rows of 2*BN bytes), read
// with ds_read_b64_tr_b16: one 16-lane group reads 4 consecutive k rows x 32
// bytes, two groups read neighbouring 32-byte column pairs.
template <int BN> __device__ __forceinline__ int swz_kn(int k) {
  if constexpr (BN >= 128)
    return 2 * (k & 3) + 8 * (k & 1);
  else
    return 2 * (k & 3);
}

// Direct global->LDS DMA.  Issued through inline asm so that the compiler
// neither tracks these loads nor inserts its own (conservative) waits for
// them: lane i of the wavefront writes bytes [16 i, 16 i + 16) (or [4 i, 4 i
// + 4) for the dword form) after the wave-uniform LDS byte address in M0
// (one wait state between the M0 write and its use).  Completion is awaited
// explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(lds_addr)
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

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// ---------------------------------------------------------------------------
// Work schedule, shared by the GEMM kernel and the fixup kernel.
//
// Tasks (row block, column block) are cut into nx contiguous ranges, one per
// XCD (workgroup w runs on XCD w % nx); the S workgroups of an XCD take its
// tasks round-robin.  When the last round would be mostly empty (the XCD
// has rem = ntx mod S leftover tasks, rem <= 3/4 S) and a partial-tile buffer
// is given, those rem tasks are not handed out whole: their rem * KT
// k-slices are split evenly over the S workgroups (a stream-K tail).  A
// workgroup then owns at most two tail segments; a segment that covers a
// whole task is finished in place, the others store fp32 partial tiles that
// the fixup kernel sums in k order.
struct Sched {
  int nx, xcd, slot, S, KT, ncol, nblk;
  int tx0, full, rem; // first task of this XCD, tasks handed out whole, tail tasks
  long U;             // tail k-slices

  __device__ void init(const GGArgs &a, int bn, int grid, int block) {
    KT = a.K / kBK;
    const int mrows = max(0, min(a.num_rows[0], a.cap));
    nblk = mrows / kBM;
    ncol = a.N / bn;
    const int ntask = nblk * ncol;
    nx = (grid % 8 == 0) ? 8 : 1;
    xcd = block % nx;
    slot = block / nx;
    S = grid / nx;
    tx0 = (int)(((long)ntask * xcd) / nx);
    const int ntx = (int)(((long)ntask * (xcd + 1)) / nx) - tx0;
    full = ntx / S * S;
    rem = ntx - full;
    if (!a.partials || rem == 0 || rem * 4 > S * 3) {
      full = ntx;
      rem = 0;
    }
    U = (long)rem * KT;
  }
  __device__ int bound(int s) const { return (int)(U * s / S); }
  // tasks this workgroup receives whole
  __device__ int n_full() const { return full > slot ? (full - slot + S - 1) / S : 0; }
  // tail segments of slot s: [bound(s), bound(s+1)) in tail k-slices
  __device__ int n_tail(int s) const {
    const int r0 = bound(s), r1 = bound(s + 1);
    return r1 > r0 ? (r1 - 1) / KT - r0 / KT + 1 : 0;
  }
  // item i of this workgroup: task, k-slice range [ka, kb), tail task index or -1
  __device__ void item(int i, int &task, int &ka, int &kb, int &tt) const {
    const int nf = n_full();
    if (i < nf) {
      task = tx0 + slot + i * S;
      ka = 0;
      kb = KT;
      tt = -1;
    } else {
      const int r0 = bound(slot), r1 = bound(slot + 1);
      tt = r0 / KT + (i - nf);
      task = tx0 + full + tt;
      ka = max(r0, tt * KT) - tt * KT;
      kb = min(r1, (tt + 1) * KT) - tt * KT;
    }
  }
};

// Partial tile of one tail segment: ACC floats per thread, stored as
// [ACC/4][threads][4] so each store and load is one coalesced 16-byte access
// per lane.  Buffer (xcd, slot, j) holds the j-th tail segment (j < 2) of
// that workgroup.
__device__ __forceinline__ float *partial_tile(float *base, const Sched &sc, int s, int j,
                                               int acc_per_thread, int threads) {
  return base + ((size_t)(sc.xcd * sc.S + s) * 2 + j) * (size_t)acc_per_thread * threads;
}

// Epilogue of one 128 x BN output tile: every 32x32 accumulator tile goes,
// 16 rows at a time, through a per-wavefront LDS tile so that each lane
// writes one 16-byte row piece (the MFMA layout gives each lane one column
// of 4-row groups; registers 0-7 hold rows 0-15, registers 8-15 rows 16-31).
constexpr int kEpiLd = 40; // row pitch (elements) of the staging tile
template <int NB, bool FP16, int MI, int NI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NB][MI][NI], uint16_t *Dt, int N,
                                           MOE_LDS uint16_t *stg, int lane, int row0,
                                           int col0) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * ((r >> 2) & 1) + 4 * (lane >> 5) + (r & 3);
          float v = acc[0][i][j][r];
          if constexpr (NB == 2) {
            const float u = acc[1][i][j][r];
            v = v / (1.0f + __expf(-v)) * u;
          }
          stg[row * kEpiLd + (lane & 31)] = FP16 ? f32_to_f16(v) : f32_to_bf16(v);
        }
        const int row = lane >> 2;
        const int col = (lane & 3) * 8;
        const u32x4 q = *(const MOE_LDS u32x4 *)(stg + row * kEpiLd + col);
        uint16_t *dst = Dt + (size_t)(row0 + i * 32 + 16 * h + row) * N + col0 + j * 32 + col;
        *reinterpret_cast<u32x4 *>(dst) = q;
      }
}

// Weighted-scatter epilogue of one wavefront's share of a tile: row r adds
// w_p * acc into the fp32 token row p / k of Dacc, p = row_pair[r] (padding
// rows, p < 0, add nothing).  Lane l fetches the pair of wavefront row l
// once; each accumulator register then takes its row's destination and
// weight from that lane (ds_bpermute).  The adds are fp32 atomics at device
// scope, so the sum over a token's k rows is order-free (not bit-stable).
template <int MI, int NI>
__device__ __forceinline__ void scatter_tile(const f32x16 (&acc)[1][MI][NI], float *Dacc, int N,
                                             const int32_t *row_pair, const float *pair_w,
                                             int k, int lane, int col) {
  int dst = -1;
  float wt = 0.0f;
  if (lane < MI * 32) {
    const int p = row_pair[lane];
    if (p >= 0) {
      dst = p / k;
      wt = pair_w[p];
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int d = __shfl(dst, rl);
      const float w = __shfl(wt, rl);
      if (d >= 0) {
        float *o = Dacc + (size_t)d * N + col + (lane & 31);
#pragma unroll
        for (int j = 0; j < NI; ++j) unsafeAtomicAdd(o + j * 32, w * acc[0][i][j][r]);
      }
    }
}

// Task order inside the whole-task phase: super-blocks of `group_rows` row
// blocks; inside one, the column block varies slowest, so the row blocks of
// a super-block (mostly one expert) read each weight tile at about the same
// time and share it in L2, while a row block's A tile is reused by its
// column tasks.
__device__ __forceinline__ void task_coords(int task, int GR, int ncol, int nblk, int bn, int &b,
                                            int &n0) {
  const int span = GR * ncol;
  const int sb = task / span;
  const int r = task - sb * span;
  const int rows = min(GR, nblk - sb * GR);
  const int n = r / rows;
  b = sb * GR + (r - n * rows);
  n0 = n * bn;
}

// BN: output columns per task (per B matrix); EPI: kEpiStore, kEpiSiluMul
// (two B matrices) or kEpiScatter; KN: B stored [K][N] (else [N][K]);
// NSTAGE: LDS ring depth; WAVES: 4 or 8.
template <int BN, int EPI, bool KN, bool FP16, int NSTAGE, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void grouped_gemm_kernel(GGArgs args) {
  constexpr int NB = EPI == kEpiSiluMul ? 2 : 1; // B matrices
  using WG = WaveGrid<BN, WAVES>;
  constexpr int NT = WG::kThreads;
  constexpr int A_BYTES = kBM * kBK * 2;
  constexpr int B_BYTES = kBK * BN * 2;
  constexpr int STAGE_BYTES = A_BYTES + NB * B_BYTES;
  constexpr int MI = WG::MI;       // 32-high MFMA tiles per wavefront
  constexpr int NI = WG::NI;       // 32-wide MFMA tiles per wavefront per matrix
  constexpr int A_INSTR = 16 / WAVES;         // DMA instructions per wavefront per A slice
  constexpr int B_INSTR = BN / (8 * WAVES);   // per wavefront per B matrix per slice
  constexpr int LOADS = A_INSTR + NB * B_INSTR; // DMA ops per wavefront per slice
  constexpr int ROWS_PW = 8 * A_INSTR;        // A rows each wavefront loads
  constexpr int IDX_SLOTS = 4;     // per-wavefront ring of task index tables
  constexpr int IDX_WORDS = 40;    // words per table: source rows, the group at word 32
  constexpr int ACC = NB * MI * NI * 16; // accumulator floats per thread
  static_assert(B_INSTR >= 1 && ROWS_PW <= 32, "DMA split");
  static_assert(LOADS * (NSTAGE - 2) < 64, "vmcnt range");
  static_assert(NSTAGE >= 2 && NSTAGE <= IDX_SLOTS, "ring depth");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int32_t idx_lds[WAVES][IDX_SLOTS][IDX_WORDS];
  __shared__ __attribute__((aligned(16))) uint16_t epi_lds[WAVES][16 * kEpiLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WG::WNC;
  const int wn = wave % WG::WNC;
  const int N = args.N, K = args.K;

  Sched sc;
  sc.init(args, BN, gridDim.x, blockIdx.x);
  const int KT = sc.KT, ncol = sc.ncol, nblk = sc.nblk;
  const int n_items = sc.n_full() + sc.n_tail(sc.slot);
  auto coords = [&](int task, int &b, int &n0) {
    task_coords(task, args.group_rows, ncol, nblk, BN, b, n0);
  };

  const uint32_t smem_addr = lds_addr_of(smem);
  MOE_LDS int32_t(*my_idx)[IDX_WORDS] = (MOE_LDS int32_t(*)[IDX_WORDS])idx_lds[wave];

  // DMA the index table of `task` (the 32 source rows this wavefront loads
  // and the block's group) into ring slot `seq`.
  auto fetch_index = [&](int task, int seq) {
    int b, n0;
    coords(task, b, n0);
    const uint32_t dst = (uint32_t)(uintptr_t)&my_idx[seq % IDX_SLOTS][0];
    if (args.a_src_row) {
      if (lane < ROWS_PW)
        dma4(args.a_src_row + (size_t)b * kBM + wave * ROWS_PW + lane, dst);
      else if (lane == 32)
        dma4(args.block_group + b, dst); // lane 32 lands at word 32
    } else if (lane == 32) {
      dma4(args.block_group + b, dst);
    }
  };

  // ---------------- issue (producer) state ----------------
  int it_i = 0;   // item being issued
  int it_k = 0;   // next k-slice of it
  int it_kb = 0;  // end of its k-slice range
  int it_len = 0; // its length
  const unsigned char *a_src[A_INSTR];
  const unsigned char *b_src[NB][B_INSTR];

  // Point the per-lane DMA sources at `task`, whose index table sits in
  // ring slot `seq` and has landed.
  auto setup_issue = [&](int task, int seq) {
    int b, n0;
    coords(task, b, n0);
    const MOE_LDS int32_t *tab = my_idx[seq % IDX_SLOTS];
    const int g = tab[32];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      // instruction i covers tile rows (wave*A_INSTR+i)*8 .. +8, lane row lane/8
      const int row = (wave * A_INSTR + i) * 8 + (lane >> 3);
      int src = b * kBM + row;
      if (args.a_src_row) {
        const int p = tab[i * 8 + (lane >> 3)];
        src = p < 0 ? 0 : p / args.a_src_div; // padding rows read a valid row
      }
      const int c = (lane & 7) ^ swz128(row);
      a_src[i] = reinterpret_cast<const unsigned char *>(args.A) + ((size_t)src * K + c * 8) * 2;
    }
    const int gg = g < 0 ? 0 : g;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const uint16_t *Bm = (m == 0 ? args.B : args.B2) + (size_t)gg * K * N;
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) {
        if constexpr (KN) {
          constexpr int GPR = BN / 8;   // granules per k row
          constexpr int RPI = 64 / GPR; // k rows per instruction
          const int k = (wave * B_INSTR + i) * RPI + lane / GPR;
          const int c = (lane % GPR) ^ swz_kn<BN>(k);
          b_src[m][i] =
              reinterpret_cast<const unsigned char *>(Bm) + ((size_t)k * N + n0 + c * 8) * 2;
        } else {
          const int n = (wave * B_INSTR + i) * 8 + (lane >> 3);
          const int c = (lane & 7) ^ swz128(n);
          b_src[m][i] =
              reinterpret_cast<const unsigned char *>(Bm) + ((size_t)(n0 + n) * K + c * 8) * 2;
        }
      }
    }
  };

  auto begin_issue_item = [&](int i) {
    int task, ka, kb, tt;
    sc.item(i, task, ka, kb, tt);
    if (i + 1 < n_items) {
      int t2, a2, b2, tt2;
      sc.item(i + 1, t2, a2, b2, tt2);
      fetch_index(t2, i + 1);
    }
    setup_issue(task, i);
    it_k = ka;
    it_kb = kb;
    it_len = kb - ka;
  };

  int n_issued = 0;
  // DMA instruction q (0 <= q < LOADS) of the slice being issued: A first,
  // then each B matrix.
  auto issue_dma = [&](int q) {
    const uint32_t stage = smem_addr + (n_issued % NSTAGE) * STAGE_BYTES;
    if (q < A_INSTR) {
      dma16(a_src[q] + (size_t)it_k * kBK * 2, stage + (wave * A_INSTR + q) * 1024);
    } else {
      const int m = (q - A_INSTR) / B_INSTR;
      const int i = (q - A_INSTR) - m * B_INSTR;
      const size_t b_off = KN ? (size_t)it_k * kBK * N * 2 : (size_t)it_k * kBK * 2;
      dma16(b_src[m][i] + b_off,
            stage + A_BYTES + m * B_BYTES + (wave * B_INSTR + i) * 1024);
    }
  };
  // bookkeeping once every instruction of the slice is out
  auto issue_done = [&]() {
    ++n_issued;
    if (++it_k == it_kb) {
      ++it_i;
      if (it_i < n_items) {
        // the table of item it_i was fetched right before the first slice of
        // the previous item; once NSTAGE of that item's slices were issued
        // it has been awaited (DMA completes in order)
        if (it_len < NSTAGE) wait_vmcnt<0>();
        begin_issue_item(it_i);
      }
    }
  };
  auto issue_next = [&]() {
    if (it_i >= n_items) return;
#pragma unroll
    for (int q = 0; q < LOADS; ++q) issue_dma(q);
    issue_done();
  };

  if (n_items > 0) {
    int task, ka, kb, tt;
    sc.item(0, task, ka, kb, tt);
    fetch_index(task, 0);
    wait_vmcnt<0>();
    begin_issue_item(0);
  }
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) issue_next();

  // ---------------- compute (consumer) ----------------
  int n_consumed = 0;
  for (int i = 0; i < n_items; ++i) {
    int task, ka, kb, tt;
    sc.item(i, task, ka, kb, tt);
    f32x16 acc[NB][MI][NI];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          for (int r = 0; r < 16; ++r) acc[m][a][j][r] = 0.0f;
    int group = 0;

    for (int kt = ka; kt < kb; ++kt) {
      // this wavefront's DMA for slice n_consumed has landed ...
      if (n_issued - n_consumed - 1 >= NSTAGE - 2)
        wait_vmcnt<LOADS * (NSTAGE - 2)>();
      else
        wait_vmcnt<0>();
      // ... and so has every other wavefront's; everyone is done with the
      // stage the next issue overwrites
      block_barrier();
      if (kt == ka) group = __builtin_amdgcn_readfirstlane(my_idx[i % IDX_SLOTS][32]);
      // the next slice's DMA is spread over the k steps of this one, so the
      // address unit drains it in the background of the MFMAs
      const bool issuing = it_i < n_items;
      constexpr int PER = (LOADS + 3) / 4;

      const MOE_LDS unsigned char *sA =
          (const MOE_LDS unsigned char *)(smem + (n_consumed % NSTAGE) * STAGE_BYTES);
      // Fragments of one 16-deep k step, double-buffered in registers: the
      // LDS reads of step kk+1 are issued before the MFMAs of step kk, so
      // their latency hides behind matrix work (one wavefront per SIMD
      // leaves nothing else to hide it).
      i16x4 fa[2][MI][2];
      i16x4 fb[2][NB][NI][2];
      auto load_frags = [&](int kk, i16x4 (&a)[MI][2], i16x4 (&b)[NB][NI][2]) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int row = wm * WG::WR + mi * 32 + (lane & 31);
          const int c = (kk * 2 + (lane >> 5)) ^ swz128(row);
          const u32x4 v = *(const MOE_LDS u32x4 *)(sA + row * 128 + c * 16);
          a[mi][0] = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
          a[mi][1] = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
        }
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          const MOE_LDS unsigned char *sB = sA + A_BYTES + m * B_BYTES;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if constexpr (KN) {
              // lane group G = lane/16 reads columns n0 + 16*(G&1) .. +16 at
              // k = 8*(G>>1) + 4*r + (lane%16)/4; each lane points at 4
              // consecutive columns, the transpose read returns 4 k of one column
              const int G = lane >> 4;
              const int q = lane & 15;
              const int n = wn * WG::WC + j * 32 + 16 * (G & 1) + 4 * (q & 3);
              const int k0 = kk * 16 + 8 * (G >> 1) + (q >> 2);
              const int k1 = k0 + 4;
              const int o0 = k0 * (BN * 2) + (((n >> 3) ^ swz_kn<BN>(k0)) << 4) + ((n & 7) << 1);
              const int o1 = k1 * (BN * 2) + (((n >> 3) ^ swz_kn<BN>(k1)) << 4) + ((n & 7) << 1);
              b[m][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4 *)(sB + o0));
              b[m][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4 *)(sB + o1));
            } else {
              const int n = wn * WG::WC + j * 32 + (lane & 31);
              const int c = (kk * 2 + (lane >> 5)) ^ swz128(n);
              const u32x4 v = *(const MOE_LDS u32x4 *)(sB + n * 128 + c * 16);
              b[m][j][0] = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
              b[m][j][1] = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
            }
          }
        }
      };
      load_frags(0, fa[0], fb[0]);
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < kBK / 16) load_frags(kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
        if (issuing) {
#pragma unroll
          for (int q = kk * PER; q < (kk + 1) * PER && q < LOADS; ++q) issue_dma(q);
        }
        // keep the next step's reads and this DMA share ahead of the MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
              acc[m][mi][j] = mfma32<FP16>(fa[cur][mi][0], fa[cur][mi][1], fb[cur][m][j][0],
                                           fb[cur][m][j][1], acc[m][mi][j]);
      }
      if (issuing) issue_done();
      ++n_consumed;
    }

    if (group < 0) continue; // block without a group: no output
    if (ka == 0 && kb == KT) {
      int b, n0;
      coords(task, b, n0);
      if constexpr (EPI == kEpiScatter)
        scatter_tile<MI, NI>(acc, args.Dacc, N, args.epi_row_pair + (size_t)b * kBM + wm * WG::WR,
                             args.pair_w, args.topk, lane, n0 + wn * WG::WC);
      else
        store_tile<NB, FP16, MI, NI>(acc, args.D + (size_t)b * kBM * N + n0, N,
                                     (MOE_LDS uint16_t *)epi_lds[wave], lane, wm * WG::WR,
                                     wn * WG::WC);
    } else {
      // a piece of a split tail task: store the fp32 partial tile
      float *pt = partial_tile(args.partials, sc, sc.slot, tt - sc.bound(sc.slot) / KT, ACC, NT);
      const float *flat = reinterpret_cast<const float *>(&acc[0][0][0]);
#pragma unroll
      for (int q = 0; q < ACC / 4; ++q) {
        f32x4 v = {flat[4 * q], flat[4 * q + 1], flat[4 * q + 2], flat[4 * q + 3]};
        *reinterpret_cast<f32x4 *>(pt + ((size_t)q * NT + tid) * 4) = v;
      }
    }
  }
  // drain any DMA still in flight before the workgroup retires its LDS
  wait_vmcnt<0>();
}

// Sums the partial tiles of every split tail task in k order (deterministic)
// and runs the epilogue.  One workgroup per (XCD, tail task); launched with
// the same grid size as the GEMM so the schedule is recomputed identically.
template <int BN, int EPI, bool FP16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void grouped_gemm_fixup(GGArgs args, int gemm_grid) {
  constexpr int NB = EPI == kEpiSiluMul ? 2 : 1;
  using WG = WaveGrid<BN, WAVES>;
  constexpr int NT = WG::kThreads;
  constexpr int MI = WG::MI;
  constexpr int NI = WG::NI;
  constexpr int ACC = NB * MI * NI * 16;
  __shared__ __attribute__((aligned(16))) uint16_t epi_lds[WAVES][16 * kEpiLd];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  Sched sc;
  // blockIdx.x = xcd + nx * tail task index: reuse the XCD / slot fields
  sc.init(args, BN, gemm_grid, blockIdx.x % (gemm_grid % 8 == 0 ? 8 : 1));
  const int tt = blockIdx.x / sc.nx;
  if (tt >= sc.rem) return;
  const int KT = sc.KT;
  // segments of tail task tt, in k order
  int nseg = 0;
  for (int s = 0; s < sc.S; ++s)
    if (max(sc.bound(s), tt * KT) < min(sc.bound(s + 1), (tt + 1) * KT)) ++nseg;
  if (nseg < 2) return; // finished in place by the GEMM kernel
  const int task = sc.tx0 + sc.full + tt;
  int b, n0;
  task_coords(task, args.group_rows, sc.ncol, sc.nblk, BN, b, n0);
  if (args.block_group[b] < 0) return;

  f32x16 acc[NB][MI][NI];
  float *flat = reinterpret_cast<float *>(&acc[0][0][0]);
  bool first = true;
  for (int s = 0; s < sc.S; ++s) {
    if (!(max(sc.bound(s), tt * KT) < min(sc.bound(s + 1), (tt + 1) * KT))) continue;
    const float *pt = partial_tile(args.partials, sc, s, tt - sc.bound(s) / KT, ACC, NT);
#pragma unroll
    for (int q = 0; q < ACC / 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(pt + ((size_t)q * NT + tid) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) flat[4 * q + e] = first ? v[e] : flat[4 * q + e] + v[e];
    }
    first = false;
  }
  const int wm = wave / WG::WNC, wn = wave % WG::WNC;
  if constexpr (EPI == kEpiScatter)
    scatter_tile<MI, NI>(acc, args.Dacc, args.N, args.epi_row_pair + (size_t)b * kBM + wm * WG::WR,
                         args.pair_w, args.topk, lane, n0 + wn * WG::WC);
  else
    store_tile<NB, FP16, MI, NI>(acc, args.D + (size_t)b * kBM * args.N + n0, args.N,
                                 (MOE_LDS uint16_t *)epi_lds[wave], lane, wm * WG::WR,
                                 wn * WG::WC);
}

template <int BN, int EPI, bool KN, bool FP16, int NSTAGE, int WAVES>
static hipError_t launch_one(const GGArgs &a, int grid, hipStream_t stream) {
  grouped_gemm_kernel<BN, EPI, KN, FP16, NSTAGE, WAVES><<<grid, 64 * WAVES, 0, stream>>>(a);
  if (a.partials)
    grouped_gemm_fixup<BN, EPI, FP16, WAVES><<<grid, 64 * WAVES, 0, stream>>>(a, grid);
  return hipGetLastError();
}

// Tile configuration of one launch: BN (columns per matrix), LDS ring depth,
// super-block rows of the task order, split tail on/off, wavefronts (4 or 8).
struct TileCfg {
  int bn, stages, group, split, waves;
};

// instantiated (BN, stages) per B-matrix count; LDS: ring + 4 KiB index
// tables + 10 KiB epilogue tiles <= 160 KiB
inline bool tile_supported(int nb, int bn, int stages) {
  if (stages < 2 || stages > 4) return false;
  if (bn == 64) return true;
  if (bn == 128) return nb == 1 || stages <= 3;
  if (bn == 256) return nb == 1 && stages <= 3;
  return false;
}

// Launch of one (epilogue, B layout, dtype) combination with the tile shape
// c.  Explicitly instantiated in gg_inst.hip, one object per combination;
// the dispatcher declares those instantiations extern.
template <int EPI, bool KN, bool FP16>
hipError_t launch_bn(const GGArgs &a, const TileCfg &c, int grid, hipStream_t s) {
  constexpr int NB = EPI == kEpiSiluMul ? 2 : 1;
#define MOE_GG_CASE(BNV, NSV)                                                                 \
  if (c.bn == BNV && c.stages == NSV)                                                         \
    return c.waves == 8 ? launch_one<BNV, EPI, KN, FP16, NSV, 8>(a, grid, s)                  \
                        : launch_one<BNV, EPI, KN, FP16, NSV, 4>(a, grid, s);
  MOE_GG_CASE(64, 2) MOE_GG_CASE(64, 3) MOE_GG_CASE(64, 4)
  MOE_GG_CASE(128, 2) MOE_GG_CASE(128, 3)
  if constexpr (NB == 1) {
    MOE_GG_CASE(128, 4)
    MOE_GG_CASE(256, 2) MOE_GG_CASE(256, 3)
  }
#undef MOE_GG_CASE
  return hipErrorInvalidValue;
}

} // namespace moe
