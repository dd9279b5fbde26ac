// grouped_gemm.hip -- the grouped GEMM of the MoE layer on CDNA4 (gfx950).
//
// What it computes ("Comm-compute fusion (3)", section 4, the grouped GEMM
// template): output rows come in 128-row blocks; block b belongs to group
// g = block_group[b] and every row r of it is  D[r] = A[a(r)] . B[g], where
// a(r) is r itself or the token row named by the permutation (the
// reorder-by-route prologue of the MoE layer0 row, "Comm-compute fusion (1)",
// section 4).  The SiLU*up epilogue fuses the activation of the serial layer
// (gate/up GEMM -> SiLU -> down GEMM, part (1), section 1) into the gate/up
// GEMM: B holds the gate weights, B2 the up weights, and each workgroup
// accumulates matching gate and up column tiles side by side.
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
#include "common.h"

namespace moe {

constexpr int kBM = 128;
constexpr int kBK = 64;
constexpr int kThreads = 256;

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
};

// 16-byte-granule XOR swizzle of a tile stored with 128-byte rows (A tiles,
// [N][K] B tiles).  Conflict-free ds_read_b128 of 16 consecutive rows at one
// logical granule for both 32- and 64-bank LDS views.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Swizzle of a [K][N] weight tile with BN columns (rows of 2*BN bytes), read
// with ds_read_b64_tr_b16: one 16-lane group reads 4 consecutive k rows x 32
// bytes, two groups read neighbouring 32-byte column pairs.
template <int BN> __device__ __forceinline__ int swz_kn(int k) {
  if constexpr (BN == 128)
    return 2 * (k & 3) + 8 * (k & 1);
  else
    return 2 * (k & 3);
}

// Direct global->LDS DMA.  Issued through inline asm so that the compiler
// neither tracks these loads nor inserts its own (conservative) waits for
// them: lane i of the wavefront writes bytes [16 i, 16 i + 16) (or [4 i, 4 i
// + 4) for the dword form) after the wave-uniform LDS byte address in M0.
// Completion is awaited explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr)
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

// BN: output columns per task (per B matrix); NB: 1 (STORE) or 2 (gate+up);
// KN: B stored [K][N] (else [N][K]); NSTAGE: LDS ring depth.
template <int BN, int NB, bool KN, bool FP16, int NSTAGE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GGArgs args) {
  constexpr int A_BYTES = kBM * kBK * 2;
  constexpr int B_BYTES = kBK * BN * 2;
  constexpr int STAGE_BYTES = A_BYTES + NB * B_BYTES;
  constexpr int WN = BN / 2;       // columns per wavefront per matrix
  constexpr int NI = WN / 32;      // 32-wide MFMA tiles per wavefront per matrix
  constexpr int MI = 2;            // 32-high MFMA tiles per wavefront
  constexpr int A_INSTR = 4;       // DMA instructions per wavefront per A slice
  constexpr int B_INSTR = BN / 32; // per wavefront per B matrix per slice
  constexpr int LOADS = A_INSTR + NB * B_INSTR; // DMA ops per wavefront per slice
  constexpr int IDX_SLOTS = 8;     // per-wavefront ring of task index tables
  constexpr int IDX_WORDS = 64;    // words per table: 32 source rows, then the group
  static_assert(LOADS * (NSTAGE - 2) < 64, "vmcnt range");
  static_assert(NSTAGE >= 2 && NSTAGE < IDX_SLOTS, "ring depth");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE_BYTES];
  __shared__ __attribute__((aligned(256))) int32_t idx_lds[4][IDX_SLOTS][IDX_WORDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int N = args.N, K = args.K;
  const int KT = K / kBK;
  const int mrows = max(0, min(args.num_rows[0], args.cap));
  const int nblk = mrows / kBM;
  const int ncol = N / BN;
  const int ntask = nblk * ncol;

  // XCD-aware split: contiguous task ranges per XCD, round-robin slots inside
  const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
  const int xcd = blockIdx.x % nx;
  const int slot = blockIdx.x / nx;
  const int S = gridDim.x / nx;
  const int t_end = (int)(((long)ntask * (xcd + 1)) / nx);
  const int t_first = (int)(((long)ntask * xcd) / nx) + slot;

  const uint32_t smem_addr = lds_addr_of(smem);
  MOE_LDS int32_t(*my_idx)[IDX_WORDS] = (MOE_LDS int32_t(*)[IDX_WORDS])idx_lds[wave];

  // DMA the index table of task `task` (the 32 source rows this wavefront
  // loads and the block's group) into ring slot `seq`.
  auto fetch_index = [&](int task, int seq) {
    const int b = task / ncol;
    const uint32_t dst = (uint32_t)(uintptr_t)&my_idx[seq % IDX_SLOTS][0];
    if (args.a_src_row) {
      if (lane < 32)
        dma4(args.a_src_row + (size_t)b * kBM + wave * 32 + lane, dst);
      else if (lane == 32)
        dma4(args.block_group + b, dst); // lane 32 lands at word 32
    } else if (lane == 32) {
      dma4(args.block_group + b, dst);
    }
  };

  // ---------------- issue (producer) state ----------------
  int it_task = t_first;
  int it_seq = 0; // sequence number of it_task among this workgroup's tasks
  int it_kt = 0;
  const unsigned char *a_src[A_INSTR];
  const unsigned char *b_src[NB][B_INSTR];

  // Point the per-lane DMA sources at task `task`, whose index table sits in
  // ring slot `seq` and has landed.
  auto setup_issue = [&](int task, int seq) {
    const int b = task / ncol;
    const int n0 = (task - b * ncol) * BN;
    const MOE_LDS int32_t *tab = my_idx[seq % IDX_SLOTS];
    const int g = tab[32];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      // instruction i covers tile rows (wave*4+i)*8 .. +8, lane row lane/8
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

  int n_issued = 0;
  auto issue_next = [&]() {
    if (it_task >= t_end) return;
    const uint32_t stage = smem_addr + (n_issued % NSTAGE) * STAGE_BYTES;
    const size_t a_off = (size_t)it_kt * kBK * 2;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) dma16(a_src[i] + a_off, stage + (wave * A_INSTR + i) * 1024);
    const size_t b_off = KN ? (size_t)it_kt * kBK * N * 2 : (size_t)it_kt * kBK * 2;
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i)
        dma16(b_src[m][i] + b_off, stage + A_BYTES + m * B_BYTES + (wave * B_INSTR + i) * 1024);
    ++n_issued;
    if (++it_kt == KT) {
      it_kt = 0;
      it_task += S;
      ++it_seq;
      if (it_task < t_end) {
        // the table of it_task was fetched before the first slice of the
        // previous task; with KT >= NSTAGE that slice has been awaited
        if (KT < NSTAGE) wait_vmcnt<0>();
        if (it_task + S < t_end) fetch_index(it_task + S, it_seq + 1);
        setup_issue(it_task, it_seq);
      }
    }
  };

  if (it_task < t_end) {
    fetch_index(it_task, 0);
    wait_vmcnt<0>();
    if (it_task + S < t_end) fetch_index(it_task + S, 1);
    setup_issue(it_task, 0);
  }
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) issue_next();

  // ---------------- compute (consumer) ----------------
  int n_consumed = 0;
  int seq = 0;
  for (int task = t_first; task < t_end; task += S, ++seq) {
    f32x16 acc[NB][MI][NI];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;
    int group = 0;

    for (int kt = 0; kt < KT; ++kt) {
      // this wavefront's DMA for slice n_consumed has landed ...
      if (n_issued - n_consumed - 1 >= NSTAGE - 2)
        wait_vmcnt<LOADS * (NSTAGE - 2)>();
      else
        wait_vmcnt<0>();
      // ... and so has every other wavefront's; everyone is done with the
      // stage the next issue overwrites
      block_barrier();
      if (kt == 0) group = my_idx[seq % IDX_SLOTS][32];
      issue_next();

      const MOE_LDS unsigned char *sA =
          (const MOE_LDS unsigned char *)(smem + (n_consumed % NSTAGE) * STAGE_BYTES);
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        i16x4 a[MI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int row = wm * 64 + i * 32 + (lane & 31);
          const int c = (kk * 2 + (lane >> 5)) ^ swz128(row);
          const u32x4 v = *(const MOE_LDS u32x4 *)(sA + row * 128 + c * 16);
          a[i][0] = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
          a[i][1] = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
        }
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          const MOE_LDS unsigned char *sB = sA + A_BYTES + m * B_BYTES;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            i16x4 b0, b1;
            if constexpr (KN) {
              // lane group G = lane/16 reads columns n0 + 16*(G&1) .. +16 at
              // k = 8*(G>>1) + 4*r + (lane%16)/4; each lane points at 4
              // consecutive columns, the transpose read returns 4 k of one column
              const int G = lane >> 4;
              const int q = lane & 15;
              const int n = wn * WN + j * 32 + 16 * (G & 1) + 4 * (q & 3);
              const int k0 = kk * 16 + 8 * (G >> 1) + (q >> 2);
              const int k1 = k0 + 4;
              const int o0 = k0 * (BN * 2) + (((n >> 3) ^ swz_kn<BN>(k0)) << 4) + ((n & 7) << 1);
              const int o1 = k1 * (BN * 2) + (((n >> 3) ^ swz_kn<BN>(k1)) << 4) + ((n & 7) << 1);
              b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4 *)(sB + o0));
              b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4 *)(sB + o1));
            } else {
              const int n = wn * WN + j * 32 + (lane & 31);
              const int c = (kk * 2 + (lane >> 5)) ^ swz128(n);
              const u32x4 v = *(const MOE_LDS u32x4 *)(sB + n * 128 + c * 16);
              b0 = __builtin_bit_cast(i16x4, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
              b1 = __builtin_bit_cast(i16x4, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
              acc[m][i][j] = mfma32<FP16>(a[i][0], a[i][1], b0, b1, acc[m][i][j]);
          }
        }
      }
      ++n_consumed;
    }

    // ---------------- epilogue ----------------
    if (group < 0) continue; // block without a group: no output
    const int b = task / ncol;
    const int n0 = (task - b * ncol) * BN;
    uint16_t *Dt = args.D + (size_t)b * kBM * N + n0;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * WN + j * 32 + (lane & 31);
          float v = acc[0][i][j][r];
          if constexpr (NB == 2) {
            const float u = acc[1][i][j][r];
            v = v / (1.0f + __expf(-v)) * u;
          }
          Dt[(size_t)row * N + col] = FP16 ? f32_to_f16(v) : f32_to_bf16(v);
        }
  }
  // drain any DMA still in flight before the workgroup retires its LDS
  wait_vmcnt<0>();
}

template <int BN, int NB, bool KN, bool FP16, int NSTAGE>
static hipError_t launch_one(const GGArgs &a, int grid, hipStream_t stream) {
  grouped_gemm_kernel<BN, NB, KN, FP16, NSTAGE><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// dtype 0 bf16 / 1 fp16; layout 0 KN / 1 NK; epilogue 0 STORE / 1 SILU_MUL
hipError_t launch_grouped_gemm(int dtype, int N, int K, int cap, const uint16_t *A,
                               const int32_t *a_src_row, int a_src_div, const uint16_t *B,
                               const uint16_t *B2, int layout, const int32_t *block_group,
                               const int32_t *num_rows, int epilogue, uint16_t *D, int num_cus,
                               hipStream_t stream) {
  GGArgs a{A, a_src_row, a_src_div, B, B2, block_group, num_rows, D, N, K, cap};
  const int grid = num_cus; // one workgroup per CU (LDS-limited)
  const bool fp16 = dtype == 1;
  const bool kn = layout == 0;
  if (epilogue == 1) {
    // gate + up, 64 columns each
    if (kn && !fp16) return launch_one<64, 2, true, false, 4>(a, grid, stream);
    if (kn && fp16) return launch_one<64, 2, true, true, 4>(a, grid, stream);
    if (!kn && !fp16) return launch_one<64, 2, false, false, 4>(a, grid, stream);
    return launch_one<64, 2, false, true, 4>(a, grid, stream);
  }
  if (N % 128 == 0) {
    if (kn && !fp16) return launch_one<128, 1, true, false, 4>(a, grid, stream);
    if (kn && fp16) return launch_one<128, 1, true, true, 4>(a, grid, stream);
    if (!kn && !fp16) return launch_one<128, 1, false, false, 4>(a, grid, stream);
    return launch_one<128, 1, false, true, 4>(a, grid, stream);
  }
  if (kn && !fp16) return launch_one<64, 1, true, false, 4>(a, grid, stream);
  if (kn && fp16) return launch_one<64, 1, true, true, 4>(a, grid, stream);
  if (!kn && !fp16) return launch_one<64, 1, false, false, 4>(a, grid, stream);
  return launch_one<64, 1, false, true, 4>(a, grid, stream);
}

} // namespace moe
