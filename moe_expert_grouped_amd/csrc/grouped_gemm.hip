// grouped_gemm.hip -- host side of the grouped GEMM: tile-shape choice and
// dispatch to the per-(epilogue, B layout, dtype) instantiations of the
// kernel templates in gg_kernel.h (compiled from gg_inst.hip, one object per
// combination, so they build in parallel).
#include "gg_kernel.h"

namespace moe {

#define MOE_GG_EXTERN(EPI, KN, FP16, NT)                                                      \
  extern template hipError_t launch_bn<EPI, KN, FP16, NT>(const GGArgs &, const TileCfg &, int, \
                                                           hipStream_t);
MOE_GG_EXTERN(kEpiStore, true, false, false)
MOE_GG_EXTERN(kEpiStore, true, true, false)
MOE_GG_EXTERN(kEpiStore, false, false, false)
MOE_GG_EXTERN(kEpiStore, false, true, false)
MOE_GG_EXTERN(kEpiSiluMul, true, false, false)
MOE_GG_EXTERN(kEpiSiluMul, true, true, false)
MOE_GG_EXTERN(kEpiSiluMul, false, false, false)
MOE_GG_EXTERN(kEpiSiluMul, false, true, false)
MOE_GG_EXTERN(kEpiScatter, true, false, false)
MOE_GG_EXTERN(kEpiScatter, true, true, false)
// weights streamed with the non-temporal policy ([K][N] layouts only)
MOE_GG_EXTERN(kEpiStore, true, false, true)
MOE_GG_EXTERN(kEpiStore, true, true, true)
MOE_GG_EXTERN(kEpiSiluMul, true, false, true)
MOE_GG_EXTERN(kEpiSiluMul, true, true, true)
MOE_GG_EXTERN(kEpiScatter, true, false, true)
MOE_GG_EXTERN(kEpiScatter, true, true, true)
#undef MOE_GG_EXTERN
extern template hipError_t launch_lp<false>(const GGArgs &, const TileCfg &, int, hipStream_t);
extern template hipError_t launch_lp<true>(const GGArgs &, const TileCfg &, int, hipStream_t);

// Tile configurations: (BN, BK, A ring depth, B ring depth, super-block row
// tasks, wavefronts).  Defaults: gate/up 128 gate + 128 up columns, down /
// dense 256 columns (128 when N is not a multiple of 256, 64 below that),
// 32-deep slices, a 3-deep A ring and a 6-deep B ring (weights are most of
// the bytes in flight; gate/up takes a 4-deep one, which measured 2-5 %
// faster where the weights stream and the same where they are re-read,
// while down was faster with 6); the 128 / 256-column tiles with eight wavefronts
// (two per SIMD: one's matrix instructions run while the other issues its
// fragment reads and DMA), except for the weighted scatter.  A configuration
// is used only if it is instantiated, divides N, and its B ring keeps the
// per-task tables safe for this K (2 * K / BK >= nb - 1); otherwise the
// 4-deep rings, instantiated for every BN.  grouped_gemm_tuned (tests and
// tuning sweeps) names another instantiated configuration explicitly; the
// product entry points always take this choice.
static bool tile_usable(const TileCfg &c, int epilogue, int N, int K) {
  return c.group >= 1 && c.bn > 0 && c.bk > 0 && N % c.bn == 0 && K % c.bk == 0 &&
         (c.waves == 4 || epilogue != kEpiScatter) &&
         2 * (K / c.bk) >= c.nb - 1 &&
         tile_supported(epilogue == kEpiSiluMul ? 2 : 1, c.bn, c.bk, c.na, c.nb, c.waves);
}

static TileCfg tile_config(int epilogue, int N, int K) {
  TileCfg c;
  // the full-size tiles run eight wavefronts (two per SIMD) except the
  // weighted scatter
  const int w = epilogue == kEpiScatter ? 4 : 8;
  if (epilogue == kEpiSiluMul)
    c = N % 128 == 0 ? TileCfg{128, 32, 3, w == 8 ? 4 : 6, 1, w} : TileCfg{64, 32, 3, 10, 1};
  else
    c = N % 256 == 0 ? TileCfg{256, 32, 3, 6, 1, w}
                     : (N % 128 == 0 ? TileCfg{128, 32, 3, 10, 1} : TileCfg{64, 32, 4, 8, 1});
  if (!tile_usable(c, epilogue, N, K)) { // short K: shallower rings, four wavefronts
    c.na = c.nb = 4;
    c.waves = 4;
  }
  return c;
}

// An explicit tile configuration {bn, bk, na, nb, group rows, wavefronts}
// (grouped_gemm_tuned): whether this GEMM can run it.
bool gg_tile_usable(const int32_t *t, int epilogue, int N, int K) {
  const TileCfg c{t[0], t[1], t[2], t[3], t[4], t[5]};
  return tile_usable(c, epilogue, N, K);
}

// Plan of row tasks (one workgroup of 1024 threads): inside each maximal run
// of blocks with the same non-negative group, blocks are paired from the
// run's first block; a run of odd length ends in a one-block task.  Blocks
// with a negative group get no task.  Chunks of 1024 blocks carry the open
// run's first block and the task count.
__global__ __launch_bounds__(1024) void gg_plan_kernel(const int32_t *__restrict__ block_group,
                                                       const int32_t *__restrict__ num_rows,
                                                       int cap, int32_t *__restrict__ plan) {
  __shared__ int s_start[16]; // per wavefront: the last run start it saw
  __shared__ int s_heads[16]; // per wavefront: its pair heads
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nblk = max(0, min(num_rows[0], cap)) / kBM;
  int carry_start = -1, carry_count = 0; // over the chunks before
  for (int base = 0; base < nblk; base += 1024) {
    const int b = base + t;
    const int g = b < nblk ? block_group[b] : -1;
    const int gp = (b > 0 && b < nblk) ? block_group[b - 1] : -1;
    const int gn = (b + 1 < nblk) ? block_group[b + 1] : -1;
    const bool start = g >= 0 && (b == 0 || gp != g);
    // the start of block b's run: inclusive max-scan of run starts
    int rs = wave_incl_max_scan(start ? b : -1);
    if (lane == 63) s_start[w] = rs;
    __syncthreads();
    int before = carry_start;
    for (int j = 0; j < w; ++j) before = max(before, s_start[j]);
    rs = max(rs, before);
    // a pair head is a block at an even distance from its run's start
    const bool head = g >= 0 && ((b - rs) & 1) == 0;
    const int hs = wave_incl_scan(head ? 1 : 0);
    if (lane == 63) s_heads[w] = hs;
    __syncthreads();
    int idx = carry_count + hs - 1;
    for (int j = 0; j < w; ++j) idx += s_heads[j];
    if (head) {
      plan[kPlanHead + 2 * idx] = b | (gn == g ? kPlanTwo : 0);
      plan[kPlanHead + 2 * idx + 1] = g;
    }
    for (int j = 0; j < 16; ++j) {
      carry_start = max(carry_start, s_start[j]);
      carry_count += s_heads[j];
    }
    __syncthreads(); // the next chunk rewrites s_start / s_heads
  }
  if (t == 0) {
    plan[0] = carry_count;
    plan[1] = nblk;
  }
}

size_t gg_plan_bytes(int cap) { return plan_ints(cap) * sizeof(int32_t); }

// Builds the row-task plan of block_group / num_rows into `plan`.
hipError_t launch_gg_plan(const int32_t *block_group, const int32_t *num_rows, int cap,
                          int32_t *plan, hipStream_t stream) {
  gg_plan_kernel<<<1, 1024, 0, stream>>>(block_group, num_rows, cap, plan);
  return hipGetLastError();
}

// [K][N] weights loaded with the non-temporal policy (each weight tile read
// by about one row task: streamed, not kept in the caches)
static hipError_t launch_kn_stream(const GGArgs &a, const TileCfg &c, int epilogue, bool fp16,
                                   int grid, hipStream_t stream) {
  if (epilogue == kEpiScatter)
    return fp16 ? launch_bn<kEpiScatter, true, true, true>(a, c, grid, stream)
                : launch_bn<kEpiScatter, true, false, true>(a, c, grid, stream);
  if (epilogue == kEpiSiluMul)
    return fp16 ? launch_bn<kEpiSiluMul, true, true, true>(a, c, grid, stream)
                : launch_bn<kEpiSiluMul, true, false, true>(a, c, grid, stream);
  return fp16 ? launch_bn<kEpiStore, true, true, true>(a, c, grid, stream)
              : launch_bn<kEpiStore, true, false, true>(a, c, grid, stream);
}

// dtype 0 bf16 / 1 fp16; layout 0 KN / 1 NK / 2 KN with gate and up
// interleaved in 128-column blocks (SILU_MUL; B2 unused); epilogue 0 STORE / 1 SILU_MUL /
// 2 WEIGHTED_SCATTER (KN only; D is then the fp32 token-row accumulator);
// b_stream: B loaded with the non-temporal policy (KN only).  `plan` holds
// the row-task plan of block_group (launch_gg_plan), built earlier on the
// same stream.  grid: persistent workgroups (one per CU in the product
// path; LDS holds one per CU, any count >= 1 computes the same result);
// tile: NULL for the default configuration.
// ksplit > 1 (split K, the layer's shapes with fewer tasks than workgroups):
// the GEMM writes each k part's raw fp32 sums of the rows with a pair to
// Dpart ([ksplit][part_R][NB][N], see GGArgs) instead of D, for a
// reduction kernel (splitk.hip) to finish; streamed bf16 [K][N] weights, the
// store or SiLU*up epilogue, a row table, the default tile, and K / 32 a
// multiple of ksplit with at least 4 slices per part.
hipError_t launch_grouped_gemm(int dtype, int N, int K, const uint16_t *A,
                               const int32_t *a_src_row, int a_src_div, const uint16_t *B,
                               const uint16_t *B2, int layout, const int32_t *plan, int epilogue,
                               const int32_t *epi_row_pair, const float *pair_w, int topk,
                               void *D, int grid, bool b_stream, hipStream_t stream,
                               const int32_t *tile, int ksplit, float *Dpart, int part_R) {
  // the default configuration, or the explicit one of grouped_gemm_tuned
  // (checked by gg_tile_usable before the call)
  const TileCfg c =
      tile ? TileCfg{tile[0], tile[1], tile[2], tile[3], tile[4], tile[5]} : tile_config(epilogue, N, K);
  if (tile && !tile_usable(c, epilogue, N, K)) return hipErrorInvalidValue;
  const bool scat = epilogue == kEpiScatter;
  const bool il = layout == 2; // [K][2N], gate/up interleaved in 128-column blocks
  GGArgs a{A, a_src_row, a_src_div, B, il ? B : B2, plan,
           scat ? nullptr : (uint16_t *)D, scat ? (float *)D : nullptr,
           epi_row_pair, pair_w, topk, N, K, c.group, il ? 2 * N : N, il ? 1 : 0};
  const bool fp16 = dtype == 1;
  const bool kn = layout == 0 || il;
  if (il && (epilogue != kEpiSiluMul || N % 128 != 0 || c.bn > 128 || 128 % c.bn != 0))
    return hipErrorInvalidValue;
  if (ksplit > 1) {
    const int kt = K / 32 / ksplit;
    if (!b_stream || fp16 || !kn || scat || tile || !Dpart || part_R <= 0 ||
        (ksplit != 2 && ksplit != 4) || K % (32 * ksplit) != 0 || kt < 4 ||
        2 * kt < c.nb - 1 || !splitk_tile(epilogue, c) ||
        !(a_src_row || epi_row_pair))
      return hipErrorInvalidValue;
    a.ksplit = ksplit;
    a.Dpart = Dpart;
    a.part_R = part_R;
  }
  if (b_stream && !kn) return hipErrorInvalidValue;
  if (b_stream) return launch_kn_stream(a, c, epilogue, fp16, grid, stream);
  if (scat) {
    if (!kn) return hipErrorInvalidValue;
    return fp16 ? launch_bn<kEpiScatter, true, true, false>(a, c, grid, stream)
                : launch_bn<kEpiScatter, true, false, false>(a, c, grid, stream);
  }
  if (epilogue == kEpiSiluMul) {
    if (kn) return fp16 ? launch_bn<kEpiSiluMul, true, true, false>(a, c, grid, stream)
                        : launch_bn<kEpiSiluMul, true, false, false>(a, c, grid, stream);
    return fp16 ? launch_bn<kEpiSiluMul, false, true, false>(a, c, grid, stream)
                : launch_bn<kEpiSiluMul, false, false, false>(a, c, grid, stream);
  }
  if (kn) return fp16 ? launch_bn<kEpiStore, true, true, false>(a, c, grid, stream)
                      : launch_bn<kEpiStore, true, false, false>(a, c, grid, stream);
  return fp16 ? launch_bn<kEpiStore, false, true, false>(a, c, grid, stream)
              : launch_bn<kEpiStore, false, false, false>(a, c, grid, stream);
}

// The fused gate/up GEMM (the reorder by route in its prologue): whether
// this shape can take it.  The routing of R pairs to E experts is staged in
// LDS (R <= kLpMaxPairs, E <= 256), the default SiLU*up tile must have a
// fused instantiation, and no workgroup may get more than kTabSlots tasks:
// with row tasks nrt = sum_e ceil(count_e / 256) <= R / 256 + min(E, R),
// the task count is bounded before the routing is known.
bool gg_fused_fits(int N, int K, int R, int E, int grid) {
  if (E < 1 || E > kLpMaxExperts || R < 1 || R > kLpMaxPairs || N % 128 != 0 || grid < 1)
    return false;
  const TileCfg c = tile_config(kEpiSiluMul, N, K);
  if (!lp_tile(c)) return false;
  const long nrt_max = R / 256 + (E < R ? E : R);
  const long ntask = nrt_max * (N / c.bn);
  const int nx = grid % 8 == 0 ? 8 : 1;
  const long S = grid / nx;
  const long range = (ntask + nx - 1) / nx;
  return (range + S - 1) / S <= kTabSlots;
}

// The fused gate/up GEMM: h = SiLU(x.Wg) * (x.Wu) over the permutation of
// route_idx, which the kernel computes itself and writes out (counts,
// offsets, pair_to_row, row_to_pair, block_expert, M_pad and the row-task
// plan, as the permutation kernel would).  Gate and up weights interleaved
// (il) or separate; x rows gathered as row_to_pair / k.
hipError_t launch_gate_up_fused(const uint16_t *x, const int32_t *route_idx, int T, int k, int E,
                                int cap, const uint16_t *B, const uint16_t *B2, bool il, int N,
                                int K, uint16_t *h, int32_t *counts, int32_t *offsets,
                                int32_t *p2r, int32_t *r2p, int32_t *bexp, int32_t *mpad,
                                int32_t *plan, int grid, bool b_stream, hipStream_t stream) {
  const int R = T * k;
  if (!gg_fused_fits(N, K, R, E, grid)) return hipErrorInvalidValue;
  const TileCfg c = tile_config(kEpiSiluMul, N, K);
  GGArgs a{x, nullptr, k, B, il ? B : B2, nullptr, h, nullptr, nullptr, nullptr, 0, N, K, c.group,
           il ? 2 * N : N, il ? 1 : 0};
  a.route_idx = route_idx;
  a.lp_R = R;
  a.lp_E = E;
  a.lp_cap = cap;
  a.o_counts = counts;
  a.o_offsets = offsets;
  a.o_p2r = p2r;
  a.o_r2p = r2p;
  a.o_bexp = bexp;
  a.o_mpad = mpad;
  a.o_plan = plan;
  return b_stream ? launch_lp<true>(a, c, grid, stream) : launch_lp<false>(a, c, grid, stream);
}

} // namespace moe
