// grouped_gemm.hip -- host side of the grouped GEMM: tile-shape choice and
// dispatch to the per-(epilogue, B layout, dtype) instantiations of the
// kernel templates in gg_kernel.h (compiled from gg_inst.hip, one object per
// combination, so they build in parallel).
#include "gg_kernel.h"

namespace moe {

#define MOE_GG_EXTERN(EPI, KN, FP16)                                                          \
  extern template hipError_t launch_bn<EPI, KN, FP16>(const GGArgs &, const TileCfg &, int,   \
                                                       hipStream_t);
MOE_GG_EXTERN(kEpiStore, true, false)
MOE_GG_EXTERN(kEpiStore, true, true)
MOE_GG_EXTERN(kEpiStore, false, false)
MOE_GG_EXTERN(kEpiStore, false, true)
MOE_GG_EXTERN(kEpiSiluMul, true, false)
MOE_GG_EXTERN(kEpiSiluMul, true, true)
MOE_GG_EXTERN(kEpiSiluMul, false, false)
MOE_GG_EXTERN(kEpiSiluMul, false, true)
MOE_GG_EXTERN(kEpiScatter, true, false)
MOE_GG_EXTERN(kEpiScatter, true, true)
#undef MOE_GG_EXTERN

// Tile configurations.  Defaults (measured on the MI355X at the shapes of
// the MoE layer share): gate/up 128 gate + 128 up columns with a 3-deep
// ring, down / dense 256 columns with a 3-deep ring; the split tail is off
// (its fp32 partial-tile round trip cost more than the balance it bought).
// Each can be overridden for tuning sweeps with
// MOE_GG_TILE="<bn>,<stages>,<group rows>[,<split>[,<waves>]]" (e.g. "128,3,4,1").
static TileCfg tile_config(int epilogue, int N) {
  TileCfg c = epilogue == kEpiSiluMul
                  ? TileCfg{N % 128 == 0 ? 128 : 64, N % 128 == 0 ? 3 : 4, 1, 0, 4}
                  : TileCfg{N % 256 == 0 ? 256 : (N % 128 == 0 ? 128 : 64), N % 256 == 0 ? 3 : 4,
                            1, 0, 4};
  if (const char *env = getenv("MOE_GG_TILE")) {
    TileCfg e{0, 0, 0, 0, 4};
    const int n =
        sscanf(env, "%d,%d,%d,%d,%d", &e.bn, &e.stages, &e.group, &e.split, &e.waves);
    if (n >= 3 && e.group >= 1 && N % e.bn == 0 && (e.waves == 4 || e.waves == 8) &&
        tile_supported(epilogue == kEpiSiluMul ? 2 : 1, e.bn, e.stages))
      c = e;
  }
  return c;
}

// Workspace for the split tail: two fp32 partial tiles per workgroup of the
// largest tile shape (128 accumulator floats per thread).
size_t gg_workspace_bytes(int grid) { return (size_t)grid * 2 * 128 * 256 * sizeof(float); }

// dtype 0 bf16 / 1 fp16; layout 0 KN / 1 NK; epilogue 0 STORE / 1 SILU_MUL /
// 2 WEIGHTED_SCATTER (KN only; D is then the fp32 token-row accumulator).
hipError_t launch_grouped_gemm(int dtype, int N, int K, int cap, const uint16_t *A,
                               const int32_t *a_src_row, int a_src_div, const uint16_t *B,
                               const uint16_t *B2, int layout, const int32_t *block_group,
                               const int32_t *num_rows, int epilogue, const int32_t *epi_row_pair,
                               const float *pair_w, int topk, void *D, void *ws,
                               size_t ws_bytes, int num_cus, hipStream_t stream) {
  const TileCfg c = tile_config(epilogue, N);
  const int grid = num_cus; // one workgroup per CU (LDS-limited)
  float *partials = (c.split && ws && ws_bytes >= gg_workspace_bytes(grid)) ? (float *)ws : nullptr;
  const bool scat = epilogue == kEpiScatter;
  GGArgs a{A, a_src_row, a_src_div, B, B2, block_group, num_rows,
           scat ? nullptr : (uint16_t *)D, N, K, cap, c.group, partials,
           scat ? (float *)D : nullptr, epi_row_pair, pair_w, topk};
  const bool fp16 = dtype == 1;
  const bool kn = layout == 0;
  if (scat) {
    if (!kn) return hipErrorInvalidValue;
    return fp16 ? launch_bn<kEpiScatter, true, true>(a, c, grid, stream)
                : launch_bn<kEpiScatter, true, false>(a, c, grid, stream);
  }
  if (epilogue == kEpiSiluMul) {
    if (kn) return fp16 ? launch_bn<kEpiSiluMul, true, true>(a, c, grid, stream)
                        : launch_bn<kEpiSiluMul, true, false>(a, c, grid, stream);
    return fp16 ? launch_bn<kEpiSiluMul, false, true>(a, c, grid, stream)
                : launch_bn<kEpiSiluMul, false, false>(a, c, grid, stream);
  }
  if (kn) return fp16 ? launch_bn<kEpiStore, true, true>(a, c, grid, stream)
                      : launch_bn<kEpiStore, true, false>(a, c, grid, stream);
  return fp16 ? launch_bn<kEpiStore, false, true>(a, c, grid, stream)
              : launch_bn<kEpiStore, false, false>(a, c, grid, stream);
}

} // namespace moe
