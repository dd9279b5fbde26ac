// gg_inst.hip -- one instantiation of the grouped GEMM launch for the
// (epilogue, B layout, dtype, B cache policy) combination chosen at compile
// time with -DGG_EPI=<0|1|2> -DGG_KN=<0|1> -DGG_FP16=<0|1> -DGG_NT=<0|1>, or
// with -DGG_LP=1 the fused gate/up form for one B cache policy; the build
// compiles this file once per combination the dispatcher in
// grouped_gemm.hip names.
#include "gg_kernel.h"

#ifndef GG_EPI
#define GG_EPI 0
#endif
#ifndef GG_KN
#define GG_KN 1
#endif
#ifndef GG_FP16
#define GG_FP16 0
#endif
#ifndef GG_NT
#define GG_NT 0
#endif

#ifndef GG_LP
#define GG_LP 0
#endif

namespace moe {
#if GG_LP
// the fused gate/up form (the permutation computed inside the kernel)
template hipError_t launch_lp<(GG_NT != 0)>(const GGArgs &, const TileCfg &, int, hipStream_t);
#else
template hipError_t launch_bn<GG_EPI, (GG_KN != 0), (GG_FP16 != 0), (GG_NT != 0)>(
    const GGArgs &, const TileCfg &, int, hipStream_t);
#endif
} // namespace moe
