// api.hip -- the C ABI (include/moe.h): argument validation, workspace
// carving and kernel launches.  Validation happens before any HIP call, so
// every error path can be exercised without a GPU.
#include <mutex>

#include "../../include/moe.h"
#include "common.h"

namespace moe {
hipError_t launch_route(const float *, int, int, int, int32_t *, float *, hipStream_t);
bool router_fits(int H, int E);
size_t router_workspace_bytes(int T, int H, int E);
hipError_t launch_router(const uint16_t *, const uint16_t *, int, int, int, int, float *,
                         int32_t *, float *, int32_t *, void *, hipStream_t);
hipError_t launch_pack_gate_up(const uint16_t *, const uint16_t *, int, int, int, uint16_t *,
                               hipStream_t);
bool permute_plan_fits(int T, int E, int k);
hipError_t launch_permute_plan(const int32_t *, int, int, int, int, int32_t *, int32_t *,
                               int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, hipStream_t,
                               const int32_t *);
size_t permute_workspace_bytes(long R, int E);
hipError_t launch_permute(const int32_t *, int, int, int, const uint16_t *, int, int32_t *,
                          int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, uint16_t *, int,
                          void *, hipStream_t);
hipError_t launch_grouped_gemm(int, int, int, const uint16_t *, const int32_t *, int,
                               const uint16_t *, const uint16_t *, int, const int32_t *, int,
                               const int32_t *, const float *, int, void *, int, bool,
                               hipStream_t, const int32_t *tile = nullptr, int ksplit = 1,
                               float *Dpart = nullptr, int part_R = 0);
hipError_t launch_splitk_silu(const float *, const int32_t *, int, int, int, int, int,
                              const int32_t *, uint16_t *, hipStream_t);
hipError_t launch_splitk_combine(const float *, const uint16_t *, const int32_t *, int, int, int,
                                 int, int, int, const int32_t *, const float *, uint16_t *,
                                 hipStream_t);
bool gg_tile_usable(const int32_t *tile, int epilogue, int N, int K);
hipError_t launch_gg_plan(const int32_t *, const int32_t *, int, int32_t *, hipStream_t);
bool gg_fused_fits(int N, int K, int R, int E, int grid);
hipError_t launch_gate_up_fused(const uint16_t *, const int32_t *, int, int, int, int,
                                const uint16_t *, const uint16_t *, bool, int, int, uint16_t *,
                                int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                                int32_t *, int, bool, hipStream_t);
size_t gg_plan_bytes(int cap);
hipError_t launch_combine(const uint16_t *, int, const int32_t *, const float *, int, int,
                          uint16_t *, hipStream_t);
hipError_t launch_finalize(const float *, long, uint16_t *, hipStream_t);
hipError_t launch_zero(float *, long, hipStream_t);
} // namespace moe

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256; // sizing when no device is visible (MI355X)
// flags a layer's combine argument may carry
constexpr int kLayerFlags = MOE_LAYER_SEPARATE_PERMUTE | MOE_LAYER_SPLIT_K;
std::mutex g_mu;
int g_cus[kMaxDevices]; // 0 = not queried yet

// Compute-unit count of the current device; 0 if there is no usable device.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_cus[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    g_cus[dev] = prop.multiProcessorCount;
  }
  return g_cus[dev];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// The row-task plan of grouped_gemm_noalloc lives here instead of in a
// caller workspace: one copy per GPU, held until the process ends, shared by
// every call on that GPU.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the device address looked up below.
__device__ __align__(256) int32_t scratch[2 + 2 * (MOE_NOALLOC_MAX_CAP / MOE_ROW_BLOCK)];
int32_t *g_scratch[kMaxDevices]; // device address of `scratch`, per device

// Device address of this device's `scratch`, looked up once per device with
// that device current; NULL if the lookup fails.
int32_t *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = (int32_t *)p;
  }
  return g_scratch[dev];
}

int check_route(const float *logits, int T, int E, int k, const int32_t *idx, const float *w) {
  if (!logits || !idx || !w) return MOE_ERR_INVALID;
  if (T <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID;
  if (E > 1024 || k > 16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

long padded_cap(long T, long k, long E) {
  const long R = T * k;
  const long cap = R + (E < R ? E : R) * (MOE_ROW_BLOCK - 1);
  return (cap + MOE_ROW_BLOCK - 1) / MOE_ROW_BLOCK * MOE_ROW_BLOCK;
}

} // namespace

extern "C" {

const char *moe_status_string(int s) {
  switch (s) {
  case MOE_OK: return "ok";
  case MOE_ERR_INVALID: return "invalid argument";
  case MOE_ERR_UNSUPPORTED: return "unsupported size or combination";
  case MOE_ERR_WORKSPACE: return "workspace or capacity too small";
  case MOE_ERR_DEVICE: return "device error";
  default: return "unknown status";
  }
}

const char *moe_version(void) { return "moe-grouped-gfx950 0.1"; }

int moe_padded_capacity(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return -1;
  const long cap = padded_cap(T, k, E);
  return cap > 0x7fffffffL ? -1 : (int)cap;
}

int moe_route(const float *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w,
              void *stream) {
  int st = check_route(logits, T, E, k, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(
      moe::launch_route(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream));
}

size_t moe_router_workspace_size(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0 || !moe::router_fits(H, E)) return 0;
  return align256(moe::router_workspace_bytes(T, H, E));
}

int moe_router(const void *x, const void *w_router, int T, int H, int E, int k, float *logits,
               int32_t *topk_idx, float *topk_w, int32_t *expert_counts, void *workspace,
               size_t ws_bytes, void *stream) {
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID;
  if (T <= 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID;
  if (!moe::router_fits(H, E) || k > 16) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::router_workspace_bytes(T, H, E);
  if (need && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return MOE_ERR_INVALID;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(moe::launch_router((const uint16_t *)x, (const uint16_t *)w_router, T, H,
                                          E, k, logits, topk_idx, topk_w, expert_counts,
                                          workspace, (hipStream_t)stream));
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  return align256(moe::permute_workspace_bytes((long)T * k, E));
}

int moe_permute(const int32_t *topk_idx, int T, int k, int E, const void *x, int H,
                int32_t *counts, int32_t *offsets, int32_t *pair_to_row, int32_t *row_to_pair,
                int32_t *block_expert, int32_t *num_padded_rows, void *x_perm, int cap,
                void *workspace, size_t ws_bytes, void *stream) {
  if (!topk_idx || !counts || !offsets || !pair_to_row || !row_to_pair || !block_expert ||
      !num_padded_rows || !workspace)
    return MOE_ERR_INVALID;
  if (T <= 0 || k <= 0 || E <= 0 || cap <= 0) return MOE_ERR_INVALID;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID;
  if (x && (H <= 0 || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  if (x && H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long)T * k > 0x7fffffffL) return MOE_ERR_UNSUPPORTED;
  if (cap % MOE_ROW_BLOCK != 0) return MOE_ERR_INVALID;
  if (cap < padded_cap(T, k, E)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < moe_permute_workspace_size(T, k, E)) return MOE_ERR_WORKSPACE;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(moe::launch_permute(
      topk_idx, T, k, E, (const uint16_t *)x, H, counts, offsets, pair_to_row, row_to_pair,
      block_expert, num_padded_rows, (uint16_t *)x_perm, cap, workspace, (hipStream_t)stream));
}

size_t grouped_gemm_workspace_size(int cap) {
  if (cap <= 0) return 0;
  return align256(moe::gg_plan_bytes(cap));
}

} // extern "C"

namespace {

// Argument checks of every grouped GEMM entry point (the workspace aside).
// Splits the MOE_B_STREAM flag off b_layout.
int check_gemm(int dtype, int N, int K, int cap, const void *A, const int32_t *a_src_row,
               int a_src_div, const void *B, const void *B2, int &b_layout, bool &b_stream,
               const int32_t *block_group, const int32_t *num_rows, int epilogue,
               const int32_t *epi_row_pair, const float *pair_w, int k, const void *D) {
  if (!A || !B || !block_group || !num_rows || !D) return MOE_ERR_INVALID;
  if (!aligned16(A) || !aligned16(B) || !aligned16(D) || (B2 && !aligned16(B2)))
    return MOE_ERR_INVALID;
  if (N <= 0 || K <= 0 || cap <= 0) return MOE_ERR_INVALID;
  if (dtype != MOE_BF16 && dtype != MOE_FP16) return MOE_ERR_UNSUPPORTED;
  b_stream = (b_layout & MOE_B_STREAM) != 0;
  b_layout &= ~MOE_B_STREAM;
  if (b_layout != MOE_B_KN && b_layout != MOE_B_NK && b_layout != MOE_B_KN_GATE_UP)
    return MOE_ERR_UNSUPPORTED;
  if (b_stream && b_layout == MOE_B_NK) return MOE_ERR_UNSUPPORTED;
  if (epilogue != MOE_EPI_STORE && epilogue != MOE_EPI_SILU_MUL &&
      epilogue != MOE_EPI_WEIGHTED_SCATTER)
    return MOE_ERR_UNSUPPORTED;
  if (b_layout == MOE_B_KN_GATE_UP) {
    // gate and up interleaved in B: the SiLU*up epilogue only, no B2
    if (epilogue != MOE_EPI_SILU_MUL || B2) return MOE_ERR_INVALID;
    if (N % 128 != 0) return MOE_ERR_UNSUPPORTED;
  } else if (epilogue == MOE_EPI_SILU_MUL && !B2) {
    return MOE_ERR_INVALID;
  }
  if (epilogue == MOE_EPI_WEIGHTED_SCATTER) {
    if (!epi_row_pair || !pair_w || k <= 0) return MOE_ERR_INVALID;
    if (b_layout != MOE_B_KN) return MOE_ERR_UNSUPPORTED;
  }
  if (a_src_row && a_src_div <= 0) return MOE_ERR_INVALID;
  if (N % 64 != 0 || K % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (cap % MOE_ROW_BLOCK != 0) return MOE_ERR_INVALID;
  return MOE_OK;
}

// The plan kernel into `plan`, then the GEMM (arguments checked).
int gemm_enqueue(int dtype, int N, int K, int cap, const void *A, const int32_t *a_src_row,
                 int a_src_div, const void *B, const void *B2, int b_layout, bool b_stream,
                 const int32_t *block_group, const int32_t *num_rows, int epilogue,
                 const int32_t *epi_row_pair, const float *pair_w, int k, void *D, int32_t *plan,
                 const int32_t *tile, int grid, hipStream_t s, bool plan_ready = false) {
  if (!plan_ready && moe::launch_gg_plan(block_group, num_rows, cap, plan, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  return launch_status(moe::launch_grouped_gemm(
      dtype, N, K, (const uint16_t *)A, a_src_row, a_src_div, (const uint16_t *)B,
      (const uint16_t *)B2, b_layout, plan, epilogue, epi_row_pair, pair_w, k, D, grid, b_stream,
      s, tile));
}

} // namespace

extern "C" {

int grouped_gemm(int dtype, int N, int K, int cap, const void *A, const int32_t *a_src_row,
                 int a_src_div, const void *B, const void *B2, int b_layout,
                 const int32_t *block_group, const int32_t *num_rows, int epilogue,
                 const int32_t *epi_row_pair, const float *pair_w, int k, void *D,
                 void *workspace, size_t ws_bytes, void *stream) {
  return grouped_gemm_tuned(dtype, N, K, cap, A, a_src_row, a_src_div, B, B2, b_layout,
                            block_group, num_rows, epilogue, epi_row_pair, pair_w, k, D, nullptr,
                            0, 0, workspace, ws_bytes, stream);
}

int grouped_gemm_tuned(int dtype, int N, int K, int cap, const void *A, const int32_t *a_src_row,
                       int a_src_div, const void *B, const void *B2, int b_layout,
                       const int32_t *block_group, const int32_t *num_rows, int epilogue,
                       const int32_t *epi_row_pair, const float *pair_w, int k, void *D,
                       const int32_t *tile, int grid, int flags, void *workspace,
                       size_t ws_bytes, void *stream) {
  bool b_stream = false;
  int st = check_gemm(dtype, N, K, cap, A, a_src_row, a_src_div, B, B2, b_layout, b_stream,
                      block_group, num_rows, epilogue, epi_row_pair, pair_w, k, D);
  if (st != MOE_OK) return st;
  if (grid < 0 || grid > 65535) return MOE_ERR_INVALID;
  if (flags & ~MOE_TUNED_PLAN_READY) return MOE_ERR_INVALID;
  if (tile) {
    if (!moe::gg_tile_usable(tile, epilogue, N, K)) return MOE_ERR_UNSUPPORTED;
    // the interleaved gate/up layout needs column tiles inside 128-column blocks
    if (b_layout == MOE_B_KN_GATE_UP && (tile[0] > 128 || 128 % tile[0] != 0))
      return MOE_ERR_UNSUPPORTED;
  }
  if (workspace && !aligned16(workspace)) return MOE_ERR_INVALID;
  if (!workspace || ws_bytes < grouped_gemm_workspace_size(cap)) return MOE_ERR_WORKSPACE;
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_DEVICE;
  return gemm_enqueue(dtype, N, K, cap, A, a_src_row, a_src_div, B, B2, b_layout, b_stream,
                      block_group, num_rows, epilogue, epi_row_pair, pair_w, k, D,
                      (int32_t *)workspace, tile, grid > 0 ? grid : cus, (hipStream_t)stream,
                      (flags & MOE_TUNED_PLAN_READY) != 0);
}

int grouped_gemm_noalloc(int dtype, int N, int K, int cap, const void *A,
                         const int32_t *a_src_row, int a_src_div, const void *B, const void *B2,
                         int b_layout, const int32_t *block_group, const int32_t *num_rows,
                         int epilogue, const int32_t *epi_row_pair, const float *pair_w, int k,
                         void *D, void *stream) {
  bool b_stream = false;
  int st = check_gemm(dtype, N, K, cap, A, a_src_row, a_src_div, B, B2, b_layout, b_stream,
                      block_group, num_rows, epilogue, epi_row_pair, pair_w, k, D);
  if (st != MOE_OK) return st;
  if (cap > MOE_NOALLOC_MAX_CAP) return MOE_ERR_WORKSPACE;
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_DEVICE;
  int32_t *plan = scratch_ptr();
  if (!plan) return MOE_ERR_DEVICE;
  // the plan kernel writes every plan entry the GEMM reads: nothing left by
  // an earlier call needs clearing
  return gemm_enqueue(dtype, N, K, cap, A, a_src_row, a_src_div, B, B2, b_layout, b_stream,
                      block_group, num_rows, epilogue, epi_row_pair, pair_w, k, D, plan, nullptr,
                      cus, (hipStream_t)stream);
}

int moe_pack_gate_up(const void *w_gate, const void *w_up, int E, int K, int N, void *out,
                     void *stream) {
  if (!w_gate || !w_up || !out) return MOE_ERR_INVALID;
  if (E <= 0 || K <= 0 || N <= 0) return MOE_ERR_INVALID;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(out)) return MOE_ERR_INVALID;
  if (N % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long)E * K > (1L << 40) / N) return MOE_ERR_UNSUPPORTED;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(moe::launch_pack_gate_up((const uint16_t *)w_gate, (const uint16_t *)w_up, E,
                                                K, N, (uint16_t *)out, (hipStream_t)stream));
}

int moe_combine(const void *y, int H, const int32_t *pair_to_row, const float *topk_w, int T,
                int k, void *out, void *stream) {
  if (!y || !pair_to_row || !topk_w || !out) return MOE_ERR_INVALID;
  if (H <= 0 || T <= 0 || k <= 0) return MOE_ERR_INVALID;
  if (!aligned16(y) || !aligned16(out)) return MOE_ERR_INVALID;
  if (H % 8 != 0 || k > 16) return MOE_ERR_UNSUPPORTED;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(moe::launch_combine((const uint16_t *)y, H, pair_to_row, topk_w, T, k,
                                           (uint16_t *)out, (hipStream_t)stream));
}

int moe_finalize(const float *acc, size_t n, void *out, void *stream) {
  if (!acc || !out || n == 0) return MOE_ERR_INVALID;
  if (!aligned16(acc) || !aligned16(out)) return MOE_ERR_INVALID;
  if (n > ((size_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  if (device_cus() == 0) return MOE_ERR_DEVICE;
  return launch_status(
      moe::launch_finalize(acc, (long)n, (uint16_t *)out, (hipStream_t)stream));
}

int moe_layer_workspace_layout(int T, int H, int E, int k, int I, size_t off[14]) {
  if (!off || T <= 0 || H <= 0 || E <= 0 || k <= 0 || I <= 0 || k > E) return MOE_ERR_INVALID;
  const long R = (long)T * k;
  const long cap = padded_cap(T, k, E);
  size_t o = 0;
  auto take = [&](int i, size_t bytes) {
    off[i] = o;
    o += align256(bytes);
  };
  take(0, R * 4);
  take(1, R * 4);
  take(2, (size_t)E * 4);
  take(3, (size_t)(E + 1) * 4);
  take(4, R * 4);
  take(5, cap * 4);
  take(6, (cap / MOE_ROW_BLOCK) * 4);
  take(7, 4);
  take(8, (size_t)cap * I * 2);
  take(9, (size_t)cap * H * 2);
  take(10, moe::permute_workspace_bytes(R, E));
  take(11, grouped_gemm_workspace_size((int)cap));
  take(12, (size_t)T * H * 4);
  off[13] = o;
  return MOE_OK;
}

size_t moe_layer_workspace_size(int T, int H, int E, int k, int I) {
  size_t off[14];
  if (moe_layer_workspace_layout(T, H, E, k, I, off) != MOE_OK) return 0;
  return off[13];
}

size_t moe_layer_workspace_size_ex(int T, int H, int E, int k, int I, int combine) {
  size_t off[14];
  if (moe_layer_workspace_layout(T, H, E, k, I, off) != MOE_OK) return 0;
  combine &= ~kLayerFlags;
  if (combine == MOE_COMBINE_GATHER) return off[12]; // out_acc, last, is the scatter's only
  return combine == MOE_COMBINE_SCATTER ? off[13] : 0;
}

int moe_layer(const void *x, const float *logits, const int32_t *topk_idx_in,
              const float *topk_w_in, const void *w_gate, const void *w_up, const void *w_down,
              int T, int H, int E, int k, int I, void *out, void *workspace, size_t ws_bytes,
              void *stream) {
  return moe_layer_ex(x, logits, topk_idx_in, topk_w_in, w_gate, w_up, w_down, T, H, E, k, I,
                      out, MOE_COMBINE_GATHER, workspace, ws_bytes, stream);
}

} // extern "C"

namespace {

// Checks of the arguments every layer entry point shares.
int check_layer(const void *x, const void *w_gate, const void *w_up, const void *w_down, int T,
                int H, int E, int k, int I, const void *out, int combine, const void *workspace) {
  // w_up == NULL: w_gate holds gate and up interleaved (moe_pack_gate_up)
  if (!x || !w_gate || !w_down || !out || !workspace) return MOE_ERR_INVALID;
  if (T <= 0 || H <= 0 || E <= 0 || k <= 0 || I <= 0 || k > E) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_gate) || (w_up && !aligned16(w_up)) || !aligned16(w_down) ||
      !aligned16(out) || !aligned16(workspace))
    return MOE_ERR_INVALID;
  if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (!w_up && I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (E > 1024 || k > 16) return MOE_ERR_UNSUPPORTED;
  if ((long)T * k > 0x7fffffffL / 2) return MOE_ERR_UNSUPPORTED;
  if ((combine & ~kLayerFlags) != MOE_COMBINE_GATHER &&
      (combine & ~kLayerFlags) != MOE_COMBINE_SCATTER)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Bytes of the layer workspace before the router's scratch (the layout
// through out_acc for the scatter combine, through y's region otherwise).
size_t layer_core_bytes(const size_t off[14], int combine) {
  return (combine & ~kLayerFlags) == MOE_COMBINE_SCATTER ? off[13] : off[12];
}

// The most k parts a layer GEMM of N columns in BN-column blocks over a k
// range of K may be split into (the GEMM picks the count on the device from
// the routed task count, splitk_parts_for): 1 unless even the most row tasks
// any routing can give (an expert of c rows has ceil(c / 256) of them, so at
// most floor((R + 255 * min(E, R)) / 256) in all) fit one wave ("Comm-compute
// fusion (1)", section 5) -- a larger share keeps the plain form and its
// launches (the split form of gate/up gives up the fused front end and adds
// its reduction's launch, whether or not it then splits); else 4 (2 if K is
// too short), parts of at least 16 slices of 32 -- shorter ones would not
// hide the pipeline's fill behind their weight stream -- and only as many as
// whose fp32 partials, parts x R x NB x N, fit in `room` bytes.
int splitk_parts(long R, int E, int N, int BN, int NB, int K, int cus, size_t room) {
  const long rt = (R + 255L * (E < R ? E : R)) / 256;
  if (N % BN != 0 || rt * (N / BN) > cus) return 1;
  for (int parts = 4; parts >= 2; parts /= 2)
    if (K % (32 * parts) == 0 && K / 32 / parts >= 16 &&
        (size_t)parts * R * NB * N * 4 <= room)
      return parts;
  return 1;
}

// The layer on arguments already checked: the routing from the router front
// end (w_router), from the logits, or given; then permutation, the two
// grouped GEMMs and the combine, all enqueued on `s`.
int layer_run(const void *x, const void *w_router, const float *logits,
              const int32_t *topk_idx_in, const float *topk_w_in, const void *w_gate,
              const void *w_up, const void *w_down, int T, int H, int E, int k, int I, void *out,
              int combine, unsigned char *ws, const size_t off[14], int cus, hipStream_t s) {
  // with MOE_LAYER_SPLIT_K, the split-K form of a GEMM that may have less
  // than one wave of tasks (its fp32 partials in y's region, free until the
  // down GEMM: gate/up's are reduced into h before it, down's replace y);
  // the down GEMM with the gather combine only (its reduction replaces the
  // combine launch)
  const long R = (long)T * k;
  const size_t room = off[10] - off[9];
  const bool split = (combine & MOE_LAYER_SPLIT_K) != 0;
  const int ks_gu = split ? splitk_parts(R, E, I, 128, 2, H, cus, room) : 1;
  const int ks_dn = split && (combine & ~kLayerFlags) == MOE_COMBINE_GATHER
                        ? splitk_parts(R, E, H, 256, 1, I, cus, room)
                        : 1;
  float *part = (float *)(ws + off[9]);
  // the reorder by route inside the gate/up GEMM's prologue (one launch
  // fewer) where the shape allows, unless the caller asks for the separate
  // permutation launch or the gate/up GEMM splits K
  const bool fused = !(combine & MOE_LAYER_SEPARATE_PERMUTE) && ks_gu == 1 &&
                     moe::gg_fused_fits(I, H, T * k, E, cus);
  combine &= ~kLayerFlags;
  int32_t *idx = (int32_t *)(ws + off[0]);
  float *w = (float *)(ws + off[1]);
  int32_t *counts = (int32_t *)(ws + off[2]);
  int32_t *offsets = (int32_t *)(ws + off[3]);
  int32_t *p2r = (int32_t *)(ws + off[4]);
  int32_t *r2p = (int32_t *)(ws + off[5]);
  int32_t *bexp = (int32_t *)(ws + off[6]);
  int32_t *mpad = (int32_t *)(ws + off[7]);
  uint16_t *h = (uint16_t *)(ws + off[8]);
  uint16_t *y = (uint16_t *)(ws + off[9]);
  void *pws = ws + off[10];
  int32_t *plan = (int32_t *)(ws + off[11]);
  float *oacc = (float *)(ws + off[12]);
  const int cap = (int)padded_cap(T, k, E);

  const int32_t *ridx = topk_idx_in;
  const float *rw = topk_w_in;
  const int32_t *counted = nullptr; // expert counts from the router front end
  hipError_t e;
  if (w_router) {
    // logits, top-k, softmax and (for a separate permutation) the expert
    // histogram it starts from
    e = moe::launch_router((const uint16_t *)x, (const uint16_t *)w_router, T, H, E, k, nullptr,
                           idx, w, fused ? nullptr : counts, ws + layer_core_bytes(off, combine),
                           s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    ridx = idx;
    rw = w;
    counted = fused ? nullptr : counts;
  } else if (logits) {
    e = moe::launch_route(logits, T, E, k, idx, w, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    ridx = idx;
    rw = w;
  }
  // weights streamed (non-temporal loads) when the experts average at most
  // two 128-row blocks: each weight tile is then read by about one row task
  const bool stream_w = (long)T * k <= 2L * MOE_ROW_BLOCK * E;
  if (fused) {
    // the gate/up GEMM computes the permutation from the routing and writes
    // it out (counts, offsets, row maps, block experts, M_pad, plan)
    e = moe::launch_gate_up_fused((const uint16_t *)x, ridx, T, k, E, cap,
                                  (const uint16_t *)w_gate, (const uint16_t *)w_up, !w_up, I, H,
                                  h, counts, offsets, p2r, r2p, bexp, mpad, plan, cus, stream_w,
                                  s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  } else if (moe::permute_plan_fits(T, E, k)) {
    // permutation and the row-task plan in one launch
    e = moe::launch_permute_plan(ridx, T, E, k, cap, counts, offsets, p2r, r2p, bexp, mpad, plan,
                                 s, counted);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  } else {
    e = moe::launch_permute(ridx, T, k, E, nullptr, 0, counts, offsets, p2r, r2p, bexp, mpad,
                            nullptr, cap, pws, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    // one row-task plan serves both GEMMs (they share the block experts)
    e = moe::launch_gg_plan(bexp, mpad, cap, plan, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  if (!fused) {
    e = moe::launch_grouped_gemm(MOE_BF16, I, H, (const uint16_t *)x, r2p, k,
                                 (const uint16_t *)w_gate, (const uint16_t *)w_up,
                                 w_up ? MOE_B_KN : MOE_B_KN_GATE_UP, plan,
                                 MOE_EPI_SILU_MUL, nullptr, nullptr, 0, h, cus, stream_w, s,
                                 nullptr, ks_gu, part, (int)R);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    if (ks_gu > 1) {
      e = moe::launch_splitk_silu(part, plan, I / 128, cus, ks_gu, (int)R, I, p2r, h, s);
      if (e != hipSuccess) return MOE_ERR_DEVICE;
    }
  }
  if (combine == MOE_COMBINE_SCATTER) {
    e = moe::launch_zero(oacc, (long)T * H, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    e = moe::launch_grouped_gemm(MOE_BF16, H, I, h, nullptr, 1, (const uint16_t *)w_down,
                                 nullptr, MOE_B_KN, plan, MOE_EPI_WEIGHTED_SCATTER, r2p, rw, k,
                                 oacc, cus, stream_w, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    return launch_status(moe::launch_finalize(oacc, (long)T * H, (uint16_t *)out, s));
  }
  if (ks_dn > 1) {
    e = moe::launch_grouped_gemm(MOE_BF16, H, I, h, nullptr, 1, (const uint16_t *)w_down,
                                 nullptr, MOE_B_KN, plan, MOE_EPI_STORE, r2p, nullptr, 0, y, cus,
                                 stream_w, s, nullptr, ks_dn, part, (int)R);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    return launch_status(
        moe::launch_splitk_combine(part, y, plan, H / 256, cus, ks_dn, T, k, H, p2r, rw,
                                   (uint16_t *)out, s));
  }
  // padding rows of y are never read: the down GEMM skips their stores
  e = moe::launch_grouped_gemm(MOE_BF16, H, I, h, nullptr, 1, (const uint16_t *)w_down, nullptr,
                               MOE_B_KN, plan, MOE_EPI_STORE, r2p, nullptr, 0, y, cus, stream_w,
                               s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  e = moe::launch_combine(y, H, p2r, rw, T, k, (uint16_t *)out, s);
  return launch_status(e);
}

} // namespace

extern "C" {

int moe_layer_ex(const void *x, const float *logits, const int32_t *topk_idx_in,
                 const float *topk_w_in, const void *w_gate, const void *w_up,
                 const void *w_down, int T, int H, int E, int k, int I, void *out, int combine,
                 void *workspace, size_t ws_bytes, void *stream) {
  int st = check_layer(x, w_gate, w_up, w_down, T, H, E, k, I, out, combine, workspace);
  if (st != MOE_OK) return st;
  if (!logits && (!topk_idx_in || !topk_w_in)) return MOE_ERR_INVALID;
  size_t off[14];
  moe_layer_workspace_layout(T, H, E, k, I, off);
  // the fp32 token-row accumulator (last in the layout) only for the scatter
  if (ws_bytes < layer_core_bytes(off, combine)) return MOE_ERR_WORKSPACE;
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_DEVICE;
  return layer_run(x, nullptr, logits, topk_idx_in, topk_w_in, w_gate, w_up, w_down, T, H, E, k,
                   I, out, combine, (unsigned char *)workspace, off, cus, (hipStream_t)stream);
}

size_t moe_layer_router_workspace_size(int T, int H, int E, int k, int I, int combine) {
  size_t off[14];
  if (moe_layer_workspace_layout(T, H, E, k, I, off) != MOE_OK) return 0;
  combine &= ~kLayerFlags;
  if (combine != MOE_COMBINE_GATHER && combine != MOE_COMBINE_SCATTER) return 0;
  if (!moe::router_fits(H, E)) return 0;
  return layer_core_bytes(off, combine) + align256(moe::router_workspace_bytes(T, H, E));
}

int moe_layer_router(const void *x, const void *w_router, const void *w_gate, const void *w_up,
                     const void *w_down, int T, int H, int E, int k, int I, void *out,
                     int combine, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_layer(x, w_gate, w_up, w_down, T, H, E, k, I, out, combine, workspace);
  if (st != MOE_OK) return st;
  if (!w_router) return MOE_ERR_INVALID;
  if (!aligned16(w_router)) return MOE_ERR_INVALID;
  if (!moe::router_fits(H, E)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe_layer_router_workspace_size(T, H, E, k, I, combine)) return MOE_ERR_WORKSPACE;
  size_t off[14];
  moe_layer_workspace_layout(T, H, E, k, I, off);
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_DEVICE;
  return layer_run(x, w_router, nullptr, nullptr, nullptr, w_gate, w_up, w_down, T, H, E, k, I,
                   out, combine, (unsigned char *)workspace, off, cus, (hipStream_t)stream);
}

} // extern "C"
