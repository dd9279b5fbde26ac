/*
 * moe.h -- C ABI of the grouped-GEMM Mixture-of-Experts library for AMD
 * Instinct MI355X (gfx950).
 *
 * One GPU's share of an MoE layer, computed as a grouped GEMM: token rows are
 * bucketed by their routed expert and each bucket is multiplied by that
 * expert's own weights.  The path is
 *
 *   moe_route -> moe_permute -> grouped_gemm (gate/up, SiLU*up epilogue)
 *             -> grouped_gemm (down) -> moe_combine          (= moe_layer)
 *
 * Sources of the operations (the pages this library follows):
 *   [P1] "Comm-compute fusion (3): ThunderKittens multi-GPU programming and a
 *        fusable GEMM template" -- section 4: the grouped GEMM template (rows
 *        grouped by expert, each group times its own weights; 128-row blocks
 *        as task and expert alignment unit; a prologue hook before a row
 *        block is loaded and an epilogue hook after a tile lands).
 *   [P2] "Comm-compute fusion (1): why write communication into the GEMM
 *        kernel" -- section 1: the serial MoE layer, expert GEMM (gate/up)
 *        -> SiLU -> GEMM (down); section 4, four-dataflow table: MoE layer0
 *        = prologue + reorder by route, layer1 = epilogue + top-k weighted
 *        reduction.
 *   [P4] "TIRx and high-performance GEMM (part 2)" -- the dense fp16
 *        D = A * B^T GEMM with fp32 accumulation (steps 7-9, performance
 *        table), which is the one-group degenerate case of grouped_gemm.
 * Routing (top-k + softmax over the k chosen logits), tie-breaks, row order
 * and padding contents are not fixed by the pages; the readings taken are
 * stated at each function.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer, owned by the caller.  The
 *     library never allocates, frees or synchronizes; scratch space comes
 *     from a caller-provided workspace.
 *   - bf16 / fp16 tensors are passed as raw 16-bit storage; every tensor is
 *     dense row-major.  Pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Each call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns at once.  Argument errors are reported before any
 *     HIP call is made; a failed launch returns MOE_ERR_DEVICE.  Faults inside
 *     kernels surface at the caller's next synchronization.
 *   - Calls are reentrant; the only global state is a per-device cache of
 *     the compute-unit count, filled on first use.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define MOE_OK 0
#define MOE_ERR_INVALID 1     /* null pointer, non-positive size, k > E, misaligned pointer */
#define MOE_ERR_UNSUPPORTED 2 /* a size or combination the kernels do not handle */
#define MOE_ERR_WORKSPACE 3   /* workspace or row capacity too small */
#define MOE_ERR_DEVICE 4      /* no usable device, or a launch failed */

/* Element types of GEMM operands. */
#define MOE_BF16 0
#define MOE_FP16 1

/* Layout of the per-group B operand of grouped_gemm. */
#define MOE_B_KN 0 /* B[g] is [K][N], N contiguous (expert weights [E,H,I] / [E,I,H]) */
#define MOE_B_NK 1 /* B[g] is [N][K], K contiguous (the dense D = A * B^T case)      */
/* B[g] is [K][2N] with the gate and up weights of MOE_EPI_SILU_MUL interleaved
 * in 128-column blocks: row k holds, for each block b of 128 output columns,
 * gate columns 128b .. 128b+127 then up columns 128b .. 128b+127
 * (moe_pack_gate_up builds it).  Each k row of a task's weight tile is then
 * one contiguous 512-byte piece instead of two 256-byte ones. */
#define MOE_B_KN_GATE_UP 2
/* Flag OR-ed into a [K][N] layout (MOE_B_KN, MOE_B_KN_GATE_UP): B is loaded
 * with the non-temporal (streaming) cache policy.  For weights each of whose
 * tiles is read by about one row task (the groups average at most two
 * 128-row blocks): the weights then do not push the A rows and the outputs
 * out of the caches.  A hint only: results are bit-identical without it.
 * Not with MOE_B_NK (MOE_ERR_UNSUPPORTED). */
#define MOE_B_STREAM 0x100

/* Epilogues of grouped_gemm. */
#define MOE_EPI_STORE 0    /* D[r][n] = round(acc)                              */
#define MOE_EPI_SILU_MUL 1 /* D[r][n] = round(SiLU(A.B)[r][n] * (A.B2)[r][n])  */
#define MOE_EPI_WEIGHTED_SCATTER 2 /* D[p/k][n] += w[p] * (A.B)[r][n], fp32 D      */

/* How moe_layer_ex returns expert outputs to token order. */
#define MOE_COMBINE_GATHER 0  /* y stored per row, then moe_combine (deterministic) */
#define MOE_COMBINE_SCATTER 1 /* down GEMM scatters w*y into fp32 rows, moe_finalize */
/* Flag OR-ed into the combine of moe_layer_ex / moe_layer_router: run the
 * permutation as its own launch before the gate/up GEMM.  Without it the
 * layer fuses the reorder by route into the gate/up GEMM's prologue
 * ([P2 s.4], MoE layer0 = prologue + reorder by route; [P1 s.4], the gate
 * hook before a row block is loaded) wherever the shape allows: at most
 * 16384 (token, slot) pairs, at most 256 experts, I % 128 == 0, and a
 * bounded number of tasks per workgroup.  Same results either way. */
#define MOE_LAYER_SEPARATE_PERMUTE 0x100
/* Flag OR-ed into the combine of moe_layer_ex / moe_layer_router: split K
 * below one wave ([P2 s.5]: with fewer tasks than compute units the rest
 * stand idle).  A GEMM of the layer that may have at most one wave of (row
 * task, column block) tasks -- at most floor((T*k + 255*min(E, T*k)) / 256)
 * row tasks times its column blocks -- and whose k range holds at least
 * 2 x 512 values is launched in its split-K form (the down GEMM with
 * MOE_COMBINE_GATHER only).  Once the routing has run, it counts the row
 * tasks on the device; where they leave at least a quarter of the compute
 * units idle, it runs each task's k range in 2 or 4 equal parts (the count
 * that gives the busiest workgroup the least work), each part a task of its
 * own writing fp32 partial sums into the y region of the workspace, and a
 * reduction adds the parts in part order and applies the epilogue (after
 * gate/up: SiLU*up into h; after down: the weighted combine itself, y never
 * stored); otherwise it runs unsplit, to the same bits as without the flag.
 * Deterministic (the part count follows from the routing), though a split
 * sum rounds differently from an unsplit one.  The permutation then runs as
 * its own launch, and the SiLU*up reduction is one more.  Measured on
 * MI355X (layer us, without / with): T=16 tokens over 16 Zipf-routed experts
 * (H=4096, I=2048) 137.0 / 85.8, T=32 137.3 / 131.9; the tp_share slicing
 * (E=64, top-4, I=512) at T=16 139.8 / 129.1; where nothing splits (T=128
 * over 16 experts, 192 tasks) 140.2 / 141.2.  For decode-sized batches. */
#define MOE_LAYER_SPLIT_K 0x200

#define MOE_ROW_BLOCK 128 /* rows per task and per-expert alignment unit [P1 s.4] */

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(int status);

/* Library version string. */
const char *moe_version(void);

/* Upper bound on the padded row count M_pad of any routing of T tokens to
 * top-k of E experts: each non-empty expert adds at most 127 padding rows,
 * rounded up to whole 128-row blocks:  ceil128(T*k + min(E, T*k) * 127).
 * Returns -1 for invalid sizes. */
int moe_padded_capacity(int T, int k, int E);

/* ------------------------------------------------------------------------
 * moe_route -- top-k routing of router logits.                    [P2 s.4]
 * For each token t: the k experts with the largest logits[t][:], slot 0 the
 * largest, equal logits ordered by the lower expert id; topk_w[t][j] is the
 * softmax over the k selected logits (fp32: exp(l_j - l_0) / sum_j').
 *   logits   [T][E] fp32 (finite)
 *   topk_idx [T][k] int32 out
 *   topk_w   [T][k] fp32 out
 * Requires 1 <= k <= E, k <= 16, E <= 1024.
 * ---------------------------------------------------------------------- */
int moe_route(const float *logits, int T, int E, int k, int32_t *topk_idx,
              float *topk_w, void *stream);

/* ------------------------------------------------------------------------
 * moe_router -- the router front end: the logits of the linear router,
 * then exactly moe_route on them, and the per-expert count of the chosen
 * (token, slot) pairs that the permutation starts from (one launch; two
 * when the hidden dimension is sliced, the second adding the slices,
 * routing and counting; with expert_counts and an unsliced hidden
 * dimension, a one-workgroup launch clears the counts first).
 *                                                       [P2 s.4, the route]
 * The pages take the logits as given; the step before them is read as the
 * plain linear router without bias:
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h]
 * accumulated in fp32 from the bf16 products: the hidden dimension is cut
 * into 4 S parts (S a power of two fixed by T and H alone), each summed on
 * the matrix cores, then the parts are added in a fixed order -- the same
 * bits on every run and every device.  The selection and weights are those
 * of moe_route taken on these fp32 logits.
 *   x        [T][H] bf16, 16-byte aligned
 *   w_router [E][H] bf16 (one row per expert, the nn.Linear layout), 16-byte
 *            aligned
 *   logits   [T][E] fp32 out, or NULL (not written)
 *   topk_idx [T][k] int32 out;  topk_w [T][k] fp32 out
 *   expert_counts [E] int32 out, or NULL: how many (token, slot) pairs chose
 *            each expert
 * Requires 1 <= k <= E, k <= 16, E <= 128, H % 64 == 0
 * (MOE_ERR_UNSUPPORTED otherwise).  workspace: moe_router_workspace_size
 * bytes, 16-byte aligned (MOE_ERR_WORKSPACE if short; NULL when that size
 * is 0); its contents need no initialization.
 * ---------------------------------------------------------------------- */
int moe_router(const void *x, const void *w_router, int T, int H, int E, int k,
               float *logits, int32_t *topk_idx, float *topk_w,
               int32_t *expert_counts, void *workspace, size_t ws_bytes,
               void *stream);

/* Workspace bytes of moe_router (0: none needed, workspace may be NULL; 0
 * also for unsupported sizes).  Fewer than 8161 tokens cut the hidden
 * dimension into up to 16 slices (S of them: S * T * E floats of partial
 * logits). */
size_t moe_router_workspace_size(int T, int H, int E);

/* ------------------------------------------------------------------------
 * moe_permute -- reorder (token, slot) pairs into expert-contiguous,
 * 128-row-aligned blocks.                              [P1 s.4; P2 s.4, s.5]
 * Pair p = t*k + j routed to expert e = topk_idx[p].  Outputs:
 *   expert_counts  [E]    rows routed to each expert
 *   expert_offsets [E+1]  exclusive prefix sum of counts rounded up to
 *                         multiples of 128 (an empty expert takes 0 rows);
 *                         offsets[E] = M_pad
 *   pair_to_row    [T*k]  row of pair p; within an expert rows follow
 *                         ascending p (a stable counting sort)
 *   row_to_pair    [cap]  inverse map; -1 for padding rows and rows >= M_pad
 *   block_expert   [cap/128] expert of each 128-row block; -1 beyond M_pad
 *   num_padded_rows [1]   M_pad (device int32, read by grouped_gemm)
 *   x_perm         [cap][H] bf16, optional (x and x_perm both non-NULL):
 *                  x_perm[row] = x[row_to_pair[row] / k] for row < M_pad, zeros
 *                  for the padding rows below M_pad; rows at or past M_pad are
 *                  not written.
 * cap must be a multiple of 128 and >= moe_padded_capacity(T, k, E).
 * A pair whose expert id lies outside [0, E) gets no row: pair_to_row[p] =
 * -1, it counts for no expert, and moe_combine adds nothing for it.
 * Workspace: moe_permute_workspace_size(T, k, E) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int T, int k, int E);
int moe_permute(const int32_t *topk_idx, int T, int k, int E, const void *x,
                int H, int32_t *expert_counts, int32_t *expert_offsets,
                int32_t *pair_to_row, int32_t *row_to_pair,
                int32_t *block_expert, int32_t *num_padded_rows, void *x_perm,
                int cap, void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * grouped_gemm -- D[r] = A[a(r)] . B[g(r)] over 128-row blocks.   [P1 s.4]
 * Row r (0 <= r < M_pad, M_pad = *num_rows read on the device and clamped to
 * cap) belongs to group g(r) = block_group[r / 128] (a negative entry skips
 * the block).  Its A row is
 *     a(r) = r                          if a_src_row == NULL
 *     a(r) = a_src_row[r] / a_src_div   otherwise (the gate/up GEMM passes
 *                                       row_to_pair and k: the row gather
 *                                       of the reorder-by-route prologue)
 * Rows with a_src_row[r] < 0 are padding: their outputs are unspecified
 * (they are not written).
 *   dtype      MOE_BF16 or MOE_FP16 (A, B, B2 and D all of this type, except
 *              D of MOE_EPI_WEIGHTED_SCATTER, which is fp32)
 *   A          [*][K]   (rows addressed by a(r))
 *   B, B2      [G][K][N] (MOE_B_KN) or [G][N][K] (MOE_B_NK); B2 only for
 *              MOE_EPI_SILU_MUL (the up weights; B holds the gate weights).
 *              MOE_B_KN_GATE_UP: B is [G][K][2N], gate and up interleaved
 *              (see the define), B2 must be NULL, the epilogue must be
 *              MOE_EPI_SILU_MUL and N % 128 == 0.  Either [K][N] layout may
 *              carry MOE_B_STREAM (non-temporal weight loads).
 *   D          [cap][N] for MOE_EPI_STORE and MOE_EPI_SILU_MUL.
 *   epi_row_pair  optional for MOE_EPI_STORE / MOE_EPI_SILU_MUL: rows r with
 *              epi_row_pair[r] < 0 are padding and are not written (the MoE
 *              down GEMM passes row_to_pair).
 *   epi_row_pair, pair_w, k   MOE_EPI_WEIGHTED_SCATTER (pair_w and k are
 *              ignored otherwise; pass NULL, 0): the top-k weighted reduction of
 *              [P2 s.4] (MoE layer1 row) done by the epilogue.  Row r with
 *              p = epi_row_pair[r] >= 0 adds pair_w[p] * (A.B)[r] into
 *              D[p / k], an fp32 [T][N] buffer the caller has zeroed; rows
 *              with p < 0 add nothing.  The adds are fp32 device-scope
 *              atomics: the k contributions to a token sum in no fixed
 *              order, so results are reproducible only up to fp32 rounding
 *              order.  MOE_B_KN only.  For the MoE down GEMM:
 *              epi_row_pair = row_to_pair, pair_w = topk_w.
 * Accumulation is fp32 (MFMA), over k in ascending 32-deep slices; the
 * store epilogues round to nearest even, so STORE and SILU_MUL results are
 * deterministic.
 * Consecutive blocks of one group are computed as 256-row tasks; the pairing
 * is planned on the device, in the workspace, before the GEMM runs.
 * Requires N % 64 == 0, K % 64 == 0, cap % 128 == 0.
 * workspace: at least grouped_gemm_workspace_size(cap) bytes, 16-byte
 * aligned, contents need not be initialized (MOE_ERR_WORKSPACE otherwise).
 * ---------------------------------------------------------------------- */
size_t grouped_gemm_workspace_size(int cap);

/* ------------------------------------------------------------------------
 * grouped_gemm_noalloc -- grouped_gemm without a workspace, for callers that
 * cannot allocate device memory or pass scratch: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same operation, arguments, limits and results as grouped_gemm; the
 * row-task plan it builds goes to a fixed array the library holds on each
 * GPU it runs on (about 64 KiB, kept until the process ends) instead of a
 * workspace.  It calls no allocating routine.
 *   cap <= MOE_NOALLOC_MAX_CAP rows (MOE_ERR_WORKSPACE otherwise).
 * Every call on one GPU uses that GPU's one array: calls that may overlap
 * on one GPU (different streams, without ordering between them) race and
 * must not be made; calls ordered on one stream are safe.  The array keeps
 * the last call's plan; each call rewrites every entry it reads, so nothing
 * needs clearing between calls.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_MAX_CAP (1 << 20)
int grouped_gemm_noalloc(int dtype, int N, int K, int cap, const void *A,
                         const int32_t *a_src_row, int a_src_div,
                         const void *B, const void *B2, int b_layout,
                         const int32_t *block_group, const int32_t *num_rows,
                         int epilogue, const int32_t *epi_row_pair,
                         const float *pair_w, int k, void *D, void *stream);

/* ------------------------------------------------------------------------
 * moe_pack_gate_up -- the MOE_B_KN_GATE_UP weight layout from separate gate
 * and up weights (a one-time weight transform, like loading a checkpoint
 * into the layout the GEMM streams best; no arithmetic).
 *   w_gate, w_up  [E][K][N] 16-bit (bf16 or fp16; the bits are copied)
 *   out           [E][K][2N]: out[e][k][256 b + c]       = w_gate[e][k][128 b + c],
 *                             out[e][k][256 b + 128 + c] = w_up[e][k][128 b + c]
 *                 for c < 128.
 * Requires N % 128 == 0; all pointers 16-byte aligned device pointers,
 * out not overlapping the inputs.
 * ---------------------------------------------------------------------- */
int moe_pack_gate_up(const void *w_gate, const void *w_up, int E, int K, int N, void *out,
                     void *stream);
int grouped_gemm(int dtype, int N, int K, int cap, const void *A,
                 const int32_t *a_src_row, int a_src_div, const void *B,
                 const void *B2, int b_layout, const int32_t *block_group,
                 const int32_t *num_rows, int epilogue,
                 const int32_t *epi_row_pair, const float *pair_w, int k,
                 void *D, void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * grouped_gemm_tuned -- grouped_gemm with the launch shape named by the
 * caller, for tests and tuning sweeps (the product entry points always take
 * the library's own choice).                                      [P1 s.4]
 * The same operation, arguments and results as grouped_gemm, plus:
 *   tile  NULL (the default configuration) or int32[6] =
 *         {columns per task (per B matrix), k per slice, A ring depth,
 *          B ring depth, row tasks per super-block of the task order,
 *          wavefronts per workgroup}; only instantiated configurations run
 *         (MOE_ERR_UNSUPPORTED otherwise, never a silent fallback).
 *   grid  persistent workgroups, 0 = one per compute unit (the product
 *         choice); a smaller grid gives each workgroup more tasks, which
 *         the result does not depend on.  0 <= grid <= 65535.
 *   flags MOE_TUNED_PLAN_READY: the workspace already holds the row-task
 *         plan of this block_group and num_rows, built by an earlier
 *         grouped_gemm call ordered before this one (the plan depends on
 *         nothing else); only the GEMM kernel is launched, so it can be
 *         timed alone.  0 otherwise.
 * ---------------------------------------------------------------------- */
#define MOE_TUNED_PLAN_READY 1
int grouped_gemm_tuned(int dtype, int N, int K, int cap, const void *A,
                       const int32_t *a_src_row, int a_src_div, const void *B,
                       const void *B2, int b_layout, const int32_t *block_group,
                       const int32_t *num_rows, int epilogue,
                       const int32_t *epi_row_pair, const float *pair_w, int k,
                       void *D, const int32_t *tile, int grid, int flags,
                       void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_combine -- top-k weighted reduction back to token order.    [P2 s.4]
 *   out[t][n] = round_bf16( sum_{j<k} topk_w[t][j] * y[pair_to_row[t*k+j]][n] )
 * accumulated in fp32 in slot order.
 *   y [*][H] bf16 (expert outputs in permuted row order), out [T][H] bf16.
 * Requires H % 8 == 0.
 * ---------------------------------------------------------------------- */
int moe_combine(const void *y, int H, const int32_t *pair_to_row,
                const float *topk_w, int T, int k, void *out, void *stream);

/* ------------------------------------------------------------------------
 * moe_finalize -- last step of the weighted-scatter combine:      [P2 s.4]
 *   out[i] = round_bf16(acc[i]) for 0 <= i < n.
 *   acc [n] fp32 (the D of grouped_gemm MOE_EPI_WEIGHTED_SCATTER),
 *   out [n] bf16.  Requires n >= 1.
 * ---------------------------------------------------------------------- */
int moe_finalize(const float *acc, size_t n, void *out, void *stream);

/* ------------------------------------------------------------------------
 * moe_layer -- the whole share:                               [P2 s.1, s.4]
 *   out[t] = sum_j w[t][j] * ( SiLU(x[t] . Wg[e]) * (x[t] . Wu[e]) ) . Wd[e],
 *   e = topk_idx[t][j].
 * If logits != NULL the routing is computed by moe_route; otherwise
 * topk_idx_in / topk_w_in give it.
 *   x [T][H] bf16; w_gate, w_up [E][H][I] bf16; w_down [E][I][H] bf16;
 *   out [T][H] bf16.
 *   w_up == NULL: w_gate is the packed [E][H][2I] tensor of
 *   moe_pack_gate_up (MOE_B_KN_GATE_UP; requires I % 128 == 0), which the
 *   gate/up GEMM streams as contiguous 512-byte row pieces.
 * When T * k <= 256 * E (the experts average at most two 128-row blocks,
 * so each weight tile is read by about one row task) both GEMMs load the
 * weights with MOE_B_STREAM.
 * Intermediates: h = SiLU(gate)*up stored as bf16 [M_pad][I], expert outputs
 * y stored as bf16 [M_pad][H]; both live in the workspace.  The combine is
 * MOE_COMBINE_GATHER (deterministic: same input, same bits).
 * Requires H % 64 == 0, I % 64 == 0, plus the limits of the steps.
 * Workspace: moe_layer_workspace_size_ex(T, H, E, k, I, MOE_COMBINE_GATHER)
 * bytes (or more), 256-byte aligned.
 * ---------------------------------------------------------------------- */
size_t moe_layer_workspace_size(int T, int H, int E, int k, int I);

/* Byte offsets of the intermediates inside the moe_layer workspace, for
 * inspection by callers and tests.  off[] receives, in order:
 *   0 topk_idx [T*k] int32      1 topk_w [T*k] fp32
 *   2 expert_counts [E] int32   3 expert_offsets [E+1] int32
 *   4 pair_to_row [T*k] int32   5 row_to_pair [cap] int32
 *   6 block_expert [cap/128]    7 num_padded_rows [1] int32
 *   8 h [cap][I] bf16           9 y [cap][H] bf16
 *  10 permute scratch          11 grouped-GEMM row-task plan
 *  12 out_acc [T][H] fp32 (MOE_COMBINE_SCATTER only; it comes last, so
 *     the gather combine needs only off[12] bytes)
 *  13 total size
 * Returns MOE_OK or MOE_ERR_INVALID. */
int moe_layer_workspace_layout(int T, int H, int E, int k, int I,
                               size_t off[14]);

/* Workspace bytes of moe_layer_ex with the given combine (the
 * MOE_LAYER_SEPARATE_PERMUTE flag changes nothing here): off[12] of the
 * layout for MOE_COMBINE_GATHER (no out_acc), off[13] for
 * MOE_COMBINE_SCATTER; 0 for invalid sizes or an unknown combine.
 * moe_layer_workspace_size is the larger of the two. */
size_t moe_layer_workspace_size_ex(int T, int H, int E, int k, int I,
                                   int combine);

int moe_layer(const void *x, const float *logits, const int32_t *topk_idx_in,
              const float *topk_w_in, const void *w_gate, const void *w_up,
              const void *w_down, int T, int H, int E, int k, int I, void *out,
              void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_layer_router -- the whole share starting from the token rows and the
 * router weights:                                      [P2 s.1, s.4; P1 s.4]
 *   moe_router (logits, top-k, softmax and expert counts)
 *   -> moe_permute (taking the router's counts) -> the two grouped GEMMs
 *   -> the combine chosen by `combine` (MOE_COMBINE_GATHER / _SCATTER).
 *   w_router [E][H] bf16; the other arguments and results as moe_layer_ex.
 * Requires the limits of moe_router (E <= 128) and of moe_layer.
 * Workspace: moe_layer_router_workspace_size bytes, 256-byte aligned: the
 * moe_layer_workspace_layout regions, then the router's scratch.
 * ---------------------------------------------------------------------- */
size_t moe_layer_router_workspace_size(int T, int H, int E, int k, int I,
                                       int combine);
int moe_layer_router(const void *x, const void *w_router, const void *w_gate,
                     const void *w_up, const void *w_down, int T, int H, int E,
                     int k, int I, void *out, int combine, void *workspace,
                     size_t ws_bytes, void *stream);

/* moe_layer with a choice of combine ([P2 s.4], MoE layer1 row: the top-k
 * weighted reduction either after the down GEMM or inside its epilogue):
 *   MOE_COMBINE_GATHER   exactly moe_layer;
 *   MOE_COMBINE_SCATTER  the down GEMM adds w * y into out_acc (fp32, zeroed
 *                        by the call) with MOE_EPI_WEIGHTED_SCATTER, then
 *                        moe_finalize rounds it into out; y is never stored.
 *                        Sums of a token's k slots are in no fixed order.
 * Workspace: moe_layer_workspace_size_ex(T, H, E, k, I, combine) bytes.
 * Same arguments and limits as moe_layer otherwise. */
int moe_layer_ex(const void *x, const float *logits,
                 const int32_t *topk_idx_in, const float *topk_w_in,
                 const void *w_gate, const void *w_up, const void *w_down,
                 int T, int H, int E, int k, int I, void *out, int combine,
                 void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
