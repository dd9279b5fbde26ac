"""Grouped-GEMM Mixture-of-Experts layer for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI declared in ``include/moe.h``: every
function here only checks and marshals arguments (torch tensors on the GPU,
the current HIP stream) and calls the library; every step of the path runs in
the HIP kernels of ``libmoe_gfx950.so``.  There is no CPU fallback: if the
library is not built, or no GPU is present, calls raise.

    idx, w = route(logits, k)
    perm   = permute(idx, E)                       # counts, offsets, row maps
    h      = grouped_gemm(x, wg, perm.block_expert, perm.num_padded_rows, N=I, K=H,
                          cap=perm.cap, a_src_row=perm.row_to_pair, a_src_div=k,
                          B2=wu, epilogue="silu_mul")
    y      = grouped_gemm(h, wd, perm.block_expert, perm.num_padded_rows, N=H, K=I, cap=perm.cap)
    out    = combine(y, perm.pair_to_row, w)
    out    = layer(x, wg, wu, wd, k, logits=logits)   # all of the above in one call

The combine can instead be folded into the down GEMM (fp32 atomics into token
rows, then a rounding pass):
    acc    = grouped_gemm(h, wd, ..., epilogue="weighted_scatter",
                          row_pair=perm.row_to_pair, pair_w=w, T=T)
    out    = finalize(acc)
    out    = layer(x, wg, wu, wd, k, logits=logits, combine="scatter")
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")
ROW_BLOCK = 128

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_B_STREAM = 0x100  # flag on a [K][N] b_layout: non-temporal weight loads
MOE_LAYER_SEPARATE_PERMUTE = 0x100  # flag on a layer's combine: the permutation as its own launch
MOE_LAYER_SPLIT_K = 0x200  # flag on a layer's combine: GEMMs below one wave of tasks split K
_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
_LAYOUTS = {"kn": 0, "nk": 1, "kn_gate_up": 2}
_EPIS = {"store": 0, "silu_mul": 1, "weighted_scatter": 2}
_COMBINES = {"gather": 0, "scatter": 1}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                "libmoe_gfx950.so is not built (%s); run `python -m moe_expert_grouped_amd.build` "
                "or __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "moe_status_string": ([I], ctypes.c_char_p),
            "moe_version": ([], ctypes.c_char_p),
            "moe_padded_capacity": ([I, I, I], I),
            "moe_route": ([P, I, I, I, P, P, P], I),
            "moe_router": ([P, P, I, I, I, I, P, P, P, P, P, Z, P], I),
            "moe_router_workspace_size": ([I, I, I], Z),
            "moe_permute_workspace_size": ([I, I, I], Z),
            "moe_permute": ([P, I, I, I, P, I, P, P, P, P, P, P, P, I, P, Z, P], I),
            "grouped_gemm_workspace_size": ([I], Z),
            "grouped_gemm": ([I, I, I, I, P, P, I, P, P, I, P, P, I, P, P, I, P, P, Z, P], I),
            "grouped_gemm_tuned": ([I, I, I, I, P, P, I, P, P, I, P, P, I, P, P, I, P, P, I, I, P, Z,
                                    P], I),
            "grouped_gemm_noalloc": ([I, I, I, I, P, P, I, P, P, I, P, P, I, P, P, I, P, P], I),
            "moe_combine": ([P, I, P, P, I, I, P, P], I),
            "moe_finalize": ([P, Z, P, P], I),
            "moe_pack_gate_up": ([P, P, I, I, I, P, P], I),
            "moe_layer_workspace_size": ([I, I, I, I, I], Z),
            "moe_layer_workspace_size_ex": ([I, I, I, I, I, I], Z),
            "moe_layer_workspace_layout": ([I, I, I, I, I, ctypes.POINTER(Z)], I),
            "moe_layer": ([P, P, P, P, P, P, P, I, I, I, I, I, P, P, Z, P], I),
            "moe_layer_ex": ([P, P, P, P, P, P, P, I, I, I, I, I, P, I, P, Z, P], I),
            "moe_layer_router_workspace_size": ([I, I, I, I, I, I], Z),
            "moe_layer_router": ([P, P, P, P, P, I, I, I, I, I, P, I, P, Z, P], I),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, load_library().moe_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if dims is not None and t.dim() != dims:
        raise ValueError("%s must have %d dims" % (name, dims))


def padded_capacity(T: int, k: int, E: int) -> int:
    return int(load_library().moe_padded_capacity(T, k, E))


# ---------------------------------------------------------------- route

def route(logits: torch.Tensor, k: int):
    """Top-k experts per token (slot 0 the largest logit, ties to the lower id)
    and the softmax over the k chosen logits.  Returns (idx int32, w fp32)."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route", load_library().moe_route(_ptr(logits), T, E, k, _ptr(idx), _ptr(w), _stream()))
    return idx, w


def router(x: torch.Tensor, w_router: torch.Tensor, k: int, with_logits: bool = False,
           workspace: torch.Tensor | None = None, with_counts: bool = False):
    """The linear router and the routing in one launch: logits = x . w_router^T
    (x [T,H] bf16, w_router [E,H] bf16, fp32 accumulation), then the top-k and
    softmax of `route` on those logits, and the per-expert count of the
    chosen pairs.  Returns (idx int32 [T,k], w fp32 [T,k], logits fp32 [T,E]
    or None), plus counts int32 [E] with with_counts=True."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.bfloat16, 2)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H]")
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if with_logits else None
    counts = torch.empty(E, dtype=torch.int32, device=dev) if with_counts else None
    lib = load_library()
    need = lib.moe_router_workspace_size(T, H, E)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("moe_router", lib.moe_router(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(lg), _ptr(idx),
                                        _ptr(w), _ptr(counts), _ptr(workspace), workspace.numel(),
                                        _stream()))
    return (idx, w, lg, counts) if with_counts else (idx, w, lg)


# ---------------------------------------------------------------- permute

@dataclass
class Permutation:
    counts: torch.Tensor          # [E]
    offsets: torch.Tensor         # [E+1]
    pair_to_row: torch.Tensor     # [T*k]
    row_to_pair: torch.Tensor     # [cap]
    block_expert: torch.Tensor    # [cap/128]
    num_padded_rows: torch.Tensor # [1] (device)
    x_perm: torch.Tensor | None   # [cap, H] or None
    cap: int


def permute(topk_idx: torch.Tensor, E: int, x: torch.Tensor | None = None, cap: int | None = None,
            workspace: torch.Tensor | None = None,
            x_perm: torch.Tensor | None = None) -> Permutation:
    """Stable expert-major permutation of the (token, slot) pairs into
    128-row-aligned blocks; optionally gathers x into x_perm [cap][H] (rows
    below M_pad; rows at or past it are not written)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    lib = load_library()
    T, k = topk_idx.shape
    dev = topk_idx.device
    if cap is None:
        cap = padded_capacity(T, k, E)
    i32 = dict(dtype=torch.int32, device=dev)
    counts = torch.empty(E, **i32)
    offsets = torch.empty(E + 1, **i32)
    p2r = torch.empty(T * k, **i32)
    r2p = torch.empty(max(cap, 0), **i32)
    be = torch.empty(max(cap, 0) // ROW_BLOCK, **i32)
    mpad = torch.empty(1, **i32)
    H = 0
    if x is not None:
        _need(x, "x", torch.bfloat16, 2)
        H = x.shape[1]
        if x_perm is None:
            x_perm = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        else:
            _need(x_perm, "x_perm", torch.bfloat16, 2)
            if tuple(x_perm.shape) != (cap, H):
                raise ValueError("x_perm must be [cap, H]")
    else:
        x_perm = None
    need = lib.moe_permute_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("moe_permute", lib.moe_permute(
        _ptr(topk_idx), T, k, E, _ptr(x), H, _ptr(counts), _ptr(offsets), _ptr(p2r), _ptr(r2p),
        _ptr(be), _ptr(mpad), _ptr(x_perm), cap, _ptr(workspace), workspace.numel(), _stream()))
    return Permutation(counts, offsets, p2r, r2p, be, mpad, x_perm, cap)


# ---------------------------------------------------------------- grouped GEMM

def grouped_gemm(A: torch.Tensor, B: torch.Tensor, block_group: torch.Tensor,
                 num_rows: torch.Tensor, *, N: int, K: int, cap: int,
                 a_src_row: torch.Tensor | None = None, a_src_div: int = 1,
                 B2: torch.Tensor | None = None, b_layout: str = "kn", epilogue: str = "store",
                 row_pair: torch.Tensor | None = None, pair_w: torch.Tensor | None = None,
                 T: int | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | str | None = None, b_stream: bool = False,
                 tile: tuple | None = None, grid: int = 0, plan_ready: bool = False) -> torch.Tensor:
    """D[r] = A[a(r)] . B[block_group[r // 128]] for r < min(num_rows, cap),
    or SiLU(A.B) * (A.B2) with epilogue="silu_mul".  Returns D [cap, N].

    b_stream=True loads B with the non-temporal cache policy (MOE_B_STREAM;
    [K][N] layouts only): for weights each tile of which is read by about one
    row task.  The results are the same bits.

    With row_pair given and epilogue "store" or "silu_mul", rows r with
    row_pair[r] < 0 are padding and are not written (nor are rows whose
    a_src_row entry is negative).

    epilogue="weighted_scatter": row r with p = row_pair[r] >= 0 adds
    pair_w[p] * (A.B)[r] into the fp32 row p // k of D [T, N] (k = pair_w's
    second dimension); D is zero-filled here unless `out` is given, in which
    case it is accumulated into.

    `workspace` holds the device-built row-task plan (grouped_gemm_workspace_size(cap)
    bytes; allocated here if not given).

    tile / grid (tests and tuning sweeps; grouped_gemm_tuned): tile is
    (columns per task, k per slice, A ring depth, B ring depth, row tasks per
    super-block, wavefronts) of an instantiated configuration, grid the
    number of persistent workgroups (0: one per compute unit).  The defaults
    are the library's own choice.  plan_ready=True: `workspace` already
    holds the row-task plan of this block_group / num_rows from an earlier
    call on the stream, so only the GEMM kernel runs (to time it alone)."""
    _need(A, "A", (torch.bfloat16, torch.float16))
    _need(B, "B", A.dtype)
    _need(block_group, "block_group", torch.int32)
    _need(num_rows, "num_rows", torch.int32)
    if B2 is not None:
        _need(B2, "B2", A.dtype)
    if a_src_row is not None:
        _need(a_src_row, "a_src_row", torch.int32)
    k = 0
    if row_pair is not None:
        _need(row_pair, "row_pair", torch.int32)
    if epilogue == "weighted_scatter":
        _need(row_pair, "row_pair", torch.int32)
        _need(pair_w, "pair_w", torch.float32, 2)
        k = pair_w.shape[1]
        if T is None:
            T = pair_w.shape[0]
        if out is None:
            out = torch.zeros((T, N), dtype=torch.float32, device=A.device)
        else:
            _need(out, "out", torch.float32)
            if out.numel() < T * N:
                raise ValueError("out must hold [T, N] = [%d, %d] floats" % (T, N))
    elif out is None:
        out = torch.empty((cap, N), dtype=A.dtype, device=A.device)
    else:
        _need(out, "out", A.dtype)
    lib = load_library()
    if workspace is None:
        workspace = gemm_workspace(cap, A.device)
    # workspace="none": grouped_gemm_noalloc, the plan in the library's own
    # per-GPU array (no scratch from the caller)
    args = (_DTYPES[A.dtype], N, K, cap, _ptr(A), _ptr(a_src_row), a_src_div, _ptr(B), _ptr(B2),
            _LAYOUTS[b_layout] | (MOE_B_STREAM if b_stream else 0), _ptr(block_group),
            _ptr(num_rows), _EPIS[epilogue], _ptr(row_pair), _ptr(pair_w), k, _ptr(out))
    if isinstance(workspace, str):
        if workspace != "none" or tile is not None or grid or plan_ready:
            raise ValueError('workspace="none" takes the default launch shape')
        _check("grouped_gemm_noalloc", lib.grouped_gemm_noalloc(*args, _stream()))
        return out
    ws = (_ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    if tile is None and not grid and not plan_ready:
        _check("grouped_gemm", lib.grouped_gemm(*args, *ws))
    else:
        t = None
        if tile is not None:
            if len(tile) != 6:
                raise ValueError("tile must have 6 entries")
            t = (ctypes.c_int32 * 6)(*[int(v) for v in tile])
        _check("grouped_gemm_tuned",
               lib.grouped_gemm_tuned(*args, t, int(grid), 1 if plan_ready else 0, *ws))
    return out


_gemm_ws = {}


def gemm_workspace(cap: int, device="cuda") -> torch.Tensor:
    """A scratch buffer of grouped_gemm_workspace_size(cap) bytes, cached per
    device and grown on demand.  Calls on one stream may share it; calls that
    may overlap on different streams need workspaces of their own."""
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    need = load_library().grouped_gemm_workspace_size(cap)
    ws = _gemm_ws.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _gemm_ws[key] = ws
    return ws


# ---------------------------------------------------------------- combine

def combine(y: torch.Tensor, pair_to_row: torch.Tensor, topk_w: torch.Tensor,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """out[t] = sum_j topk_w[t, j] * y[pair_to_row[t*k + j]] (fp32 sum, bf16 out)."""
    _need(y, "y", torch.bfloat16, 2)
    _need(pair_to_row, "pair_to_row", torch.int32)
    _need(topk_w, "topk_w", torch.float32, 2)
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check("moe_combine", load_library().moe_combine(
        _ptr(y), H, _ptr(pair_to_row), _ptr(topk_w), T, k, _ptr(out), _stream()))
    return out


def pack_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """The interleaved gate/up weight layout (b_layout="kn_gate_up"): [E][K][2N]
    with, per block of 128 output columns, the 128 gate columns then the 128
    up columns.  A copy on the device."""
    _need(w_gate, "w_gate", (torch.bfloat16, torch.float16), 3)
    _need(w_up, "w_up", w_gate.dtype, 3)
    if w_up.shape != w_gate.shape:
        raise ValueError("w_gate and w_up must have the same shape")
    E, K, N = w_gate.shape
    if out is None:
        out = torch.empty((E, K, 2 * N), dtype=w_gate.dtype, device=w_gate.device)
    else:
        _need(out, "out", w_gate.dtype, 3)
        if tuple(out.shape) != (E, K, 2 * N):
            raise ValueError("out must be [E, K, 2N]")
    _check("moe_pack_gate_up", load_library().moe_pack_gate_up(
        _ptr(w_gate), _ptr(w_up), E, K, N, _ptr(out), _stream()))
    return out


def finalize(acc: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out = bf16(acc), round to nearest even (the weighted-scatter combine's last step)."""
    _need(acc, "acc", torch.float32)
    if out is None:
        out = torch.empty(acc.shape, dtype=torch.bfloat16, device=acc.device)
    else:
        _need(out, "out", torch.bfloat16)
        if out.numel() != acc.numel():
            raise ValueError("out must have as many elements as acc")
    _check("moe_finalize", load_library().moe_finalize(_ptr(acc), acc.numel(), _ptr(out), _stream()))
    return out


# ---------------------------------------------------------------- whole layer

LAYOUT_NAMES = ["topk_idx", "topk_w", "expert_counts", "expert_offsets", "pair_to_row",
                "row_to_pair", "block_expert", "num_padded_rows", "h", "y", "permute_scratch",
                "gemm_scratch", "out_acc"]


def layer_workspace_layout(T, H, E, k, I):
    arr = (ctypes.c_size_t * 14)()
    _check("moe_layer_workspace_layout", load_library().moe_layer_workspace_layout(T, H, E, k, I, arr))
    return {name: int(arr[i]) for i, name in enumerate(LAYOUT_NAMES)} | {"total": int(arr[13])}


def layer_workspace(T, H, E, k, I, device="cuda", combine: str = "scatter") -> torch.Tensor:
    """A moe_layer workspace; combine="gather" sizes it for the gather combine
    only (no fp32 token-row accumulator), "scatter" for both."""
    n = load_library().moe_layer_workspace_size_ex(T, H, E, k, I, _COMBINES[combine])
    if n == 0:
        raise ValueError("invalid layer sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def layer(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, k: int,
          logits: torch.Tensor | None = None, topk_idx: torch.Tensor | None = None,
          topk_w: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          out: torch.Tensor | None = None, combine: str = "gather",
          separate_permute: bool = False, split_k: bool = False) -> torch.Tensor:
    """The MoE layer share: route (or the given routing) -> permute -> gate/up
    grouped GEMM with SiLU*up -> down grouped GEMM -> top-k weighted combine.
    w_up=None: w_gate is the interleaved [E][H][2I] tensor of pack_gate_up.
    combine="gather" (deterministic) stores y and runs the combine kernel;
    "scatter" folds the weighted sum into the down GEMM's epilogue.  The
    permutation runs inside the gate/up GEMM's prologue where the shape
    allows; separate_permute=True gives it its own launch (same results).
    split_k=True (MOE_LAYER_SPLIT_K, for decode-sized batches): a GEMM that
    may have at most one wave of tasks takes its split-K form, which splits
    each task's k range on the device where the routed tasks leave at least
    a quarter of the compute units idle (fp32 partial sums, reduced in a
    fixed order), and gives the unsplit bits otherwise."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_gate, "w_gate", torch.bfloat16, 3)
    if w_up is not None:
        _need(w_up, "w_up", torch.bfloat16, 3)
    _need(w_down, "w_down", torch.bfloat16, 3)
    T, H = x.shape
    E, _, I = w_gate.shape
    if w_up is None:  # w_gate is pack_gate_up(gate, up): [E][H][2I]
        I //= 2
    if logits is not None:
        _need(logits, "logits", torch.float32, 2)
    else:
        _need(topk_idx, "topk_idx", torch.int32, 2)
        _need(topk_w, "topk_w", torch.float32, 2)
    if workspace is None:
        workspace = layer_workspace(T, H, E, k, I, x.device, combine)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if combine == "gather" and not separate_permute and not split_k:
        _check("moe_layer", load_library().moe_layer(
            _ptr(x), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(w_gate), _ptr(w_up),
            _ptr(w_down), T, H, E, k, I, _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check("moe_layer_ex", load_library().moe_layer_ex(
            _ptr(x), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(w_gate), _ptr(w_up),
            _ptr(w_down), T, H, E, k, I, _ptr(out), _layer_flags(combine, separate_permute, split_k),
            _ptr(workspace), workspace.numel(), _stream()))
    return out


def _layer_flags(combine, separate_permute, split_k):
    return (_COMBINES[combine] | (MOE_LAYER_SEPARATE_PERMUTE if separate_permute else 0) |
            (MOE_LAYER_SPLIT_K if split_k else 0))


def layer_router(x: torch.Tensor, w_router: torch.Tensor, w_gate: torch.Tensor,
                 w_up: torch.Tensor | None, w_down: torch.Tensor, k: int,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 combine: str = "gather", separate_permute: bool = False,
                 split_k: bool = False) -> torch.Tensor:
    """The MoE layer share from the token rows and the router weights: the
    router front end (logits, top-k, softmax; the expert counts too when the
    permutation runs separately), then the permutation, the two grouped GEMMs
    and the combine (split K as in layer()).  The workspace holds the
    moe_layer_workspace_layout regions first, then the router's scratch."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.bfloat16, 2)
    _need(w_gate, "w_gate", torch.bfloat16, 3)
    if w_up is not None:
        _need(w_up, "w_up", torch.bfloat16, 3)
    _need(w_down, "w_down", torch.bfloat16, 3)
    T, H = x.shape
    E, _, I = w_gate.shape
    if w_up is None:
        I //= 2
    lib = load_library()
    if workspace is None:
        n = lib.moe_layer_router_workspace_size(T, H, E, k, I, _COMBINES[combine])
        if n == 0:
            raise ValueError("unsupported layer sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check("moe_layer_router", lib.moe_layer_router(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), T, H, E, k, I, _ptr(out),
        _layer_flags(combine, separate_permute, split_k), _ptr(workspace), workspace.numel(), _stream()))
    return out


def workspace_view(workspace: torch.Tensor, T, H, E, k, I, name: str) -> torch.Tensor:
    """A typed view of one intermediate inside a moe_layer workspace."""
    lay = layer_workspace_layout(T, H, E, k, I)
    cap = padded_capacity(T, k, E)
    shapes = {
        "topk_idx": ((T, k), torch.int32), "topk_w": ((T, k), torch.float32),
        "expert_counts": ((E,), torch.int32), "expert_offsets": ((E + 1,), torch.int32),
        "pair_to_row": ((T * k,), torch.int32), "row_to_pair": ((cap,), torch.int32),
        "block_expert": ((cap // ROW_BLOCK,), torch.int32), "num_padded_rows": ((1,), torch.int32),
        "h": ((cap, I), torch.bfloat16), "y": ((cap, H), torch.bfloat16),
        "out_acc": ((T, H), torch.float32),
    }
    shape, dt = shapes[name]
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dt).element_size()
    start = lay[name]
    return workspace[start:start + nbytes].view(dt).view(shape)
