"""The oracle: a plain CPU implementation of the grouped-GEMM MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
never links, loads or calls it, and it imports nothing from the HIP package.

The arithmetic lives in ``moe_oracle.c`` (plain C loops, double accumulation,
ascending index order); this module only builds it with gcc, loads it with
ctypes and marshals numpy arrays.  Every function names the passage of the
pages it follows in the C source.

Pins (tests under ``tests/test_oracle_*.py``) tie each function to brute force,
closed forms, invariants and special cases that reduce to textbook routines;
nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

ROW_BLOCK = 128


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the .so path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_router_logits.argtypes = [P, P, I, I, I, P]
    lib.oracle_router_logits.restype = None
    lib.oracle_route.argtypes = [P, I, I, I, P, P]
    lib.oracle_route.restype = None
    lib.oracle_permute.argtypes = [P, I, I, I, I, P, P, P, P, P]
    lib.oracle_permute.restype = I
    lib.oracle_gather.argtypes = [P, I, P, I, I, P]
    lib.oracle_gather.restype = None
    lib.oracle_grouped_gemm.argtypes = [I, I, I, I, P, P, I, P, P, I, P, I, P, I, P]
    lib.oracle_grouped_gemm.restype = None
    lib.oracle_combine.argtypes = [P, I, P, P, I, I, P]
    lib.oracle_combine.restype = None
    lib.oracle_weighted_scatter.argtypes = [P, I, I, P, P, I, I, P]
    lib.oracle_weighted_scatter.restype = None
    lib.oracle_moe_tokens.argtypes = [P, P, P, P, P, P, I, I, I, I, P, I, P]
    lib.oracle_moe_tokens.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _bind(build())
    return _lib


class _Variant:
    """The oracle API bound to another compiled copy of the C source.  Used
    only by the tests that plant a mistake in a copy of the oracle and check
    that the pins catch it."""

    def __init__(self, so_path):
        self._lib = _bind(so_path)

    def __getattr__(self, name):
        fn = globals()[name]

        def call(*a, **kw):
            global _lib
            saved = _lib
            _lib = self._lib
            try:
                return fn(*a, **kw)
            finally:
                _lib = saved
        return call


def compile_variant(src_text: str, out_path: str) -> "_Variant":
    """Compile C source text (a modified copy of the oracle) and bind it."""
    c_path = out_path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                           "-o", out_path, c_path, "-lm"])
    return _Variant(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def padded_capacity(T: int, k: int, E: int) -> int:
    """Largest padded row count any routing can need: each non-empty expert
    adds at most 127 padding rows, rounded up to whole 128-row blocks."""
    R = T * k
    cap = R + min(E, R) * (ROW_BLOCK - 1)
    return (cap + ROW_BLOCK - 1) // ROW_BLOCK * ROW_BLOCK


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """logits[t][e] = x[t] . W[e] in double (x [T][H], W [E][H], bf16 bits):
    the linear router whose output the routing takes.  Returns float64 [T,E]."""
    xb, xp = _c(x_bits, np.uint16)
    wb, wp = _c(w_bits, np.uint16)
    T, H = xb.shape
    E = wb.shape[0]
    if wb.shape[1] != H:
        raise ValueError("W must be [E][H]")
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(xp, wp, T, H, E, out.ctypes.data_as(ctypes.c_void_p))
    return out


def route(logits: np.ndarray, k: int):
    """Top-k experts of each token (slot 0 largest, ties to the lower id) and
    the softmax over the k chosen logits.  Returns (idx int32 [T,k], w fp32 [T,k])."""
    lg, lp = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_route(lp, T, E, k, idx.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p))
    return idx, w


def permute(idx: np.ndarray, E: int, cap: int | None = None):
    """Stable expert-major permutation with 128-row padding per expert.
    Returns a dict of counts [E], offsets [E+1], pair_to_row [R],
    row_to_pair [cap], block_expert [cap/128], m_pad."""
    ix, ip = _c(idx, np.int32)
    T, k = ix.shape
    if cap is None:
        cap = padded_capacity(T, k, E)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    p2r = np.empty(T * k, np.int32)
    r2p = np.empty(cap, np.int32)
    be = np.empty(cap // ROW_BLOCK, np.int32)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    m_pad = _load().oracle_permute(ip, T, k, E, cap, vp(counts), vp(offsets), vp(p2r), vp(r2p), vp(be))
    if m_pad < 0:
        raise ValueError("capacity %d too small" % cap)
    return dict(counts=counts, offsets=offsets, pair_to_row=p2r, row_to_pair=r2p,
                block_expert=be, m_pad=int(m_pad), cap=cap)


def gather(x_bits: np.ndarray, row_to_pair: np.ndarray, k: int) -> np.ndarray:
    """x_perm[row] = x[token of row], zero rows for padding (uint16 bits)."""
    xb, xp = _c(x_bits, np.uint16)
    r2p, rp = _c(row_to_pair, np.int32)
    H = xb.shape[1]
    cap = r2p.shape[0]
    out = np.empty((cap, H), np.uint16)
    _load().oracle_gather(xp, H, rp, k, cap, out.ctypes.data_as(ctypes.c_void_p))
    return out


def grouped_gemm(A_bits, B_bits, block_group, *, N, K, is_fp16=False, b_layout="kn",
                 a_src_row=None, a_src_div=1, B2_bits=None, epilogue="store", rows=None,
                 M=None):
    """D[r] = A[a(r)] . B[block_group[r/128]]  (or SiLU(A.B)*(A.B2)), in double.

    b_layout "kn": B is [G][K][N]; "nk": B is [G][N][K].  Rows listed in
    `rows` (default: all M rows) are computed; rows without a source are NaN."""
    Ab, Ap = _c(A_bits, np.uint16)
    Bb, Bp = _c(B_bits, np.uint16)
    bg, bgp = _c(block_group, np.int32)
    if B2_bits is not None:
        B2b, B2p = _c(B2_bits, np.uint16)
    else:
        B2p = None
    if a_src_row is not None:
        asr, asp = _c(a_src_row, np.int32)
        Mrows = asr.shape[0]
    else:
        asp = None
        Mrows = Ab.shape[0]
    if M is None:
        M = Mrows
    if rows is not None:
        rw, rwp = _c(rows, np.int32)
        nrows = rw.shape[0]
    else:
        rwp, nrows = None, M
    D = np.empty((nrows, N), np.float64)
    epi = {"store": 0, "silu_mul": 1}[epilogue]
    lay = {"kn": 0, "nk": 1}[b_layout]
    _load().oracle_grouped_gemm(int(is_fp16), M, N, K, Ap, asp, a_src_div, Bp, B2p, lay, bgp, epi,
                                rwp, nrows, D.ctypes.data_as(ctypes.c_void_p))
    return D


def combine(y_bits, pair_to_row, w):
    """out[t] = sum_j w[t,j] * y[pair_to_row[t*k+j]] in double; y is bf16 bits."""
    yb, yp = _c(y_bits, np.uint16)
    wa, wp = _c(w, np.float32)
    pr, pp = _c(pair_to_row, np.int32)
    T, k = wa.shape
    H = yb.shape[1]
    out = np.empty((T, H), np.float64)
    _load().oracle_combine(yp, H, pp, wp, T, k, out.ctypes.data_as(ctypes.c_void_p))
    return out


def weighted_scatter(Y, row_to_pair, w, k, T):
    """out[p // k] += w[p] * Y[r] for every row r with p = row_to_pair[r] >= 0,
    in double; Y is [M, N] double (rows in permuted order), w is [T*k] fp32."""
    Ya = np.ascontiguousarray(Y, dtype=np.float64)
    rp, rpp = _c(row_to_pair, np.int32)
    wa, wp = _c(np.asarray(w, dtype=np.float32).reshape(-1), np.float32)
    M, N = Ya.shape
    if rp.shape[0] < M:
        raise ValueError("row_to_pair shorter than Y")
    out = np.empty((T, N), np.float64)
    _load().oracle_weighted_scatter(Ya.ctypes.data_as(ctypes.c_void_p), M, N, rpp, wp, k, T,
                                    out.ctypes.data_as(ctypes.c_void_p))
    return out


def moe_tokens(x_bits, idx, w, Wg_bits, Wu_bits, Wd_bits, tokens=None):
    """The layer by its definition, one token at a time (double):
    out[t] = sum_j w[t,j] * (SiLU(x_t.Wg[e]) * (x_t.Wu[e])) . Wd[e],  e = idx[t,j]."""
    xb, xp = _c(x_bits, np.uint16)
    ix, ip = _c(idx, np.int32)
    wa, wp = _c(w, np.float32)
    g, gp = _c(Wg_bits, np.uint16)
    u, up = _c(Wu_bits, np.uint16)
    d, dp = _c(Wd_bits, np.uint16)
    T, H = xb.shape
    E, _, I = g.shape
    k = ix.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tk, tp = _c(tokens, np.int32)
    out = np.empty((tk.shape[0], H), np.float64)
    _load().oracle_moe_tokens(xp, ip, wp, gp, up, dp, H, E, k, I, tp, tk.shape[0],
                              out.ctypes.data_as(ctypes.c_void_p))
    return out
