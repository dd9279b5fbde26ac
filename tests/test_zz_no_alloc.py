"""grouped_gemm_noalloc -- the grouped GEMM without a workspace, its row-task
plan in the library's own per-GPU array -- against grouped_gemm with a
caller workspace, through the C ABI: the same bits, on calls in a row whose
sizes shrink (the array keeps the previous call's plan; each call must
rewrite what it reads)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import dev16, say

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _p(t):
    return None if t is None else P(t.data_ptr())


def _case(T, k, E, K, N, seed, epi, dense_values=True):
    g = np.random.default_rng(seed)
    idx, w = oracle.route(g.standard_normal((T, E)).astype(np.float32), k)
    Pm = oracle.permute(idx, E)
    cap = Pm["cap"]
    if dense_values:
        # gate/up (epi 1) gathers A rows as row_to_pair / k: T rows; the store
        # reads A row r for every row r below M_pad: cap rows
        A = syn.bf16_bits(g.standard_normal((T if epi == 1 else cap, K)).astype(np.float32))
        B = syn.bf16_bits((g.standard_normal((E, K, N)) / np.sqrt(K)).astype(np.float32))
        B2 = syn.bf16_bits((g.standard_normal((E, K, N)) / np.sqrt(K)).astype(np.float32))
    else:  # integer values: the scatter's atomic sums are then unique
        A = syn.sparse_ternary_bits((cap, K), seed + 1, 0.5)
        B = syn.sparse_ternary_bits((E, K, N), seed + 2, 0.5)
        B2 = None
        w = g.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), size=(T, k))
    return dict(T=T, k=k, E=E, K=K, N=N, epi=epi, cap=cap, m_pad=Pm["m_pad"],
                bexp=torch.from_numpy(Pm["block_expert"]).cuda(), r2p=torch.from_numpy(Pm["row_to_pair"]).cuda(),
                A=dev16(A), B=dev16(B), B2=None if B2 is None or epi != 1 else dev16(B2),
                w=torch.from_numpy(w).cuda())


def _run(lib, c, noalloc):
    epi, N, K, cap, T = c["epi"], c["N"], c["K"], c["cap"], c["T"]
    mpad = torch.tensor([c["m_pad"]], dtype=torch.int32, device="cuda")
    if epi == 2:
        D = torch.zeros((T, N), dtype=torch.float32, device="cuda")
        src, div, rp, pw = None, 1, c["r2p"], c["w"]
    else:
        D = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        # gate/up: A rows gathered through the row map; store: identity rows, padding skipped
        src, div, rp, pw = (c["r2p"], c["k"], None, None) if epi == 1 else (None, 1, c["r2p"], None)
    args = (0, N, K, cap, _p(c["A"]), _p(src), div, _p(c["B"]), _p(c["B2"]), 0, _p(c["bexp"]), _p(mpad), epi,
            _p(rp), _p(pw), c["k"] if epi == 2 else 0, _p(D))
    stream = P(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.grouped_gemm_noalloc(*args, stream)
    else:
        ws = torch.empty(lib.grouped_gemm_workspace_size(cap), dtype=torch.uint8, device="cuda")
        st = lib.grouped_gemm(*args, _p(ws), ws.numel(), stream)
    assert st == moe.MOE_OK, moe.load_library().moe_status_string(st)
    torch.cuda.synchronize()
    return D


def test_noalloc_matches_workspace_entry_point():
    lib = moe.load_library()
    # calls in a row, each smaller than the one before: a gate/up GEMM of the
    # tp_share routing (98 blocks), a down GEMM of a small routing, then a
    # weighted scatter of a smaller one still
    cases = [(2048, 4, 64, 1024, 512, 1, 1, True), (300, 2, 6, 256, 256, 2, 0, True),
             (90, 2, 3, 128, 256, 3, 2, False)]
    for T, k, E, K, N, seed, epi, dense in cases:
        c = _case(T, k, E, K, N, seed, epi, dense)
        say("noalloc", dict(T=T, k=k, E=E, K=K, N=N, epi=epi, cap=c["cap"]))
        ref = _run(lib, c, noalloc=False)
        got = _run(lib, c, noalloc=True)
        iv = torch.int32 if epi == 2 else torch.int16
        assert torch.equal(got.view(iv), ref.view(iv)), (T, k, E, epi)
        if epi != 2:
            assert not torch.isnan(got[:c["m_pad"]][c["r2p"][:c["m_pad"]] >= 0]).any()


def test_noalloc_rejects_capacity_beyond_its_array():
    lib = moe.load_library()
    big = (1 << 20) + 128
    st = lib.grouped_gemm_noalloc(0, 128, 128, big, P(4096), None, 1, P(4096), None, 0, P(4096), P(4096), 0,
                                  None, None, 0, P(4096), None)
    assert st == moe.MOE_ERR_WORKSPACE
