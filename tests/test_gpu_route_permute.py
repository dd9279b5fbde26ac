"""GPU parity of routing and permutation with the oracle: bit-exact indices,
counts, offsets, row maps and block experts; weights within 1e-6 relative."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import dev16, host16, say

pytestmark = pytest.mark.gpu


def _route_case(logits, k, what):
    say("route", what, logits.shape, "k", k)
    idx, w = moe.route(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    ridx, rw = oracle.route(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx), what
    wg = w.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(wg - rw) / np.abs(rw)) <= 1e-6, what


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (2048, 64, 4), (1000, 64, 8), (77, 5, 5),
                                   (300, 1, 1), (513, 130, 3), (64, 1024, 16), (16384, 64, 8)])
def test_route_random(T, E, k):
    g = np.random.default_rng(T * 7 + E)
    _route_case(g.standard_normal((T, E)).astype(np.float32), k, "random")


def test_route_ties_and_special_rows():
    g = np.random.default_rng(11)
    lg = g.integers(-2, 3, size=(500, 12)).astype(np.float32)  # many ties
    for k in (1, 3, 12):
        _route_case(lg, k, "ties")
    _route_case(np.zeros((40, 64), np.float32), 8, "all-equal")
    big = g.standard_normal((64, 200)).astype(np.float32) * 30
    _route_case(big, 6, "wide-range")


def test_route_config_shapes():
    for name in ("tiny", "tp_share", "prefill"):
        d = syn.make_config(name, with_weights=False)
        _route_case(d["logits"], d["k"], name)


def _permute_case(idx_np, E, with_x=False, H=64, what=""):
    T, k = idx_np.shape
    say("permute", what, "T", T, "k", k, "E", E)
    ref = oracle.permute(idx_np, E)
    x_bits = None
    if with_x:
        x_bits = np.random.default_rng(T).integers(0, 65535, size=(T, H)).astype(np.uint16)
        x_bits[x_bits & 0x7f80 == 0x7f80] = 0  # keep values finite (bits are copied anyway)
    P = moe.permute(torch.from_numpy(idx_np).cuda(), E, x=dev16(x_bits) if with_x else None)
    torch.cuda.synchronize()
    for name in ("counts", "offsets", "pair_to_row", "row_to_pair", "block_expert"):
        got = getattr(P, name).cpu().numpy()
        assert np.array_equal(got, ref[name]), "%s %s" % (what, name)
    assert int(P.num_padded_rows.item()) == ref["m_pad"]
    if with_x:
        assert np.array_equal(host16(P.x_perm), oracle.gather(x_bits, ref["row_to_pair"], k))


def test_permute_cases():
    g = np.random.default_rng(5)
    _permute_case(g.integers(0, 8, size=(256, 2)).astype(np.int32), 8, True, what="random")
    _permute_case(np.zeros((3000, 1), np.int32), 4, True, what="one expert")
    _permute_case(np.array([[2]], np.int32), 3, True, what="one token")
    for n in (127, 128, 129, 255, 256, 257):
        _permute_case(np.full((n, 1), 1, np.int32), 2, what="count %d" % n)
    _permute_case(g.integers(0, 1, size=(999, 1)).astype(np.int32), 1, True, what="E=1")
    _permute_case(g.integers(0, 1024, size=(5000, 3)).astype(np.int32), 1024, what="E=1024")
    # empty experts
    idx = g.integers(0, 16, size=(700, 4)).astype(np.int32)
    idx[np.isin(idx, [3, 7, 8])] = 0
    _permute_case(idx, 16, True, H=4096, what="empty experts")


def test_permute_config_shapes():
    for name in ("tiny", "tp_share", "ep_skew", "ep_skew_small", "prefill"):
        d = syn.make_config(name, with_weights=False)
        idx = d["topk_idx"] if "topk_idx" in d else oracle.route(d["logits"], d["k"])[0]
        _permute_case(idx, d["E"], with_x=(name != "prefill"), H=d["H"], what=name)


def test_permute_repeatable():
    g = np.random.default_rng(9)
    idx = torch.from_numpy(g.integers(0, 64, size=(16384, 8)).astype(np.int32)).cuda()
    say("permute repeat")
    a = moe.permute(idx, 64)
    b = moe.permute(idx, 64)
    torch.cuda.synchronize()
    assert torch.equal(a.pair_to_row, b.pair_to_row) and torch.equal(a.row_to_pair, b.row_to_pair)
