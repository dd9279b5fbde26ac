"""GPU checks of the layer's split-K form (MOE_LAYER_SPLIT_K, split_k=True).
A GEMM of the layer with at most one wave of (row task, column block) tasks
("Comm-compute fusion (1)", section 5: below one wave the compute units stand
idle) runs its k range in parts whose fp32 partial sums a reduction adds in a
fixed order, applying SiLU*up after gate/up and the top-k weighted combine
after down.

* against the oracle, every token, at the bf16 tolerances of the layer
  (ragged experts, an expert of two 128-row blocks, pairs routed outside
  [0, E), both combines, the router front end);
* on integer-valued inputs chosen so that every sum is exact in fp32 (gate
  columns of one sign and |gate| >= 128, where SiLU is exactly the identity
  or zero; sparse +-1 up and down weights bounding every partial sum below
  2^24), bit for bit against the unsplit layer: a part missing, doubled or
  written to the wrong pair or column would change an output.  The
  workspace's y region then holds the down GEMM's partials, which must add
  up to the unsplit layer's y."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import assert_close, dev16, say, to_f64

pytestmark = pytest.mark.gpu


def _parts(R, E, N, bn, nb, K, room, cus=256):
    """k parts of a layer GEMM as moe.h states the rule: split when even the
    most row tasks any routing gives, floor((R + 255 min(E, R)) / 256), times
    the column blocks fit one wave; 4 parts, else 2, of >= 16 slices of 32."""
    rt = (R + 255 * min(E, R)) // 256
    if N % bn or rt * (N // bn) > cus:
        return 1
    for p in (4, 2):
        if K % (32 * p) == 0 and K // 32 // p >= 16 and p * R * nb * N * 4 <= room:
            return p
    return 1


def _heavy_routing(T, E, k, seed, bad=True):
    """Distinct experts per token; the first 150 tokens all take expert 0
    (two 128-row blocks) when k > 1, the first third of them when k == 1;
    with bad=True some pairs name no valid expert."""
    heavy = 150 if k > 1 else T // 3
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    for t in range(min(heavy, T)):
        if 0 in idx[t]:
            j = int(np.nonzero(idx[t] == 0)[0][0])
            idx[t, [0, j]] = idx[t, [j, 0]]
        else:
            idx[t, 0] = 0
    if bad:
        idx[::29, k - 1] = -1
        idx[7, 0] = E + 2
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    return idx, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def _case(T, H, E, k, I, seed):
    d = syn.make_moe(T, H, E, k, I, seed=seed, routing="uniform_idx")
    d["topk_idx"], d["topk_w"] = _heavy_routing(T, E, k, seed)
    return d


def _oracle_out(d, idx, w):
    """The oracle's layer, every token; a pair naming no valid expert adds
    nothing (the layer gives it no row), i.e. it enters with weight 0."""
    bad = (idx < 0) | (idx >= d["E"])
    return oracle.moe_tokens(d["x"], np.where(bad, 0, idx).astype(np.int32),
                             np.where(bad, 0, w).astype(np.float32), d["wg"], d["wu"], d["wd"],
                             tokens=np.arange(d["T"], dtype=np.int32))


# (T, H, E, k, I, seed): both GEMMs in 2 parts (4 would not fit the
# workspace, or leave parts under 16 slices); both in 4 with several items
# per workgroup; a shape where only gate/up splits
CASES = [(160, 2048, 8, 2, 1024, 11), (128, 2048, 16, 1, 2048, 12), (96, 4096, 64, 1, 512, 13)]


def _split_parts(T, H, E, k, I):
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    room = lay["permute_scratch"] - lay["y"]  # the partials live in y's region
    R = T * k
    return _parts(R, E, I, 128, 2, H, room), _parts(R, E, H, 256, 1, I, room)


def _dev(d):
    return {n: dev16(d[n]) for n in ("x", "wg", "wu", "wd")}


def _layer(D, d, split_k=True, combine="gather", ws=None):
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    ws = moe.layer_workspace(T, H, E, k, I) if ws is None else ws
    out = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=torch.from_numpy(d["topk_idx"]).cuda(),
                    topk_w=torch.from_numpy(d["topk_w"]).cuda(), workspace=ws, combine=combine,
                    split_k=split_k)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_E%d_k%d_I%d" % c[:5])
def test_split_layer_matches_oracle(case):
    T, H, E, k, I, seed = case
    d = _case(*case)
    ks = _split_parts(T, H, E, k, I)
    assert max(ks) > 1, "not a split-K shape"
    say("split K vs oracle", case, "parts gate/up %d down %d" % ks)
    D = _dev(d)
    ref = _oracle_out(d, d["topk_idx"], d["topk_w"])
    for combine in ("gather", "scatter"):
        out, ws = _layer(D, d, combine=combine)
        r = assert_close(to_f64(out), ref, "split %s %s" % (combine, case))
        say("split K", combine, "max|err|/max|ref| %.2e  relFro %.2e" % r)
        # the unsplit sums: within the tolerance of the split ones
        out_n, _ = _layer(D, d, split_k=False, combine=combine)
        assert_close(to_f64(out_n), ref, "unsplit %s %s" % (combine, case))
    # deterministic: the same bits on a second run (gather)
    o1, _ = _layer(D, d)
    o2, _ = _layer(D, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # pairs routed to no valid expert have no row
    flat = d["topk_idx"].ravel()
    bad = (flat < 0) | (flat >= E)
    p2r = moe.workspace_view(ws, T, H, E, k, I, "pair_to_row").cpu().numpy()
    assert bad.any() and np.all(p2r[bad] == -1)


def _integer_inputs(T, H, E, k, I, seed, nu, nd):
    """Integer-valued bf16 inputs whose every fp32 sum is exact (module
    docstring); nu / nd: nonzeros per up / down weight column."""
    assert 4 * H * nu * nd * 1.01 < 2 ** 24 and H % nu == 0 and I % nd == 0
    g = torch.Generator(device="cuda").manual_seed(seed)
    dev = "cuda"
    x = torch.randint(1, 3, (T, H), generator=g, device=dev, dtype=torch.int8)
    sgn = torch.randint(0, 2, (E, 1, I), generator=g, device=dev, dtype=torch.int8) * 2 - 1
    keep = torch.randint(0, 2, (E, H, I), generator=g, device=dev, dtype=torch.int8)
    keep[:, :128, :] = 1  # |gate| >= 128: e^-gate is 0 or overflows
    wg = sgn * keep
    hh = torch.arange(H, device=dev).view(1, H, 1)
    ee = torch.arange(E, device=dev).view(E, 1, 1)
    cu = torch.arange(I, device=dev).view(1, 1, I)
    su = torch.randint(0, 2, (E, H, I), generator=g, device=dev, dtype=torch.int8) * 2 - 1
    wu = su * ((hh + 7 * cu + 13 * ee) % (H // nu) == 0).to(torch.int8)
    ii = torch.arange(I, device=dev).view(1, I, 1)
    ch = torch.arange(H, device=dev).view(1, 1, H)
    sd = torch.randint(0, 2, (E, I, H), generator=g, device=dev, dtype=torch.int8) * 2 - 1
    wd = sd * ((ii + 3 * ch + 5 * ee) % (I // nd) == 0).to(torch.int8)
    bf = lambda t: t.to(torch.bfloat16).contiguous()
    return dict(x=bf(x), wg=bf(wg), wu=bf(wu), wd=bf(wd))


# (T, H, E, k, I, seed, nu, nd)
EXACT = [(160, 2048, 8, 2, 1024, 21, 32, 32), (128, 4096, 16, 1, 2048, 22, 16, 32),
         (96, 4096, 64, 1, 512, 23, 16, 32)]


@pytest.mark.parametrize("case", EXACT, ids=lambda c: "T%d_H%d_E%d_k%d_I%d" % c[:5])
def test_split_exact_sums_same_bits_as_unsplit(case):
    T, H, E, k, I, seed, nu, nd = case
    d = dict(T=T, H=H, E=E, k=k, I=I)
    d["topk_idx"], d["topk_w"] = _heavy_routing(T, E, k, seed)
    R = T * k
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    ks_gu, ks_dn = _split_parts(T, H, E, k, I)
    say("split K exact", case, "parts gate/up %d down %d" % (ks_gu, ks_dn))
    assert max(ks_gu, ks_dn) > 1
    D = _integer_inputs(T, H, E, k, I, seed, nu, nd)
    out_s, ws_s = _layer(D, d, split_k=True)
    out_n, ws_n = _layer(D, d, split_k=False)
    assert torch.isfinite(out_s.float()).all()
    assert torch.equal(out_s.view(torch.int16), out_n.view(torch.int16))
    view = lambda ws, n: moe.workspace_view(ws, T, H, E, k, I, n)
    p2r = view(ws_n, "pair_to_row").long()
    ok = p2r >= 0
    rows = p2r[ok]
    # h of every pair's row (written by the reduction after a split gate/up)
    assert torch.equal(view(ws_s, "h")[rows].view(torch.int16), view(ws_n, "h")[rows].view(torch.int16))
    if ks_dn > 1:
        # the down GEMM's fp32 partials, [parts][pairs][H], in y's region:
        # their sum (exact) rounds to the unsplit layer's y of the pair's row
        part = ws_s[lay["y"]:lay["y"] + ks_dn * R * H * 4].view(torch.float32).view(ks_dn, R, H)
        y_s = part.sum(0)[ok].to(torch.bfloat16)
        y_n = view(ws_n, "y")[rows]
        assert torch.equal(y_s.view(torch.int16), y_n.view(torch.int16))
        # and no part is empty: each holds nonzero sums of real pairs
        assert all(bool((part[s][ok] != 0).any()) for s in range(ks_dn))


def test_split_router_front_end():
    # the router front end with a split layer: the same bits as the layer
    # given the router's own routing (both take the separate permutation)
    T, H, E, k, I, seed = CASES[0]
    d = syn.make_moe(T, H, E, k, I, seed=seed, routing="uniform_idx")
    D = _dev(d)
    wr = dev16(syn.bf16_bits((np.random.default_rng(5).standard_normal((E, H)) / np.sqrt(H))
                             .astype(np.float32)))
    lib = moe.load_library()
    ws = torch.empty(lib.moe_layer_router_workspace_size(T, H, E, k, I, 0), dtype=torch.uint8, device="cuda")
    say("split K router front end", (T, H, E, k, I))
    out = moe.layer_router(D["x"], wr, D["wg"], D["wu"], D["wd"], k, workspace=ws, split_k=True)
    torch.cuda.synchronize()
    idx = moe.workspace_view(ws, T, H, E, k, I, "topk_idx").clone()
    w = moe.workspace_view(ws, T, H, E, k, I, "topk_w").clone()
    out2 = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=idx, topk_w=w, split_k=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert_close(to_f64(out), _oracle_out(d, idx.cpu().numpy(), w.cpu().numpy()), "split router")


def test_split_hip_graph_replays():
    # the split layer (GEMMs, the SiLU*up reduction, the combining reduction)
    # captured in one HIP graph replays to the eager bits every time
    T, H, E, k, I, seed = CASES[0]
    d = _case(T, H, E, k, I, seed)
    D = _dev(d)
    ws = moe.layer_workspace(T, H, E, k, I)
    idx, w = torch.from_numpy(d["topk_idx"]).cuda(), torch.from_numpy(d["topk_w"]).cuda()
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    run = lambda o=None: moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=idx, topk_w=w,
                                   workspace=ws, out=o, split_k=True)
    say("split K graph")
    eager = run().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep


def test_split_small_expert_share_matches_oracle():
    # the small-T expert share (T=128, E=16 under Zipf routing, H=4096,
    # I=2048) split in 4 parts in both GEMMs: every token against the oracle
    d = syn.make_config("ep_skew_small")
    assert _split_parts(d["T"], d["H"], d["E"], d["k"], d["I"]) == (4, 4)
    D = _dev(d)
    say("split ep_skew_small")
    out, _ = _layer(D, d, split_k=True)
    tokens = np.arange(d["T"], dtype=np.int32)
    ref = oracle.moe_tokens(d["x"], d["topk_idx"], d["topk_w"], d["wg"], d["wu"], d["wd"], tokens=tokens)
    assert_close(to_f64(out), ref, "split ep_skew_small")
