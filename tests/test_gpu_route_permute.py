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


def test_route_special_values():
    """The selection order on the fp32 bit patterns that order tricks get
    wrong: -0 equal to +0 (ties to the lower id), denormals, the smallest
    normals and +-FLT_MAX, with many duplicates.  Weights of experts far below
    the top are exactly 0 on both sides, so they are compared with an absolute
    floor."""
    vals = np.array([-0.0, 0.0, 1e-45, -1e-45, 1.1754944e-38, -1.1754944e-38, 3.4028235e38,
                     -3.4028235e38, 1.0, -1.0, 2.0, -2.0], dtype=np.float32)
    g = np.random.default_rng(23)
    for E, k in ((12, 4), (70, 9), (130, 16)):
        lg = vals[g.integers(0, len(vals), size=(300, E))]
        lg[0, :] = -0.0
        lg[1, :] = 0.0
        lg[2, ::2] = -0.0  # alternating -0 / +0: equal, so the lowest ids win
        lg[2, 1::2] = 0.0
        say("route special values E", E, "k", k)
        idx, w = moe.route(torch.from_numpy(lg).cuda(), k)
        torch.cuda.synchronize()
        ridx, rw = oracle.route(lg, k)
        assert np.array_equal(idx.cpu().numpy(), ridx), (E, k)
        assert np.array_equal(ridx[2], np.arange(k)), "the oracle takes -0 == +0"
        wg = w.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(wg - rw) <= 1e-6 * np.abs(rw) + 1e-37), (E, k)


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
    cap = moe.padded_capacity(T, k, E)
    xp = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device="cuda") if with_x else None
    P = moe.permute(torch.from_numpy(idx_np).cuda(), E, x=dev16(x_bits) if with_x else None, x_perm=xp)
    torch.cuda.synchronize()
    for name in ("counts", "offsets", "pair_to_row", "row_to_pair", "block_expert"):
        got = getattr(P, name).cpu().numpy()
        assert np.array_equal(got, ref[name]), "%s %s" % (what, name)
    m = ref["m_pad"]
    assert int(P.num_padded_rows.item()) == m
    if with_x:
        got = host16(P.x_perm)
        assert np.array_equal(got[:m], oracle.gather(x_bits, ref["row_to_pair"], k)[:m])
        assert np.all(got[m:] == host16(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0])


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


def _small_layer_inputs(T, H, E, k, I, seed):
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E)).astype(np.float32)
    bits = lambda shape: syn.bf16_bits((g.standard_normal(shape) * 0.05).astype(np.float32))
    return (logits, dev16(bits((T, H))), dev16(bits((E, H, I))), dev16(bits((E, H, I))),
            dev16(bits((E, I, H))))


# router front end: every column-tile count (E up to 32, 64, 96, 128), a
# hidden quarter below and above one load batch, ragged token blocks, the
# tp_share router shape
@pytest.mark.parametrize("T,H,E,k", [(2048, 4096, 64, 4), (77, 256, 5, 2), (300, 192, 128, 16),
                                     (33, 64, 33, 3), (1, 512, 1, 1), (1000, 1024, 96, 8),
                                     (512, 4096, 16, 1), (8192, 512, 64, 8)])
def test_router_matches_oracle(T, H, E, k):
    g = np.random.default_rng(T + H + E + k)
    x = syn.bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    W = syn.bf16_bits((g.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    say("router", "T", T, "H", H, "E", E, "k", k)
    # a workspace of garbage: its contents need no clearing
    ws = torch.full((max(256, moe.load_library().moe_router_workspace_size(T, H, E)),), 0xA5,
                    dtype=torch.uint8, device="cuda")
    idx, w, lg, counts = moe.router(dev16(x), dev16(W), k, with_logits=True, workspace=ws, with_counts=True)
    torch.cuda.synchronize()
    idx, w, lg, counts = idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy(), counts.cpu().numpy()
    # the expert histogram of the launch: exactly the count of the routing it wrote
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    # logits: within the fp32 summation bound of the exact sum (bf16 products
    # are exact in fp32; H additions at most, each off by half an ulp)
    ref = oracle.router_logits(x, W)
    mag = oracle.router_logits(x & 0x7FFF, W & 0x7FFF)    # sum of |x||w|
    bound = H * 2.0 ** -24 / (1 - H * 2.0 ** -24) * mag
    assert np.all(np.abs(lg.astype(np.float64) - ref) <= bound)
    # the selection on the kernel's own fp32 logits: exactly the routing rule
    ridx, rw = oracle.route(lg, k)
    assert np.array_equal(idx, ridx)
    assert np.max(np.abs(w.astype(np.float64) - rw) / np.abs(rw)) <= 1e-6
    # against the routing of the exact logits: a token may differ only at a
    # near tie, where the two choices are within the logits' error bound
    oidx, _ = oracle.route(ref.astype(np.float32), k)
    for t in np.nonzero(np.any(idx != oidx, axis=1))[0]:
        a, b = set(idx[t]), set(oidx[t])
        pairs = [(e, f) for e in a - b for f in b - a] or list(zip(idx[t], oidx[t]))
        for e, f in pairs:
            assert abs(ref[t, e] - ref[t, f]) <= 2 * (bound[t, e] + bound[t, f]), (t, e, f)


@pytest.mark.parametrize("T,H,E,k", [(2048, 4096, 64, 4), (8192, 256, 16, 2)])
def test_router_repeats_and_graph_replays(T, H, E, k):
    # one workspace across calls, and the call captured in a HIP graph and
    # replayed with eager work between replays: the same bits every time
    # (the slices are added in a fixed order; the counts are cleared by the
    # call itself)
    g = np.random.default_rng(5)
    x = dev16(syn.bf16_bits(g.standard_normal((T, H)).astype(np.float32)))
    W = dev16(syn.bf16_bits((g.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)))
    ws = torch.zeros(max(256, moe.load_library().moe_router_workspace_size(T, H, E)), dtype=torch.uint8,
                     device="cuda")
    say("router repeats and graph", T, H, E, k)
    ref = moe.router(x, W, k, with_logits=True, workspace=ws, with_counts=True)
    ref = [t.clone() for t in ref]
    for _ in range(3):
        again = moe.router(x, W, k, with_logits=True, workspace=ws, with_counts=True)
        for a, b in zip(ref, again):
            assert torch.equal(a, b)
    outs = [torch.empty_like(t) for t in ref]
    lib = moe.load_library()

    def call():
        st = lib.moe_router(moe._ptr(x), moe._ptr(W), T, H, E, k, moe._ptr(outs[2]), moe._ptr(outs[0]),
                            moe._ptr(outs[1]), moe._ptr(outs[3]), moe._ptr(ws), ws.numel(), moe._stream())
        assert st == moe.MOE_OK
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        for t in outs:
            t.zero_()
        moe.router(x, W, k, workspace=ws)  # an eager call between the replays, same workspace
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), rep


@pytest.mark.parametrize("name,combine", [("tiny", "gather"), ("tp_share", "gather"), ("tp_share", "scatter")])
def test_layer_router_matches_oracle(name, combine):
    # the layer from x and the router weights: its routing is the routing
    # rule on the router's own fp32 logits (bit for bit), its permutation the
    # oracle's of that routing, its output the layer's definition
    d = syn.make_config(name)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    Wr = syn.bf16_bits((np.random.default_rng(11).standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    x, wr = dev16(d["x"]), dev16(Wr)
    wg, wu, wd = dev16(d["wg"]), dev16(d["wu"]), dev16(d["wd"])
    lib = moe.load_library()
    ws = torch.full((lib.moe_layer_router_workspace_size(T, H, E, k, I, 0 if combine == "gather" else 1),),
                    0x3C, dtype=torch.uint8, device="cuda")
    say("layer router", name, combine)
    out = moe.layer_router(x, wr, moe.pack_gate_up(wg, wu), None, wd, k, workspace=ws, combine=combine)
    _, _, lg = moe.router(x, wr, k, with_logits=True)
    torch.cuda.synchronize()
    idx, w = oracle.route(lg.cpu().numpy(), k)
    view = lambda n: moe.workspace_view(ws, T, H, E, k, I, n).cpu().numpy()
    assert np.array_equal(view("topk_idx"), idx)
    assert np.max(np.abs(view("topk_w") - w) / w) <= 1e-6
    P = oracle.permute(idx, E)
    for n_ws, n_or in [("expert_counts", "counts"), ("expert_offsets", "offsets"),
                       ("pair_to_row", "pair_to_row"), ("row_to_pair", "row_to_pair"),
                       ("block_expert", "block_expert")]:
        assert np.array_equal(view(n_ws), P[n_or]), n_ws
    tokens = np.arange(T, dtype=np.int32) if T <= 256 else np.sort(
        np.random.default_rng(0).choice(T, 96, replace=False)).astype(np.int32)
    ref = oracle.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"], tokens=tokens)
    from _util import assert_close, to_f64
    r = assert_close(to_f64(out)[tokens], ref, "layer router " + name)
    say("layer router", name, "max|err|/max|ref| %.2e  relFro %.2e" % r)


# shapes of every variant of the one-launch routing + permutation + plan
# (tokens per thread 1, 2, 4 x top-k list of 4, 8, 16) and one shape that
# takes the separate kernels instead (E not a multiple of 4)
@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (1000, 64, 8), (64, 1024, 16), (2048, 64, 4),
                                   (2000, 16, 7), (4096, 32, 4), (77, 5, 5)])
def test_layer_routing_permutation_and_plan(T, E, k):
    H = I = 64
    logits, x, wg, wu, wd = _small_layer_inputs(T, H, E, k, I, T + E + k)
    lg = torch.from_numpy(logits).cuda()
    say("layer routing + permutation + plan", "T", T, "E", E, "k", k)
    ws = moe.layer_workspace(T, H, E, k, I)
    moe.layer(x, wg, wu, wd, k, logits=lg, workspace=ws)
    idx, w = moe.route(lg, k)
    torch.cuda.synchronize()
    view = lambda n: moe.workspace_view(ws, T, H, E, k, I, n).cpu().numpy()
    # the layer's routing: the same bits as the routing entry point
    assert np.array_equal(view("topk_idx"), idx.cpu().numpy())
    assert np.array_equal(view("topk_w").view(np.uint32), w.cpu().numpy().view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), oracle.route(logits, k)[0])
    ref = oracle.permute(idx.cpu().numpy(), E)
    for name, key in (("expert_counts", "counts"), ("expert_offsets", "offsets"),
                      ("pair_to_row", "pair_to_row"), ("row_to_pair", "row_to_pair"),
                      ("block_expert", "block_expert")):
        assert np.array_equal(view(name), ref[key]), name
    assert int(view("num_padded_rows")[0]) == ref["m_pad"]
    # the layer's row-task plan: the same as the grouped GEMM's own plan kernel
    P = moe.permute(idx, E)
    cap = P.cap
    gws = torch.zeros(moe.gemm_workspace(cap).numel(), dtype=torch.uint8, device="cuda")
    say("plan reference", "cap", cap)
    moe.grouped_gemm(x, wg, P.block_expert, P.num_padded_rows, N=I, K=H, cap=cap,
                     a_src_row=P.row_to_pair, a_src_div=k, B2=wu, epilogue="silu_mul",
                     workspace=gws)
    torch.cuda.synchronize()
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    n = 2 + 2 * (cap // 128)
    plan = ws[lay["gemm_scratch"]:lay["gemm_scratch"] + 4 * n].view(torch.int32).cpu().numpy()
    plan_ref = gws[:4 * n].view(torch.int32).cpu().numpy()
    used = 2 + 2 * int(plan_ref[0])
    assert np.array_equal(plan[:used], plan_ref[:used])


@pytest.mark.parametrize("T,k,E", [(700, 3, 8), (5000, 4, 37), (9000, 8, 64)])
def test_permute_skips_invalid_ids(T, k, E):
    # expert ids outside [0, E) get no row; the valid pairs are still a stable
    # counting sort (checked by its defining properties).  Up to 16384 pairs
    # take the one-launch kernel, more the three-pass counting sort.
    g = np.random.default_rng(21)
    idx = g.integers(0, E, size=(T, k)).astype(np.int32)
    idx[::7, 0] = -3
    idx[::11, k - 1] = E
    idx[5, 1] = 1 << 20
    idx[T - 1, :] = -(1 << 30)
    say("permute invalid ids", T, k, E)
    P = moe.permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    p2r = P.pair_to_row.cpu().numpy()
    r2p = P.row_to_pair.cpu().numpy()
    bexp = P.block_expert.cpu().numpy()
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(P.counts.cpu().numpy(), counts)
    padded = (counts + 127) // 128 * 128
    offs = np.concatenate([[0], np.cumsum(padded)])
    assert np.array_equal(P.offsets.cpu().numpy(), offs)
    assert np.all(p2r[~valid] == -1)
    pv = np.nonzero(valid)[0]
    rows = p2r[pv]
    assert np.array_equal(r2p[rows], pv)
    for e in range(E):
        re = rows[flat[pv] == e]
        assert np.array_equal(re, np.arange(offs[e], offs[e] + counts[e]))
        assert np.all(bexp[offs[e] // 128:offs[e + 1] // 128] == e)
    real = np.zeros(P.cap, bool)
    real[rows] = True
    assert np.all(r2p[~real] == -1)
