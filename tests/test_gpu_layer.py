"""GPU parity of the whole MoE layer share (moe_layer and the step-by-step
path) with the oracle, on every workload shape: bit-exact routing and
permutation inside the layer's workspace, outputs within the bf16
tolerances (max |err| <= 2e-2 max |ref|, relative Frobenius <= 5e-3).
Small shapes compare every output; full shapes compare all index arrays and
a seeded sample of tokens (tokens are independent)."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import assert_close, dev16, host16, say, to_f64

pytestmark = pytest.mark.gpu


def _inputs_dev(d):
    return dict(x=dev16(d["x"]), wg=dev16(d["wg"]), wu=dev16(d["wu"]), wd=dev16(d["wd"]))


def _routing(d):
    if "logits" in d:
        return oracle.route(d["logits"], d["k"])
    return d["topk_idx"], d["topk_w"]


def _run_layer(d, D, combine="gather"):
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    ws = moe.layer_workspace(T, H, E, k, I)
    if "logits" in d:
        out = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, logits=torch.from_numpy(d["logits"]).cuda(),
                        workspace=ws, combine=combine)
    else:
        out = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=torch.from_numpy(d["topk_idx"]).cuda(),
                        topk_w=torch.from_numpy(d["topk_w"]).cuda(), workspace=ws, combine=combine)
    torch.cuda.synchronize()
    return out, ws


def _check_layer(d, tokens=None, what="", combine="gather"):
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    say("layer", what, combine, dict(T=T, H=H, E=E, k=k, I=I))
    D = _inputs_dev(d)
    out, ws = _run_layer(d, D, combine)
    idx, w = _routing(d)
    # routing and permutation inside the layer: bit-exact
    view = lambda n: moe.workspace_view(ws, T, H, E, k, I, n).cpu().numpy()
    if "logits" in d:
        assert np.array_equal(view("topk_idx"), idx), what
        assert np.max(np.abs(view("topk_w") - w) / w) <= 1e-6
    P = oracle.permute(idx, E)
    for n_ws, n_or in [("expert_counts", "counts"), ("expert_offsets", "offsets"),
                       ("pair_to_row", "pair_to_row"), ("row_to_pair", "row_to_pair"),
                       ("block_expert", "block_expert")]:
        assert np.array_equal(view(n_ws), P[n_or]), "%s %s" % (what, n_ws)
    assert int(view("num_padded_rows")[0]) == P["m_pad"]
    # values: the layer's definition, token by token
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    ref = oracle.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"], tokens=tokens)
    got = to_f64(out)[tokens]
    r = assert_close(got, ref, what)
    say("layer", what, "max|err|/max|ref| %.2e  relFro %.2e" % r)
    return out, ws, D


def test_layer_tiny_every_token():
    _check_layer(syn.make_config("tiny"), what="tiny")


def test_layer_tiny_steps_match_layer():
    # the five entry points called one by one give the same bits as moe_layer
    d = syn.make_config("tiny")
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    D = _inputs_dev(d)
    say("layer steps tiny")
    out, ws = _run_layer(d, D)
    idx, w = moe.route(torch.from_numpy(d["logits"]).cuda(), k)
    P = moe.permute(idx, E)
    h = moe.grouped_gemm(D["x"], D["wg"], P.block_expert, P.num_padded_rows, N=I, K=H, cap=P.cap,
                         a_src_row=P.row_to_pair, a_src_div=k, B2=D["wu"], epilogue="silu_mul")
    y = moe.grouped_gemm(h, D["wd"], P.block_expert, P.num_padded_rows, N=H, K=I, cap=P.cap)
    out2 = moe.combine(y, P.pair_to_row, w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    # intermediate h against the oracle's gate/up GEMM (real rows)
    Po = oracle.permute(idx.cpu().numpy(), E)
    href = oracle.grouped_gemm(d["x"], d["wg"], Po["block_expert"], N=I, K=H, a_src_row=Po["row_to_pair"],
                               a_src_div=k, B2_bits=d["wu"], epilogue="silu_mul", M=Po["m_pad"])
    real = Po["row_to_pair"][:Po["m_pad"]] >= 0
    # only the real rows leave the device: padding rows of h are never written
    h_real = h[:Po["m_pad"]][torch.from_numpy(real).cuda()]
    assert_close(to_f64(h_real), href[real], "h")
    # combine against the oracle's combine of the GPU's own y (only the reduction differs)
    cref = oracle.combine(host16(y), Po["pair_to_row"], w.cpu().numpy())
    assert_close(to_f64(out2), cref, "combine", max_frac=8e-3, rel_fro=3e-3)


def test_layer_deterministic_and_linear():
    d = syn.make_config("tiny")
    D = _inputs_dev(d)
    say("layer determinism")
    o1, _ = _run_layer(d, D)
    o2, _ = _run_layer(d, D)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # scaling the down weights by 2 scales every output by 2, bit for bit
    D2 = dict(D)
    D2["wd"] = (D["wd"].float() * 2).to(torch.bfloat16)
    o3, _ = _run_layer(d, D2)
    assert torch.equal((o1.float() * 2).to(torch.bfloat16).view(torch.int16), o3.view(torch.int16))


def test_layer_small_shapes():
    # ragged experts, several tiles, K slices below the ring depth, E = 1
    for (T, H, E, k, I, seed) in [(300, 128, 6, 2, 192, 1), (97, 256, 16, 4, 64, 2), (130, 64, 1, 1, 128, 3),
                                  (40, 512, 3, 3, 256, 4)]:
        d = syn.make_moe(T, H, E, k, I, seed=seed)
        _check_layer(d, what="small T%d H%d E%d k%d I%d" % (T, H, E, k, I))


def _degenerate_case(name):
    """Edge shapes of the layer: one token (decode), every pair on the same
    two experts, k = E, and a routing whose every id lies outside [0, E)."""
    if name == "one_token":
        return syn.make_moe(1, 256, 4, 1, 128, seed=21)
    if name == "one_token_tp_slice":
        return syn.make_moe(1, 4096, 64, 4, 512, seed=22, routing="uniform_idx")
    if name == "two_experts":
        d = syn.make_moe(64, 256, 8, 2, 128, seed=23, routing="uniform_idx")
        d["topk_idx"][:, 0], d["topk_idx"][:, 1] = 3, 5
        return d
    if name == "k_equals_E":
        return syn.make_moe(8, 128, 3, 3, 64, seed=24)
    if name == "all_invalid":
        d = syn.make_moe(16, 128, 4, 2, 128, seed=25, routing="uniform_idx")
        d["topk_idx"][:] = -1
        d["topk_idx"][::3, 1] = 4  # == E: also outside
        return d
    raise ValueError(name)


@pytest.mark.parametrize("name", ["one_token", "one_token_tp_slice", "two_experts", "k_equals_E", "all_invalid"])
def test_layer_degenerate_cases(name):
    # every token against the oracle with both combines, the permutation as
    # its own launch, and split K (a pair outside [0, E) adds nothing: it
    # enters the oracle with weight 0)
    d = _degenerate_case(name)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    idx, w = _routing(d)
    bad = (idx < 0) | (idx >= E)
    ref = oracle.moe_tokens(d["x"], np.where(bad, 0, idx).astype(np.int32), np.where(bad, 0, w).astype(np.float32),
                            d["wg"], d["wu"], d["wd"], tokens=np.arange(T, dtype=np.int32))
    D = _inputs_dev(d)
    kw = dict(logits=torch.from_numpy(d["logits"]).cuda()) if "logits" in d else dict(
        topk_idx=torch.from_numpy(d["topk_idx"]).cuda(), topk_w=torch.from_numpy(d["topk_w"]).cuda())
    for combine, sep, split in (("gather", False, False), ("scatter", False, False), ("gather", True, False),
                                ("gather", False, True)):
        say("layer degenerate", name, combine, "separate" if sep else "", "split" if split else "")
        ws = torch.full((moe.layer_workspace(T, H, E, k, I).numel(),), 0x7F, dtype=torch.uint8, device="cuda")
        out = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, workspace=ws, combine=combine, separate_permute=sep,
                        split_k=split, **kw)
        torch.cuda.synchronize()
        if name == "all_invalid":
            assert not torch.any(out.float() != 0), combine
            assert int(moe.workspace_view(ws, T, H, E, k, I, "num_padded_rows")[0]) == 0
        else:
            assert_close(to_f64(out), ref, "%s %s" % (name, combine))


def _sample(T, n, seed=0):
    s = np.random.default_rng(seed).choice(T, n, replace=False)
    return np.sort(np.concatenate([s, [0, T - 1]])).astype(np.int32)


def _check_h_rows_per_block(d, ws, what):
    """One real row of every 128-row block of the layer's h (its gate/up
    GEMM with SiLU*up, in the workspace) against the oracle's grouped GEMM on
    the oracle's own permutation (bit-exact with the layer's, checked
    before): every row task of the persistent schedule is sampled."""
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    idx, _ = _routing(d)
    P = oracle.permute(idx, E)
    r2p, m_pad = P["row_to_pair"], P["m_pad"]
    rows = []
    for b in range(m_pad // 128):
        real = np.nonzero(r2p[b * 128:(b + 1) * 128] >= 0)[0]
        rows.append(b * 128 + real[(b * 37) % len(real)])
    rows = np.array(rows, np.int32)
    h = moe.workspace_view(ws, T, H, E, k, I, "h")
    got = to_f64(h[torch.from_numpy(rows).long().cuda()])
    ref = oracle.grouped_gemm(d["x"], d["wg"], P["block_expert"], N=I, K=H, a_src_row=r2p, a_src_div=k,
                              B2_bits=d["wu"], epilogue="silu_mul", rows=rows)
    r = assert_close(got, ref, what + " h rows")
    say("layer", what, "h: %d rows (one per block) max|err|/max|ref| %.2e  relFro %.2e" % ((len(rows),) + r))


@pytest.mark.parametrize("name,n", [("tp_share", 96), ("ep_skew", 96), ("ep_skew_small", 128), ("prefill", 40)])
def test_layer_full_size(name, n):
    d = syn.make_config(name)
    _, ws, _ = _check_layer(d, tokens=_sample(d["T"], min(n, d["T"] - 2)), what=name)
    _check_h_rows_per_block(d, ws, name)


# ---------------------------------------------------------------- weighted-scatter combine

def test_layer_scatter_tiny_every_token():
    out, _, _ = _check_layer(syn.make_config("tiny"), what="tiny", combine="scatter")


def test_layer_scatter_small_shapes_and_gather_agree():
    for (T, H, E, k, I, seed) in [(300, 128, 6, 2, 192, 1), (130, 64, 1, 1, 128, 3), (40, 512, 3, 3, 256, 4)]:
        d = syn.make_moe(T, H, E, k, I, seed=seed)
        out_s, _, D = _check_layer(d, what="scatter small T%d E%d k%d" % (T, E, k), combine="scatter")
        out_g, _ = _run_layer(d, D, "gather")
        # the two combines differ only in y's bf16 rounding and the fp32 sum order
        assert_close(to_f64(out_s), to_f64(out_g), "scatter vs gather", max_frac=1e-2, rel_fro=4e-3)


@pytest.mark.parametrize("name,n", [("tp_share", 96), ("ep_skew", 96), ("prefill", 24)])
def test_layer_scatter_full_size(name, n):
    d = syn.make_config(name)
    _check_layer(d, tokens=_sample(d["T"], min(n, d["T"] - 2)), what=name, combine="scatter")


@pytest.mark.parametrize("name", ["tiny", "tp_share", "ep_skew"])
def test_layer_packed_gate_up_same_bits(name):
    # the layer on pack_gate_up weights (w_up=None) gives the same bits as on
    # the separate gate and up weights, with both combines
    d = syn.make_config(name)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    D = _inputs_dev(d)
    say("layer packed gate/up", name)
    wgu = moe.pack_gate_up(D["wg"], D["wu"])
    kw = dict(logits=torch.from_numpy(d["logits"]).cuda()) if "logits" in d else dict(
        topk_idx=torch.from_numpy(d["topk_idx"]).cuda(), topk_w=torch.from_numpy(d["topk_w"]).cuda())
    for combine in ("gather", "scatter"):
        a = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, combine=combine, **kw)
        b = moe.layer(D["x"], wgu, None, D["wd"], k, combine=combine, **kw)
        torch.cuda.synchronize()
        if combine == "gather":
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        else:  # the scatter's fp32 atomics sum a token's slots in no fixed order
            assert_close(to_f64(b), to_f64(a), name + " scatter", max_frac=1e-2, rel_fro=2e-3)


@pytest.mark.parametrize("combine", ["gather", "scatter", "router"])
def test_layer_hip_graph_replays(combine):
    # the whole layer captured in one HIP graph (it launches kernels only: no
    # memset node, no host synchronization, no allocation inside) replays to
    # the eager result on every replay, with eager work and synchronizations
    # between the replays
    d = syn.make_config("tiny")
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    D = _inputs_dev(d)
    wgu = moe.pack_gate_up(D["wg"], D["wu"])
    logits = torch.from_numpy(d["logits"]).cuda()
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    say("layer graph", combine)
    if combine == "router":
        # the router front end inside the graph (its expert counts cleared and
        # added by the replayed kernels themselves)
        wr = dev16(syn.bf16_bits((np.random.default_rng(3).standard_normal((E, H)) / np.sqrt(H))
                                 .astype(np.float32)))
        ws = torch.empty(moe.load_library().moe_layer_router_workspace_size(T, H, E, k, I, 0), dtype=torch.uint8,
                         device="cuda")
        run = lambda o=None: moe.layer_router(D["x"], wr, wgu, None, D["wd"], k, workspace=ws, out=o)
    else:
        ws = moe.layer_workspace(T, H, E, k, I)
        run = lambda o=None: moe.layer(D["x"], wgu, None, D["wd"], k, logits=logits, workspace=ws, out=o,
                                       combine=combine)
    eager = run().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the path on the capture stream
        run(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(4):
        out.fill_(float("nan"))
        ws[:4096].zero_()  # eager work on the buffers the graph reads and writes
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if combine != "scatter":
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
        else:
            assert_close(to_f64(out), to_f64(eager), "graph scatter %d" % rep, max_frac=1e-2, rel_fro=2e-3)


# ---------------------------------------------------------------- the fused front end

def _fused_case(name):
    if name in syn.CONFIGS:
        return syn.make_config(name)
    T, H, E, k, I, seed = name
    d = syn.make_moe(T, H, E, k, I, seed=seed, routing="uniform_idx")
    # a few pairs routed outside [0, E): they get no row and add nothing
    d["topk_idx"][::37, 0] = -1
    d["topk_idx"][5, k - 1] = E + 3
    return d


@pytest.mark.parametrize("name", ["tiny", "tp_share", "ep_skew", "ep_skew_small", (130, 64, 1, 1, 128, 3),
                                  (40, 512, 3, 3, 256, 4), (1000, 256, 256, 8, 256, 5)],
                         ids=lambda n: n if isinstance(n, str) else "T%d_H%d_E%d_k%d_I%d" % n[:5])
def test_fused_front_end_same_bits(name):
    # the reorder by route inside the gate/up GEMM's prologue against the
    # separate permutation launch: the same permutation (every index array of
    # the workspace, including the plan the down GEMM runs on), the same h on
    # every real row, the same output bits
    d = _fused_case(name)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    D = _inputs_dev(d)
    wgu = moe.pack_gate_up(D["wg"], D["wu"])
    kw = dict(logits=torch.from_numpy(d["logits"]).cuda()) if "logits" in d else dict(
        topk_idx=torch.from_numpy(d["topk_idx"]).cuda(), topk_w=torch.from_numpy(d["topk_w"]).cuda())
    say("fused front end", name)
    res = []
    for sep in (False, True):
        ws = torch.full((moe.layer_workspace(T, H, E, k, I).numel(),), 0x7F, dtype=torch.uint8, device="cuda")
        out = moe.layer(D["x"], wgu, None, D["wd"], k, workspace=ws, separate_permute=sep, **kw)
        torch.cuda.synchronize()
        res.append((out, ws))
    (o1, w1), (o2, w2) = res
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    view = lambda ws, n: moe.workspace_view(ws, T, H, E, k, I, n)
    for n in ["topk_idx", "expert_counts", "expert_offsets", "pair_to_row", "row_to_pair", "block_expert",
              "num_padded_rows"]:
        assert torch.equal(view(w1, n), view(w2, n)), n
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    plan = lambda ws: ws[lay["gemm_scratch"]:lay["gemm_scratch"] + 8].view(torch.int32)
    nrt = int(plan(w2)[0])
    n = 4 * (2 + 2 * nrt)
    assert torch.equal(w1[lay["gemm_scratch"]:lay["gemm_scratch"] + n], w2[lay["gemm_scratch"]:lay["gemm_scratch"] + n])
    m_pad = int(view(w1, "num_padded_rows")[0])
    real = view(w1, "row_to_pair")[:m_pad] >= 0
    h1, h2 = view(w1, "h")[:m_pad][real], view(w2, "h")[:m_pad][real]
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    if "logits" not in d:
        # the given routing with ids outside [0, E): their pairs get no row
        flat = d["topk_idx"].ravel()
        bad = (flat < 0) | (flat >= E)
        assert np.all(view(w1, "pair_to_row").cpu().numpy()[bad] == -1)
