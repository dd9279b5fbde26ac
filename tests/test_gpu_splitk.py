"""GPU checks of the layer's split-K form (MOE_LAYER_SPLIT_K, split_k=True).
A GEMM of the layer that may have at most one wave of (row task, column
block) tasks ("Comm-compute fusion (1)", section 5: below one wave the
compute units stand idle) is launched in its split-K form; it counts the
routed row tasks on the device and, where they leave at least a quarter of
the CUs idle, runs each task's k range in 2 or 4 parts whose fp32 partial
sums a reduction adds in a fixed order (SiLU*up after gate/up, the top-k
weighted combine after down).

* against the oracle, every token, at the bf16 tolerances of the layer
  (ragged experts, an expert of two 128-row blocks, pairs routed outside
  [0, E), both combines, the router front end, a graph replay);
* on integer-valued inputs chosen so that every sum is exact in fp32 (gate
  columns of one sign and |gate| >= 128, where SiLU is exactly the identity
  or zero; sparse +-1 up and down weights bounding every partial sum below
  2^24), bit for bit against the unsplit path (the entry points called one
  by one): a part missing, doubled or written to the wrong pair or column
  would change an output.  The workspace's y region then holds the down
  GEMM's partials, which must add up to the unsplit y;
* where the routed tasks fill the CUs (ep_skew_small), nothing splits: the
  layer gives the unsplit path's bits on random inputs, with and without the
  flag."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import assert_close, dev16, say, to_f64

pytestmark = pytest.mark.gpu


def _grid():
    """Workgroups of the layer's GEMMs: one per compute unit (256 on MI355X)."""
    return torch.cuda.get_device_properties(0).multi_processor_count


def _max_parts(T, H, E, k, I, N, bn, nb, K):
    """The part bound the layer launches a GEMM with (moe.h): 1 unless the
    most row tasks any routing gives, floor((R + 255 min(E, R)) / 256), times
    the column blocks fit one wave; 4, else 2, parts of >= 16 slices of 32
    whose fp32 partials fit y's workspace region."""
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    room = lay["permute_scratch"] - lay["y"]
    R = T * k
    rt = (R + 255 * min(E, R)) // 256
    if N % bn or rt * (N // bn) > _grid():
        return 1
    for p in (4, 2):
        if K % (32 * p) == 0 and K // 32 // p >= 16 and p * R * nb * N * 4 <= room:
            return p
    return 1


def _device_parts(tasks, max_parts):
    """The part count the GEMM picks on the device (moe.h): 1 unless the tasks
    leave at least a quarter of the workgroups idle; else the count whose
    busiest workgroup (items dealt out per XCD) has the least work, fewer on
    a tie."""
    grid = _grid()
    if tasks <= 0 or 4 * tasks >= 3 * grid:
        return 1
    nx = 8 if grid % 8 == 0 else 1
    S = grid // nx
    items = lambda p: -(-(-(-tasks * p // nx)) // S)
    best = 1
    for p in (2, 4):
        if p <= max_parts and items(p) * best < items(best) * p:
            best = p
    return best


def _row_tasks(idx, E):
    flat = idx.ravel()
    c = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    blocks = -(-c // 128)
    return int((-(-blocks // 2)).sum())


def _parts(d):
    """(gate/up, down) part counts the layer will use with MOE_LAYER_SPLIT_K."""
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    rt = _row_tasks(d["topk_idx"], E)
    gu = _device_parts(rt * (I // 128), _max_parts(T, H, E, k, I, I, 128, 2, H))
    dn = _device_parts(rt * (H // 256), _max_parts(T, H, E, k, I, H, 256, 1, I))
    return gu, dn


def _routing(name, T, E, k, seed):
    """Distinct experts per token with invalid ids here and there:
    'heavy' -- the first 150 tokens all take expert 0 (two 128-row blocks);
    'few' -- tokens dealt round-robin to 8 of the experts;
    'nine' -- tokens dealt round-robin to 9 experts (k == 1)."""
    rng = np.random.default_rng(seed)
    if name == "heavy":
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        for t in range(min(150, T)):
            if 0 in idx[t]:
                j = int(np.nonzero(idx[t] == 0)[0][0])
                idx[t, [0, j]] = idx[t, [j, 0]]
            else:
                idx[t, 0] = 0
    else:
        ex = rng.permutation(E)[:8 if name == "few" else 9]
        idx = np.stack([ex[(np.arange(T) + j) % len(ex)] for j in range(k)], axis=1).astype(np.int32)
    idx[::29, k - 1] = -1
    idx[7, 0] = E + 2
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    return idx, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


# (T, H, E, k, I, routing, seed, expected (gate/up, down) parts):
# both GEMMs in 2 parts (4 would not fit the workspace or leave parts under
# 16 slices), an expert of two blocks; gate/up in 2 and down in 4 parts;
# both in 4 parts with two or three items per workgroup; gate/up in 2 parts
# of an odd 17 slices (H = 1088, whose 64-column down tile has no split form)
CASES = [(160, 2048, 8, 2, 1024, "heavy", 11, (2, 2)), (32, 2048, 16, 1, 2048, "few", 12, (2, 4)),
         (72, 4096, 16, 1, 2048, "nine", 13, (4, 4)), (24, 1088, 8, 2, 1024, "few", 14, (2, 1))]
IDS = ["T%d_H%d_E%d_k%d_I%d" % c[:5] for c in CASES]


def _case(c):
    T, H, E, k, I, routing, seed, _ = c
    d = syn.make_moe(T, H, E, k, I, seed=seed, routing="uniform_idx")
    d["topk_idx"], d["topk_w"] = _routing(routing, T, E, k, seed)
    return d


def _dev(d):
    return {n: dev16(d[n]) for n in ("x", "wg", "wu", "wd")}


def _layer(D, d, split_k=False, combine="gather", ws=None):
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    ws = moe.layer_workspace(T, H, E, k, I) if ws is None else ws
    out = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=torch.from_numpy(d["topk_idx"]).cuda(),
                    topk_w=torch.from_numpy(d["topk_w"]).cuda(), workspace=ws, combine=combine,
                    split_k=split_k)
    torch.cuda.synchronize()
    return out, ws


def _unsplit(D, d):
    """The path through the entry points one by one (no GEMM splits there)."""
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    P = moe.permute(torch.from_numpy(d["topk_idx"]).cuda(), E)
    h = moe.grouped_gemm(D["x"], D["wg"], P.block_expert, P.num_padded_rows, N=I, K=H, cap=P.cap,
                         a_src_row=P.row_to_pair, a_src_div=k, B2=D["wu"], epilogue="silu_mul")
    y = moe.grouped_gemm(h, D["wd"], P.block_expert, P.num_padded_rows, N=H, K=I, cap=P.cap,
                         row_pair=P.row_to_pair)
    out = moe.combine(y, P.pair_to_row, torch.from_numpy(d["topk_w"]).cuda())
    torch.cuda.synchronize()
    return out, h, y, P


def _oracle_out(d, idx, w):
    """The oracle's layer, every token; a pair naming no valid expert adds
    nothing (the layer gives it no row), i.e. it enters with weight 0."""
    bad = (idx < 0) | (idx >= d["E"])
    return oracle.moe_tokens(d["x"], np.where(bad, 0, idx).astype(np.int32),
                             np.where(bad, 0, w).astype(np.float32), d["wg"], d["wu"], d["wd"],
                             tokens=np.arange(d["T"], dtype=np.int32))


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_split_layer_matches_oracle(case):
    d = _case(case)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    assert _parts(d) == case[7]
    say("split K vs oracle", case[:5], "parts gate/up %d down %d" % case[7])
    D = _dev(d)
    ref = _oracle_out(d, d["topk_idx"], d["topk_w"])
    for split_k, combine in ((False, "gather"), (True, "gather"), (True, "scatter")):
        out, ws = _layer(D, d, split_k=split_k, combine=combine)
        r = assert_close(to_f64(out), ref, "split_k=%s %s %s" % (split_k, combine, case[:5]))
        say("split K", split_k, combine, "max|err|/max|ref| %.2e  relFro %.2e" % r)
    # deterministic: the same bits on a second run
    o1, _ = _layer(D, d, split_k=True)
    o2, _ = _layer(D, d, split_k=True)
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


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_split_exact_sums_same_bits_as_unsplit(case):
    T, H, E, k, I, routing, seed, parts = case
    d = dict(T=T, H=H, E=E, k=k, I=I)
    d["topk_idx"], d["topk_w"] = _routing(routing, T, E, k, seed + 10)
    assert _parts(d) == parts
    ks_gu, ks_dn = parts
    say("split K exact", case[:5], "parts gate/up %d down %d" % parts)
    nu, nd = (16, 32) if H > 2048 else (32, 32)  # H % nu == 0 for every case
    D = _integer_inputs(T, H, E, k, I, seed, nu, nd)
    out_n, h_n, y_n, P = _unsplit(D, d)
    out_s, ws_s = _layer(D, d, split_k=True)
    assert torch.isfinite(out_s.float()).all()
    assert torch.equal(out_s.view(torch.int16), out_n.view(torch.int16))
    view = lambda n: moe.workspace_view(ws_s, T, H, E, k, I, n)
    p2r = P.pair_to_row.long()
    ok = p2r >= 0
    rows = p2r[ok]
    assert torch.equal(view("pair_to_row").long(), p2r)
    # h of every pair's row (written by the reduction after the split gate/up)
    assert torch.equal(view("h")[rows].view(torch.int16), h_n[rows].view(torch.int16))
    if ks_dn > 1:
        # the down GEMM's fp32 partials, [parts][pairs][H], in y's region: their
        # sum (exact) rounds to the unsplit y of the pair's row, and no part is empty
        lay = moe.layer_workspace_layout(T, H, E, k, I)
        R = T * k
        part = ws_s[lay["y"]:lay["y"] + ks_dn * R * H * 4].view(torch.float32).view(ks_dn, R, H)
        y_s = part.sum(0)[ok].to(torch.bfloat16)
        assert torch.equal(y_s.view(torch.int16), y_n[rows].view(torch.int16))
        assert all(bool((part[s][ok] != 0).any()) for s in range(ks_dn))
    else:
        # not split: the down GEMM stored y itself
        assert torch.equal(view("y")[rows].view(torch.int16), y_n[rows].view(torch.int16))


def test_no_split_where_tasks_fill_the_cus():
    # ep_skew_small (T=128, 16 experts under Zipf routing, 12 routed, H=4096,
    # I=2048): both GEMMs are launched in the split form (4 parts at most),
    # but 192 tasks each fill 3/4 of the CUs, so neither splits -- the layer
    # gives the unsplit path's bits, with and without the flag
    d = syn.make_config("ep_skew_small")
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    assert _max_parts(T, H, E, k, I, I, 128, 2, H) == 4 and _max_parts(T, H, E, k, I, H, 256, 1, I) == 4
    assert _parts(d) == (1, 1)
    D = _dev(d)
    say("no split ep_skew_small")
    out_n, _, _, _ = _unsplit(D, d)
    for split_k in (False, True):
        out, _ = _layer(D, d, split_k=split_k)
        assert torch.equal(out.view(torch.int16), out_n.view(torch.int16)), split_k
    tokens = np.arange(0, T, 4, dtype=np.int32)
    ref = oracle.moe_tokens(d["x"], d["topk_idx"], d["topk_w"], d["wg"], d["wu"], d["wd"], tokens=tokens)
    assert_close(to_f64(out_n)[tokens], ref, "ep_skew_small")


def test_split_router_front_end():
    # the router front end with a split layer: the same bits as the layer
    # given the router's own routing (both take the separate permutation)
    T, H, E, k, I = 16, 2048, 8, 2, 2048
    d = syn.make_moe(T, H, E, k, I, seed=5, routing="uniform_idx")
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
    d["topk_idx"] = idx.cpu().numpy()
    assert min(_parts(d)) > 1
    out2 = moe.layer(D["x"], D["wg"], D["wu"], D["wd"], k, topk_idx=idx, topk_w=w, split_k=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert_close(to_f64(out), _oracle_out(d, idx.cpu().numpy(), w.cpu().numpy()), "split router")


def test_split_hip_graph_replays():
    # the split layer (GEMMs, the SiLU*up reduction, the combining reduction)
    # captured in one HIP graph replays to the eager bits every time
    d = _case(CASES[1])
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
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
