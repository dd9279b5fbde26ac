"""Bit-exact grouped GEMM on the persistent path where each workgroup runs
many tasks one after another.

With one workgroup per compute unit, small shapes give each workgroup at
most one task, so the task switches inside the A and weight DMA streams, the
wrap-around of the per-task table and plan rings, the weight stream running
onto a later task than the A stream, and the short-K waits (K = 64: two
slices per task) run only at production sizes.  These tests reach them two
ways: a test-only grid size (grouped_gemm_tuned) that gives small shapes
many tasks per workgroup, and the production shapes themselves at the
default grid (the tp_share down GEMM runs 4 tasks per workgroup, the
prefill GEMMs 24-33).

The data is integer (entries in {-1, 0, +1}, sparse enough that every
product stays small): every fp32 partial sum is exact in any order, and the
stored bf16 / fp16 value is exact, so STORE and WEIGHTED_SCATTER results
must equal the oracle's bit for bit; a dropped, repeated or misplaced
32-deep k slice changes an integer and shows.  SiLU*up is held to one
rounding: gate and up are exact integers, so the result must lie within
half a bf16 unit (plus the fp32 error of exp and the reciprocal) of the
oracle's exact value."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import dev16, say, to_f64

pytestmark = pytest.mark.gpu

# |got - exact| bound for SiLU(g) * u with integer g, u: half a bf16 unit
# (2^-8 relative) plus the fp32 error of the epilogue's exp and reciprocal
# (a few 1e-6 relative for |g| < 80)
SILU_REL = 2.0 ** -8 + 2.0 ** -14


def row_tasks(bg, num_rows, cap):
    """Row tasks of the plan, by its definition: inside each maximal run of
    blocks with one non-negative group, blocks pair up from the run's first
    block (an odd run ends in a one-block task)."""
    nblk = max(0, min(num_rows, cap)) // 128
    n, b = 0, 0
    while b < nblk:
        g = int(bg[b])
        e = b + 1
        while e < nblk and bg[e] == g:
            e += 1
        if g >= 0:
            n += (e - b + 1) // 2
        b = e
    return n


def items_per_workgroup(ntask, grid):
    """Tasks each workgroup runs: the task list is cut into 8 contiguous
    ranges, one per XCD, when the grid is a multiple of 8, else one range;
    workgroup w takes every S-th task of its range from its slot on."""
    nx = 8 if grid % 8 == 0 else 1
    S = grid // nx
    out = []
    for w in range(grid):
        xcd, slot = w % nx, w // nx
        t0, t1 = ntask * xcd // nx, ntask * (xcd + 1) // nx
        out.append((t1 - t0 - slot + S - 1) // S if t1 - t0 > slot else 0)
    return out


def assert_silu_exact(got, ref, what):
    assert np.all(np.isfinite(got)), what
    bad = np.abs(got - ref) > SILU_REL * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements off, first at %s: got %r, exact %r"
                             % (what, int(bad.sum()), tuple(i), got[tuple(i)], ref[tuple(i)]))


def one_row_per_block(row_to_pair, m_pad, seed=0):
    """One real row (row_to_pair >= 0) of every 128-row block below M_pad, at
    a position that varies from block to block."""
    rows = []
    for b in range(m_pad // 128):
        real = np.nonzero(row_to_pair[b * 128:(b + 1) * 128] >= 0)[0]
        if len(real):
            rows.append(b * 128 + real[(b * 37 + seed) % len(real)])
    return np.array(rows, np.int32)


# ---------------------------------------------------------------- small shapes, small grid

# a ragged group table: runs of odd and even length, a group that comes back,
# a block without a group inside and one at the end
GROUPS = np.array([0, 0, 0, 1, 1, 4, 2, 2, 2, 2, 2, -1, 3, 3, 0, 0, 0, 0, 4, 4, 4, 1, 1, 1,
                   2, 3, 3, 3, -1], np.int32)
G = 5


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def _small_case(K, N, seed, dtype, layout="kn", gather=True, epi="store"):
    nblk = len(GROUPS)
    cap = (nblk + 1) * 128
    bg = np.concatenate([GROUPS, [-1]]).astype(np.int32)
    T = 900
    A = syn.sparse_ternary_bits((T if gather else cap, K), seed, 0.5, dtype)
    shape = (G, K, N) if layout != "nk" else (G, N, K)
    B = syn.sparse_ternary_bits(shape, seed + 1, 0.5, dtype)
    B2 = syn.sparse_ternary_bits(shape, seed + 2, 0.5, dtype) if epi == "silu_mul" else None
    src = None
    if gather:
        g = np.random.default_rng(seed)
        src = g.integers(0, 2 * T, size=cap).astype(np.int32)
        src[g.random(cap) < 0.15] = -1
    return dict(A=A, B=B, B2=B2, bg=bg, cap=cap, m_rows=nblk * 128, src=src, K=K, N=N)


def _run_small(c, *, dtype, layout, epi, tile, grid):
    tdt = _tdt(dtype)
    out = torch.full((c["cap"], c["N"]), float("nan"), dtype=tdt, device="cuda")
    Bt = dev16(c["B"], tdt)
    B2t = None if c["B2"] is None else dev16(c["B2"], tdt)
    if layout == "kn_gate_up":
        Bt, B2t = moe.pack_gate_up(Bt, B2t), None
    D = moe.grouped_gemm(dev16(c["A"], tdt), Bt, torch.from_numpy(c["bg"]).cuda(),
                         torch.tensor([c["m_rows"]], dtype=torch.int32, device="cuda"), N=c["N"], K=c["K"],
                         cap=c["cap"], a_src_row=None if c["src"] is None else torch.from_numpy(c["src"]).cuda(),
                         a_src_div=2, B2=B2t, b_layout=layout, epilogue=epi, out=out, tile=tile, grid=grid)
    torch.cuda.synchronize()
    return to_f64(D)


def _oracle_small(c, *, dtype, layout, epi):
    return oracle.grouped_gemm(c["A"], c["B"], c["bg"], N=c["N"], K=c["K"], is_fp16=dtype == "fp16",
                               b_layout="nk" if layout == "nk" else "kn", a_src_row=c["src"], a_src_div=2,
                               B2_bits=c["B2"], epilogue=epi, M=c["cap"] if c["src"] is not None else None,
                               rows=np.arange(c["m_rows"], dtype=np.int32))


def _real_rows(c):
    real = np.repeat(c["bg"][:c["m_rows"] // 128], 128) >= 0
    if c["src"] is not None:
        real &= c["src"][:c["m_rows"]] >= 0
    return real


def _items(c, bn, grid):
    ntask = row_tasks(c["bg"], c["m_rows"], c["cap"]) * (c["N"] // bn)
    return items_per_workgroup(ntask, grid)


# (tile, K): every instantiated store tile, with K from 64 (two slices per
# task: the short-K waits of the 4-deep rings) up; the 3/6 and 3/10 rings
# run the weight stream 3 or 7 slices ahead of the A stream, onto later tasks
STORE_TILES = [((256, 32, 3, 6, 1, 8), 128), ((256, 32, 3, 6, 1, 8), 320),
               ((256, 32, 3, 6, 1, 4), 192), ((256, 32, 4, 4, 1, 4), 64),
               ((256, 32, 4, 4, 2, 4), 128), ((128, 32, 3, 10, 1, 4), 320),
               ((128, 32, 4, 4, 3, 4), 64), ((64, 32, 4, 8, 1, 4), 128), ((64, 32, 4, 4, 1, 4), 64)]


@pytest.mark.parametrize("grid", [3, 8])
@pytest.mark.parametrize("tile,K", STORE_TILES, ids=["%s-K%d" % (",".join(map(str, t)), k) for t, k in STORE_TILES])
def test_store_many_items_per_workgroup(tile, K, grid):
    c = _small_case(K, 512, 100 + K + tile[0], "bf16")
    items = _items(c, tile[0], grid)
    assert max(items) >= 5 and min(items) >= 1, items
    say("gemm many items store", tile, "K", K, "grid", grid, "items", max(items))
    got = _run_small(c, dtype="bf16", layout="kn", epi="store", tile=tile, grid=grid)
    ref = _oracle_small(c, dtype="bf16", layout="kn", epi="store")
    real = _real_rows(c)
    assert np.abs(ref[real]).max() <= 256
    assert np.array_equal(got[:c["m_rows"]][real], ref[real])
    assert np.all(np.isnan(got[:c["m_rows"]][~real]))   # padding and group-less blocks: not written
    assert np.all(np.isnan(got[c["m_rows"]:]))          # rows past num_rows: not written


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("K", [64, 320])
def test_store_many_items_dtypes_layouts(dtype, layout, K):
    # the default tile of each shape (K = 64 falls back to the 4-deep rings),
    # identity A rows, on 8 workgroups: one per XCD range
    c = _small_case(K, 768, 200 + K, dtype, layout=layout, gather=False)
    items = _items(c, 256, 8)
    assert max(items) >= 5, items
    say("gemm many items store", dtype, layout, "K", K)
    got = _run_small(c, dtype=dtype, layout=layout, epi="store", tile=None, grid=8)
    ref = _oracle_small(c, dtype=dtype, layout=layout, epi="store")
    real = _real_rows(c)
    assert np.array_equal(got[:c["m_rows"]][real], ref[real])
    assert np.all(np.isnan(got[:c["m_rows"]][~real]))


SILU_TILES = [(None, 128), ((128, 32, 3, 6, 1, 8), 320), ((128, 32, 3, 4, 1, 8), 64),
              ((128, 32, 3, 4, 1, 8), 320), ((128, 32, 3, 6, 1, 4), 128),
              ((128, 32, 4, 4, 1, 4), 64), ((128, 32, 4, 4, 2, 4), 128), ((64, 32, 3, 10, 1, 4), 320),
              ((64, 32, 4, 4, 1, 4), 64)]


@pytest.mark.parametrize("layout", ["kn", "kn_gate_up", "nk"])
@pytest.mark.parametrize("tile,K", SILU_TILES, ids=["%s-K%d" % (t and ",".join(map(str, t)), k) for t, k in SILU_TILES])
def test_silu_mul_many_items_per_workgroup(layout, tile, K):
    grid = 5
    c = _small_case(K, 384, 300 + K, "bf16", layout=layout, epi="silu_mul")
    items = _items(c, tile[0] if tile else 128, grid)
    assert max(items) >= 5, items
    say("gemm many items silu", layout, tile, "K", K, "items", max(items))
    got = _run_small(c, dtype="bf16", layout=layout, epi="silu_mul", tile=tile, grid=grid)
    ref = _oracle_small(c, dtype="bf16", layout=layout, epi="silu_mul")
    real = _real_rows(c)
    assert_silu_exact(got[:c["m_rows"]][real], ref[real], "silu many items")
    assert np.all(np.isnan(got[:c["m_rows"]][~real]))
    assert np.all(np.isnan(got[c["m_rows"]:]))


def _scatter_case(T, k, E, K, N, seed, dtype="bf16"):
    g = np.random.default_rng(seed)
    idx, _ = oracle.route(g.standard_normal((T, E)).astype(np.float32), k)
    P = oracle.permute(idx, E)
    A = syn.sparse_ternary_bits((P["cap"], K), seed + 1, 0.5, dtype)
    B = syn.sparse_ternary_bits((E, K, N), seed + 2, 0.5, dtype)
    w = g.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), size=(T, k))
    return P, A, B, w


SCATTER_TILES = [(None, 256), ((256, 32, 4, 4, 1, 4), 64), ((128, 32, 3, 10, 1, 4), 320),
                 ((64, 32, 4, 8, 2, 4), 128)]


@pytest.mark.parametrize("grid", [3, 8])
@pytest.mark.parametrize("tile,K", SCATTER_TILES, ids=["%s-K%d" % (t and ",".join(map(str, t)), k) for t, k in SCATTER_TILES])
def test_weighted_scatter_many_items_per_workgroup(tile, K, grid):
    T, k, E, N = 700, 3, 6, 1024
    P, A, B, w = _scatter_case(T, k, E, K, N, seed=400 + K)
    bn = tile[0] if tile else 256
    items = items_per_workgroup(row_tasks(P["block_expert"], P["m_pad"], P["cap"]) * (N // bn), grid)
    assert max(items) >= 5, items
    say("gemm many items scatter", tile, "K", K, "grid", grid, "items", max(items))
    got = moe.grouped_gemm(dev16(A), dev16(B), torch.from_numpy(P["block_expert"]).cuda(),
                           torch.tensor([P["m_pad"]], dtype=torch.int32, device="cuda"), N=N, K=K,
                           cap=P["cap"], epilogue="weighted_scatter",
                           row_pair=torch.from_numpy(P["row_to_pair"]).cuda(),
                           pair_w=torch.from_numpy(w).cuda(), tile=tile, grid=grid)
    torch.cuda.synchronize()
    Y = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K)
    ref = oracle.weighted_scatter(Y, P["row_to_pair"], w, k, T)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), ref)


# ---------------------------------------------------------------- production shapes, default grid

def _routing_maps(name):
    d = syn.make_config(name, with_weights=False)
    if "logits" in d:
        idx, w = oracle.route(d["logits"], d["k"])
    else:
        idx, w = d["topk_idx"], d["topk_w"]
    return d, idx, oracle.permute(idx, d["E"])


def _num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("epi", ["store", "weighted_scatter"])
def test_tp_share_down_shape(epi):
    # the down GEMM of the tp_share layer (N = 4096, K = 512, its block
    # experts and row map, weights streamed as the layer streams them):
    # 4 tasks per workgroup; one row of every 128-row block checked in full
    d, idx, P = _routing_maps("tp_share")
    T, E, k, H, I = d["T"], d["E"], d["k"], d["H"], d["I"]
    cap, m_pad, r2p = P["cap"], P["m_pad"], P["row_to_pair"]
    bn = 256
    items = items_per_workgroup(row_tasks(P["block_expert"], m_pad, cap) * (H // bn), _num_cus())
    assert max(items) >= 4, max(items)
    A = syn.sparse_ternary_bits((cap, I), 501, 0.5)
    B = syn.sparse_ternary_bits((E, I, H), 502, 0.5)
    say("tp_share down shape", epi, "items", max(items))
    At, Bt = dev16(A), dev16(B)
    bexp = torch.from_numpy(P["block_expert"]).cuda()
    mpad = torch.tensor([m_pad], dtype=torch.int32, device="cuda")
    r2pt = torch.from_numpy(r2p).cuda()
    rows = one_row_per_block(r2p, m_pad)
    if epi == "store":
        out = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        D = moe.grouped_gemm(At, Bt, bexp, mpad, N=H, K=I, cap=cap, row_pair=r2pt, out=out, b_stream=True)
        torch.cuda.synchronize()
        ref = oracle.grouped_gemm(A, B, P["block_expert"], N=H, K=I, rows=rows)
        assert np.abs(ref).max() <= 256
        assert np.array_equal(to_f64(D)[rows], ref)
        pad = np.nonzero(r2p[:m_pad] < 0)[0]
        assert torch.isnan(D[torch.from_numpy(pad).cuda()]).all()   # padding rows not written
    else:
        w = np.random.default_rng(503).choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), size=(T, k))
        got = moe.grouped_gemm(At, Bt, bexp, mpad, N=H, K=I, cap=cap, epilogue="weighted_scatter",
                               row_pair=r2pt, pair_w=torch.from_numpy(w).cuda(), b_stream=True)
        torch.cuda.synchronize()
        # the tokens of one row of every block, with all k of their rows
        toks = np.unique(r2p[rows] // k)
        pair_rows = P["pair_to_row"].reshape(T, k)[toks].ravel().astype(np.int32)
        Y = oracle.grouped_gemm(A, B, P["block_expert"], N=H, K=I, rows=pair_rows)
        sub_r2p = np.arange(len(pair_rows), dtype=np.int32)          # row i of Y is pair i of the sample
        ref = oracle.weighted_scatter(Y, sub_r2p, w[toks].ravel(), k, len(toks))
        assert np.array_equal(got.cpu().numpy().astype(np.float64)[toks], ref)


def test_prefill_gate_up_shape():
    # the gate/up GEMM of the prefill layer (N = 1536, K = 4096, gate and up
    # interleaved as the layer takes them, A rows gathered through the row
    # map): 24-25 tasks per workgroup; one row of every 128-row block
    d, idx, P = _routing_maps("prefill")
    T, E, k, H, I = d["T"], d["E"], d["k"], d["H"], d["I"]
    cap, m_pad, r2p = P["cap"], P["m_pad"], P["row_to_pair"]
    items = items_per_workgroup(row_tasks(P["block_expert"], m_pad, cap) * (I // 128), _num_cus())
    assert max(items) >= 20, max(items)
    x = syn.sparse_ternary_bits((T, H), 601, 0.15)
    wg = syn.sparse_ternary_bits((E, H, I), 602, 0.15)
    wu = syn.sparse_ternary_bits((E, H, I), 603, 0.15)
    say("prefill gate/up shape", "items", max(items))
    wgu = moe.pack_gate_up(dev16(wg), dev16(wu))
    out = torch.full((cap, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    h = moe.grouped_gemm(dev16(x), wgu, torch.from_numpy(P["block_expert"]).cuda(),
                         torch.tensor([m_pad], dtype=torch.int32, device="cuda"), N=I, K=H, cap=cap,
                         a_src_row=torch.from_numpy(r2p).cuda(), a_src_div=k, b_layout="kn_gate_up",
                         epilogue="silu_mul", out=out)
    torch.cuda.synchronize()
    del wgu
    rows = one_row_per_block(r2p, m_pad)
    ref = oracle.grouped_gemm(x, wg, P["block_expert"], N=I, K=H, a_src_row=r2p, a_src_div=k, B2_bits=wu,
                              epilogue="silu_mul", rows=rows)
    assert_silu_exact(to_f64(h[torch.from_numpy(rows).long().cuda()]), ref, "prefill gate/up")
    pad = np.nonzero(r2p[:m_pad] < 0)[0]
    assert torch.isnan(h[torch.from_numpy(pad).cuda()]).all()


def test_prefill_down_shape():
    # the down GEMM of the prefill layer (N = 4096, K = 1536): 33 tasks per
    # workgroup; one row of every 128-row block
    d, idx, P = _routing_maps("prefill")
    E, H, I = d["E"], d["H"], d["I"]
    cap, m_pad, r2p = P["cap"], P["m_pad"], P["row_to_pair"]
    items = items_per_workgroup(row_tasks(P["block_expert"], m_pad, cap) * (H // 256), _num_cus())
    assert max(items) >= 30, max(items)
    A = syn.sparse_ternary_bits((cap, I), 701, 0.3)
    B = syn.sparse_ternary_bits((E, I, H), 702, 0.3)
    say("prefill down shape", "items", max(items))
    out = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    D = moe.grouped_gemm(dev16(A), dev16(B), torch.from_numpy(P["block_expert"]).cuda(),
                         torch.tensor([m_pad], dtype=torch.int32, device="cuda"), N=H, K=I, cap=cap,
                         row_pair=torch.from_numpy(r2p).cuda(), out=out)
    torch.cuda.synchronize()
    rows = one_row_per_block(r2p, m_pad)
    ref = oracle.grouped_gemm(A, B, P["block_expert"], N=H, K=I, rows=rows)
    assert np.abs(ref).max() <= 256
    assert np.array_equal(to_f64(D[torch.from_numpy(rows).long().cuda()]), ref)
