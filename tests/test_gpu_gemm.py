"""GPU parity of the grouped GEMM with the oracle.

Integer-exact cases (entries in {-1, 0, 1}) must match bit for bit: every
partial sum is a small integer, exact in fp32 in any order, so any row,
column, group or k-slice mapping mistake shows.  Random cases are held to
the bf16 tolerances."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_amd as moe
import oracle
from moe_expert_grouped_amd import synthetic as syn
from _util import assert_close, dev16, host16, say, to_f64

pytestmark = pytest.mark.gpu


def _groups(nblk, G, seed, neg_tail=0):
    g = np.random.default_rng(seed)
    bg = np.sort(g.integers(0, G, size=nblk)).astype(np.int32)
    if neg_tail:
        bg[-neg_tail:] = -1
    return bg


def _tile(spec):
    """"bn,bk,na,nb[,group rows[,wavefronts]]" -> the 6-entry tile of grouped_gemm_tuned."""
    v = [int(x) for x in spec.split(",")]
    return tuple(v + [1, 4][len(v) - 4:])


def _run(A_bits, B_bits, bg, *, N, K, cap, m_rows, dtype, layout="kn", src=None, div=1, B2_bits=None,
         epi="store", tile=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    out = torch.full((cap, N), float("nan"), dtype=tdt, device="cuda")
    D = moe.grouped_gemm(dev16(A_bits, tdt), dev16(B_bits, tdt), torch.from_numpy(bg).cuda(),
                         torch.tensor([m_rows], dtype=torch.int32, device="cuda"), N=N, K=K, cap=cap,
                         a_src_row=None if src is None else torch.from_numpy(src).cuda(), a_src_div=div,
                         B2=None if B2_bits is None else dev16(B2_bits, tdt), b_layout=layout,
                         epilogue=epi, out=out, tile=tile)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("N,K", [(256, 320), (192, 128), (128, 64), (64, 512)])
def test_integer_exact(dtype, layout, N, K):
    G, nblk = 3, 5
    cap = (nblk + 1) * 128
    m_rows = nblk * 128
    bg = _groups(cap // 128, G, N + K, neg_tail=1)
    A = syn.ternary_bits((cap, K), 1, dtype)
    B = syn.ternary_bits((G, K, N) if layout == "kn" else (G, N, K), 2, dtype)
    say("gemm integer", dtype, layout, N, K)
    D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=m_rows, dtype=dtype, layout=layout)
    ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, is_fp16=(dtype == "fp16"), b_layout=layout,
                              rows=np.arange(m_rows, dtype=np.int32))
    got = to_f64(D)
    assert np.array_equal(got[:m_rows], ref)
    assert np.all(np.isnan(got[m_rows:]))  # rows beyond num_rows untouched


def test_integer_exact_gather_and_negative_group():
    # A rows gathered through a permutation with padding; one block without a group
    K, N, G = 256, 128, 4
    T = 300
    A = syn.ternary_bits((T, K), 3)
    B = syn.ternary_bits((G, K, N), 4)
    cap = 6 * 128
    bg = np.array([0, 3, -1, 3, 1, 2], np.int32)
    g = np.random.default_rng(1)
    src = g.integers(0, T * 2, size=cap).astype(np.int32)
    src[g.random(cap) < 0.2] = -1
    say("gemm gather")
    D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=cap, dtype="bf16", src=src, div=2)
    ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, a_src_row=src, a_src_div=2)
    got = to_f64(D)
    real = (src >= 0) & (np.repeat(bg, 128) >= 0)
    assert np.array_equal(got[real], ref[real])
    assert np.all(np.isnan(got[256:384]))  # the block without a group is not written


def test_integer_exact_silu_mul_gate_only_rows():
    # up weights all one-hot so up = one A entry; gate ternary: checks gate/up pairing per column
    K, N, G = 192, 128, 2
    A = syn.ternary_bits((256, K), 5)
    Bg = syn.ternary_bits((G, K, N), 6)
    Bu = syn.ternary_bits((G, K, N), 7)
    bg = np.array([1, 0], np.int32)
    say("gemm silu integer")
    D = _run(A, Bg, bg, N=N, K=K, cap=256, m_rows=256, dtype="bf16", B2_bits=Bu, epi="silu_mul")
    ref = oracle.grouped_gemm(A, Bg, bg, N=N, K=K, B2_bits=Bu, epilogue="silu_mul")
    assert_close(to_f64(D), ref, "silu integer", max_frac=8e-3, rel_fro=4e-3)


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("epi", ["store", "silu_mul"])
def test_random_vs_oracle(layout, epi):
    G, K, N = 5, 448, 320
    cap = 9 * 128
    bg = _groups(9, G, 3)
    g = np.random.default_rng(7)
    A = syn.bf16_bits(g.standard_normal((700, K)).astype(np.float32))
    shape = (G, K, N) if layout == "kn" else (G, N, K)
    B = syn.bf16_bits((g.standard_normal(shape) / np.sqrt(K)).astype(np.float32))
    B2 = syn.bf16_bits((g.standard_normal(shape) / np.sqrt(K)).astype(np.float32)) if epi == "silu_mul" else None
    src = g.integers(-1, 700, size=cap).astype(np.int32)
    say("gemm random", layout, epi)
    D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=cap, dtype="bf16", layout=layout, src=src, div=1,
             B2_bits=B2, epi=epi)
    ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, b_layout=layout, a_src_row=src, B2_bits=B2, epilogue=epi)
    real = src >= 0
    assert_close(to_f64(D)[real], ref[real], "random %s %s" % (layout, epi))


def test_dense_fp16_degenerate_case_sampled():
    # D = A . B^T, 4096^3 fp16, one group: sampled rows against the oracle,
    # and every element against the library GEMM (hipBLASLt via torch)
    d = syn.make_config("dense")
    M = N = K = 4096
    say("dense 4096 fp16")
    A = dev16(d["A"], torch.float16)
    B = dev16(d["B"], torch.float16)
    D = moe.grouped_gemm(A, B, torch.zeros(32, dtype=torch.int32, device="cuda"),
                         torch.tensor([M], dtype=torch.int32, device="cuda"), N=N, K=K, cap=M,
                         b_layout="nk")
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 24, replace=False).astype(np.int32)
    rows = np.concatenate([rows, [0, 127, 128, 4095]]).astype(np.int32)
    ref = oracle.grouped_gemm(d["A"], d["B"].reshape(1, N, K), np.zeros(32, np.int32), N=N, K=K,
                              is_fp16=True, b_layout="nk", rows=rows)
    got = to_f64(D)[rows]
    # fp16 output of values up to ~100: half-ulp 0.03; fp32 accumulation of 4096 terms
    assert np.max(np.abs(got - ref)) <= 0.07
    assert_close(got, ref, "dense sampled")
    lib = (A.float() @ B.float().T)
    assert_close(to_f64(D), lib.double().cpu().numpy(), "dense vs library")


# bn, bk, A ring depth, B ring depth[, super-block row tasks]
TILES = [("store", "256,32,3,6"), ("store", "256,32,4,4,2"), ("store", "128,32,3,10"),
         ("store", "64,32,4,8,3"), ("store", "256,32,3,6,4"), ("store", "256,32,3,6,1,8"),
         ("silu_mul", "128,32,3,6"), ("silu_mul", "128,32,4,4,2"), ("silu_mul", "64,32,3,10"),
         ("silu_mul", "128,32,3,6,3"), ("silu_mul", "128,32,3,6,1,8")]


@pytest.mark.parametrize("epi,tile", TILES, ids=["%s-%s" % t for t in TILES])
def test_tile_configurations_integer_exact(epi, tile):
    # every instantiated tile shape / ring depths / task order gives the
    # exact result; K = 64 and 128 have fewer slices than the B ring has
    # stages: a configuration whose table ring is unsafe for them is refused
    # (MOE_ERR_UNSUPPORTED), never run
    t = _tile(tile)
    G, N = 4, 512
    cap = 11 * 128
    bg = _groups(cap // 128, G, 17)
    for K in (64, 128, 320, 640):
        A = syn.ternary_bits((cap, K), 8)
        B = syn.ternary_bits((G, K, N), 9)
        B2 = syn.ternary_bits((G, K, N), 10) if epi == "silu_mul" else None
        m_rows = 9 * 128
        say("gemm tile", epi, tile, "K", K)
        if 2 * (K // t[1]) < t[3] - 1:
            with pytest.raises(moe.MoeError) as ex:
                _run(A, B, bg, N=N, K=K, cap=cap, m_rows=m_rows, dtype="bf16", B2_bits=B2, epi=epi, tile=t)
            assert ex.value.status == moe.MOE_ERR_UNSUPPORTED
            continue
        D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=m_rows, dtype="bf16", B2_bits=B2, epi=epi, tile=t)
        ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, B2_bits=B2, epilogue=epi,
                                  rows=np.arange(m_rows, dtype=np.int32))
        got = to_f64(D)
        if epi == "store":
            assert np.array_equal(got[:m_rows], ref)
        else:
            assert_close(got[:m_rows], ref, "tile " + tile, max_frac=8e-3, rel_fro=4e-3)
        assert np.all(np.isnan(got[m_rows:]))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_eight_wavefronts_integer_exact(dtype, layout):
    # the eight-wavefront workgroups (two per SIMD, a 128-row x 64-column
    # share of a 256 x 256 task each) on both B layouts, gathered rows, a
    # ragged group table and a block without a group
    G, N, K = 3, 768, 384
    cap = 9 * 128
    bg = np.array([0, 0, 0, 2, -1, 1, 1, 2, 2], np.int32)
    T = 700
    A = syn.ternary_bits((T, K), 31, dtype)
    B = syn.ternary_bits((G, K, N) if layout == "kn" else (G, N, K), 32, dtype)
    src = np.random.default_rng(3).integers(0, T * 2, size=cap).astype(np.int32)
    say("gemm eight wavefronts", dtype, layout)
    D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=cap, dtype=dtype, layout=layout, src=src, div=2,
             tile=(256, 32, 3, 6, 1, 8))
    ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, is_fp16=dtype == "fp16", b_layout=layout,
                              a_src_row=src, a_src_div=2)
    got = to_f64(D)
    real = np.repeat(bg, 128) >= 0
    assert np.array_equal(got[real], ref[real])
    assert np.all(np.isnan(got[~real]))


# block-group patterns for the pairing of blocks into 256-row tasks: runs of
# odd and even length, a group that comes back after another, blocks without
# a group inside and at the ends, one-block runs, a single run
PAIRINGS = [[0, 0, 0, 1, 1, 2, 2, 2, 2, 3],
            [-1, 5, 5, 5, -1, 5, 5, 2, -1, -1],
            [1, 0, 1, 0, 1, 1, 1, 0, 0, 0, 2],
            [3] * 13,
            [2, -1, -1, 4, 4, -1, 0],
            [4, 3, 2, 1, 0]]


@pytest.mark.parametrize("pattern", range(len(PAIRINGS)))
@pytest.mark.parametrize("epi", ["store", "silu_mul"])
def test_block_pairing_integer_exact(pattern, epi):
    bg = np.array(PAIRINGS[pattern], np.int32)
    G, K = 6, 192
    N = 256 if epi == "store" else 128
    nblk = len(bg)
    cap = (nblk + 1) * 128
    bgc = np.concatenate([bg, [-1]]).astype(np.int32)
    A = syn.ternary_bits((cap, K), 40 + pattern)
    B = syn.ternary_bits((G, K, N), 50 + pattern)
    B2 = syn.ternary_bits((G, K, N), 60 + pattern) if epi == "silu_mul" else None
    m_rows = nblk * 128
    say("gemm pairing", epi, PAIRINGS[pattern])
    D = _run(A, B, bgc, N=N, K=K, cap=cap, m_rows=m_rows, dtype="bf16", B2_bits=B2, epi=epi)
    ref = oracle.grouped_gemm(A, B, bgc, N=N, K=K, B2_bits=B2, epilogue=epi,
                              rows=np.arange(m_rows, dtype=np.int32))
    got = to_f64(D)
    real = np.repeat(bg, 128) >= 0
    if epi == "store":
        assert np.array_equal(got[:m_rows][real], ref[real])
    else:
        assert_close(got[:m_rows][real], ref[real], "pairing", max_frac=8e-3, rel_fro=4e-3)
    assert np.all(np.isnan(got[:m_rows][~real]))  # blocks without a group: not written
    assert np.all(np.isnan(got[m_rows:]))          # rows past num_rows: not written


def _plan_by_definition(bg, num_rows, cap):
    """The row-task plan from its definition: inside each maximal run of blocks
    with one non-negative group, blocks pair up from the run's first block (an
    odd run ends in a one-block task); entries in block order."""
    nblk = max(0, min(num_rows, cap)) // 128
    out, b = [], 0
    while b < nblk:
        g = int(bg[b])
        if g < 0:
            b += 1
            continue
        e = b
        while e < nblk and bg[e] == g:
            e += 1
        for s in range(b, e, 2):
            out += [s | ((1 << 30) if s + 1 < e else 0), g]
        b = e
    return np.array([len(out) // 2, nblk] + out, np.int32)


# block counts around the plan kernel's 1024-block chunks, runs of every
# length crossing them, negative groups, row counts past cap and not whole blocks
@pytest.mark.parametrize("nblk,num_rows_extra", [(1, 0), (5, 77), (1023, 0), (1024, 0), (1025, 5),
                                                 (2050, 0), (3000, 1 << 20)])
def test_row_task_plan_matches_definition(nblk, num_rows_extra):
    g = np.random.default_rng(nblk)
    runs, total = [], 0
    while total < nblk:
        n = int(g.integers(1, 8)) if g.random() < 0.9 else int(g.integers(8, 1500))
        grp = -1 if g.random() < 0.15 else int(g.integers(0, 5))
        runs.append(np.full(n, grp, np.int32))
        total += n
    bg = np.concatenate(runs)[:nblk]
    cap = nblk * 128
    num_rows = cap - 64 if num_rows_extra == 77 else cap + num_rows_extra
    K = N = 64
    A = torch.zeros((cap, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((5, K, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(moe.gemm_workspace(cap).numel(), dtype=torch.uint8, device="cuda")
    say("row-task plan", "blocks", nblk, "num_rows", num_rows)
    moe.grouped_gemm(A, B, torch.from_numpy(bg).cuda(),
                     torch.tensor([num_rows], dtype=torch.int32, device="cuda"),
                     N=N, K=K, cap=cap, workspace=ws)
    torch.cuda.synchronize()
    ref = _plan_by_definition(bg, num_rows, cap)
    got = ws[:4 * len(ref)].view(torch.int32).cpu().numpy()
    assert np.array_equal(got, ref)


def test_zero_rows_write_nothing():
    """A device-side row count of 0 (a share that received no rows): the plan
    holds no task, no workgroup runs one, and no output element is written,
    for every epilogue."""
    K, N, cap, T, k = 128, 256, 4 * 128, 64, 2
    bg_np = np.array([0, 1, 1, 0], np.int32)
    bg = torch.from_numpy(bg_np).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    A = torch.ones((cap, K), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((2, K, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((moe.gemm_workspace(cap).numel(),), 0x55, dtype=torch.uint8, device="cuda")
    for epi in ("store", "silu_mul"):
        say("zero rows", epi)
        out = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.grouped_gemm(A, B, bg, zero, N=N, K=K, cap=cap, B2=B if epi == "silu_mul" else None,
                         epilogue=epi, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(out).all(), epi
        assert np.array_equal(ws[:8].view(torch.int32).cpu().numpy(), _plan_by_definition(bg_np, 0, cap))
    say("zero rows", "weighted_scatter")
    acc = torch.full((T, N), 3.0, dtype=torch.float32, device="cuda")
    row_pair = (torch.arange(cap, dtype=torch.int32, device="cuda") % (T * k)).contiguous()
    moe.grouped_gemm(A, B, bg, zero, N=N, K=K, cap=cap, epilogue="weighted_scatter", row_pair=row_pair,
                     pair_w=torch.ones((T, k), dtype=torch.float32, device="cuda"), out=acc, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(acc, torch.full_like(acc, 3.0))


def test_padding_rows_not_written():
    # rows whose source (or epilogue pair) is negative are padding: left untouched
    K, N, G, T = 128, 256, 3, 200
    cap = 5 * 128
    bg = np.array([0, 0, 1, 2, 2], np.int32)
    g = np.random.default_rng(4)
    src = g.integers(0, T, size=cap).astype(np.int32)
    src[g.random(cap) < 0.3] = -1
    A = syn.ternary_bits((T, K), 70)
    B = syn.ternary_bits((G, K, N), 71)
    say("gemm padding rows")
    D = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=cap, dtype="bf16", src=src, div=1)
    got = to_f64(D)
    ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, a_src_row=src, a_src_div=1)
    assert np.array_equal(got[src >= 0], ref[src >= 0])
    assert np.all(np.isnan(got[src < 0]))
    # identity A rows, padding named by the epilogue pair map instead
    A2 = syn.ternary_bits((cap, K), 72)
    out = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    D2 = moe.grouped_gemm(dev16(A2), dev16(B), torch.from_numpy(bg).cuda(),
                          torch.tensor([cap], dtype=torch.int32, device="cuda"), N=N, K=K, cap=cap,
                          row_pair=torch.from_numpy(src).cuda(), out=out)
    torch.cuda.synchronize()
    got2 = to_f64(D2)
    ref2 = oracle.grouped_gemm(A2, B, bg, N=N, K=K)
    assert np.array_equal(got2[src >= 0], ref2[src >= 0])
    assert np.all(np.isnan(got2[src < 0]))


def _scatter_case(T, k, E, K, N, seed, dtype="bf16"):
    """A down-GEMM-shaped scatter case: routing by the oracle, integer
    (ternary) A and B, power-of-two weights -- every fp32 partial sum is exact
    in any order, so the atomically accumulated result is unique."""
    g = np.random.default_rng(seed)
    idx, _ = oracle.route(g.standard_normal((T, E)).astype(np.float32), k)
    P = oracle.permute(idx, E)
    cap = P["cap"]
    A = syn.ternary_bits((cap, K), seed + 1, dtype)
    B = syn.ternary_bits((E, K, N), seed + 2, dtype)
    w = g.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), size=(T, k))
    return P, A, B, w


def _run_scatter(P, A, B, w, *, N, K, dtype="bf16", out=None, tile=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return moe.grouped_gemm(dev16(A, tdt), dev16(B, tdt), torch.from_numpy(P["block_expert"]).cuda(),
                            torch.tensor([P["m_pad"]], dtype=torch.int32, device="cuda"), N=N, K=K,
                            cap=P["cap"], epilogue="weighted_scatter",
                            row_pair=torch.from_numpy(P["row_to_pair"]).cuda(),
                            pair_w=torch.from_numpy(w).cuda(), out=out, tile=tile)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("epi,layout", [("store", "kn"), ("silu_mul", "kn"), ("silu_mul", "kn_gate_up"),
                                        ("weighted_scatter", "kn")])
def test_streamed_weights_same_bits(dtype, epi, layout):
    # MOE_B_STREAM changes only the cache policy of the weight loads: the
    # same bits as without it (integer-exact data, so the scatter's atomic
    # sums are unique too)
    T, k, E, K = 300, 2, 5, 256
    N = 128 if epi == "silu_mul" else 256
    P, A, B, w = _scatter_case(T, k, E, K, N, 70, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    Bt = dev16(B, tdt)
    B2t = dev16(syn.ternary_bits((E, K, N), 71, dtype), tdt) if epi == "silu_mul" else None
    if layout == "kn_gate_up":
        Bt, B2t = moe.pack_gate_up(Bt, B2t), None
    At = dev16(A, tdt)
    bexp = torch.from_numpy(P["block_expert"]).cuda()
    mpad = torch.tensor([P["m_pad"]], dtype=torch.int32, device="cuda")
    r2p = torch.from_numpy(P["row_to_pair"]).cuda()
    say("streamed weights", dtype, epi, layout)

    def run(stream):
        if epi == "weighted_scatter":
            return moe.grouped_gemm(At, Bt, bexp, mpad, N=N, K=K, cap=P["cap"], epilogue=epi,
                                    row_pair=r2p, pair_w=torch.from_numpy(w).cuda(), b_stream=stream)
        out = torch.full((P["cap"], N), float("nan"), dtype=tdt, device="cuda")
        return moe.grouped_gemm(At, Bt, bexp, mpad, N=N, K=K, cap=P["cap"], B2=B2t, b_layout=layout,
                                epilogue=epi, row_pair=r2p, out=out, b_stream=stream)
    plain, streamed = run(False), run(True)
    torch.cuda.synchronize()
    iv = torch.int32 if epi == "weighted_scatter" else torch.int16
    assert torch.equal(plain.view(iv), streamed.view(iv))


@pytest.mark.parametrize("epi,layout", [("store", "kn"), ("silu_mul", "kn_gate_up"), ("weighted_scatter", "kn")])
def test_streamed_form_skips_only_dead_row_groups(epi, layout):
    # The streamed-weight form skips the matrix instructions of the second
    # half of a one-block task and of 32-row groups that are all padding.
    # Expert sizes that make every case: an empty expert, one-block experts
    # whose last 1, 2 or 3 groups are dead (1, 10, 33, 96 rows), a full block,
    # two-block tasks whose second block holds 1 row or three live groups
    # (129, 200 rows).  Every real row: the same bits as the plain form, and
    # (store, scatter) the oracle's exact result.
    counts = [1, 10, 33, 96, 97, 0, 129, 128, 200]
    E, K = len(counts), 192
    N = 128 if epi == "silu_mul" else 256
    g = np.random.default_rng(91)
    ids = g.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(-1, 1)
    T = ids.shape[0]
    P = oracle.permute(ids, E)
    cap, m_pad, r2p = P["cap"], P["m_pad"], P["row_to_pair"]
    assert list(P["counts"]) == counts
    real = np.nonzero(r2p[:m_pad] >= 0)[0]
    A = syn.ternary_bits((T if epi == "silu_mul" else cap, K), 92)
    B = syn.ternary_bits((E, K, N), 93)
    B2 = syn.ternary_bits((E, K, N), 94) if epi == "silu_mul" else None
    w = g.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), size=(T, 1))
    At, Bt = dev16(A), dev16(B)
    B2t = dev16(B2) if B2 is not None else None
    if layout == "kn_gate_up":
        Bt, B2t = moe.pack_gate_up(Bt, B2t), None
    bexp = torch.from_numpy(P["block_expert"]).cuda()
    mpad = torch.tensor([m_pad], dtype=torch.int32, device="cuda")
    r2pt = torch.from_numpy(r2p).cuda()
    say("streamed skip", epi, layout, "rows", T, "m_pad", m_pad)

    def run(stream):
        if epi == "weighted_scatter":
            return moe.grouped_gemm(At, Bt, bexp, mpad, N=N, K=K, cap=cap, epilogue=epi, row_pair=r2pt,
                                    pair_w=torch.from_numpy(w).cuda(), b_stream=stream)
        out = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        if epi == "silu_mul":
            return moe.grouped_gemm(At, Bt, bexp, mpad, N=N, K=K, cap=cap, a_src_row=r2pt, a_src_div=1,
                                    B2=B2t, b_layout=layout, epilogue=epi, out=out, b_stream=stream)
        return moe.grouped_gemm(At, Bt, bexp, mpad, N=N, K=K, cap=cap, row_pair=r2pt, out=out,
                                b_stream=stream)
    plain, streamed = run(False), run(True)
    torch.cuda.synchronize()
    if epi == "weighted_scatter":
        assert torch.equal(plain.view(torch.int32), streamed.view(torch.int32))
        Y = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K)
        ref = oracle.weighted_scatter(Y, r2p, w, 1, T)
        assert np.array_equal(streamed.cpu().numpy().astype(np.float64), ref)
        return
    rt = torch.from_numpy(real).cuda()
    assert torch.equal(plain[rt].view(torch.int16), streamed[rt].view(torch.int16))
    pad = np.nonzero(r2p[:m_pad] < 0)[0]
    assert torch.isnan(streamed[torch.from_numpy(pad).cuda()]).all()   # padding rows not written
    if epi == "store":
        ref = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K, rows=real)
        assert np.array_equal(to_f64(streamed)[real], ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("T,k,E,K,N", [(150, 3, 4, 320, 256), (200, 1, 5, 64, 128), (90, 2, 3, 128, 192)])
def test_weighted_scatter_integer_exact(dtype, T, k, E, K, N):
    P, A, B, w = _scatter_case(T, k, E, K, N, seed=T + N, dtype=dtype)
    say("scatter integer", dtype, T, k, E, K, N)
    got = _run_scatter(P, A, B, w, N=N, K=K, dtype=dtype)
    torch.cuda.synchronize()
    Y = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K, is_fp16=(dtype == "fp16"))
    ref = oracle.weighted_scatter(Y, P["row_to_pair"], w, k, T)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), ref)


def test_weighted_scatter_accumulates_and_tiles():
    # `out` is accumulated into (the caller zeroes it); every tile shape gives
    # the exact result
    T, k, E, K, N = 260, 2, 6, 512, 256
    P, A, B, w = _scatter_case(T, k, E, K, N, seed=5)
    Y = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K)
    ref = oracle.weighted_scatter(Y, P["row_to_pair"], w, k, T)
    for tile in ["256,32,3,6", "256,32,4,4,2", "128,32,3,10", "64,32,4,8"]:
        say("scatter tile", tile)
        base = torch.full((T, N), 3.0, dtype=torch.float32, device="cuda")
        got = _run_scatter(P, A, B, w, N=N, K=K, out=base, tile=_tile(tile))
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().astype(np.float64), ref + 3.0), tile


def test_weighted_scatter_random_values():
    # bf16 random data, fp32 atomics: within the tolerances of the oracle's exact sum
    T, k, E, K, N = 300, 4, 8, 256, 512
    g = np.random.default_rng(21)
    idx, w = oracle.route(g.standard_normal((T, E)).astype(np.float32), k)
    P = oracle.permute(idx, E)
    A = syn.bf16_bits(g.standard_normal((P["cap"], K)).astype(np.float32))
    B = syn.bf16_bits((g.standard_normal((E, K, N)) / np.sqrt(K)).astype(np.float32))
    say("scatter random")
    got = _run_scatter(P, A, B, w, N=N, K=K)
    torch.cuda.synchronize()
    Y = oracle.grouped_gemm(A, B, P["block_expert"], N=N, K=K)
    ref = oracle.weighted_scatter(Y, P["row_to_pair"], w, k, T)
    assert_close(got.cpu().numpy().astype(np.float64), ref, "scatter random", max_frac=1e-4, rel_fro=1e-5)


@pytest.mark.parametrize("n", [8, 1000003, 4096 * 2048])
def test_finalize_rounds_to_nearest_even(n):
    # against torch's CPU fp32 -> bf16 conversion (round to nearest even)
    g = torch.Generator().manual_seed(n)
    acc = torch.randn(n, generator=g) * 100
    acc[: min(n, 4)] = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0])[: min(n, 4)]
    say("finalize", n)
    out = moe.finalize(acc.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), acc.to(torch.bfloat16).view(torch.int16))


def _interleave(gate, up):
    """[G][K][N] gate and up -> [G][K][2N]: per 128-column block, gate then up
    (a reshape of the test's own arrays, no arithmetic)."""
    G, K, N = gate.shape
    return np.concatenate([gate.reshape(G, K, N // 128, 128), up.reshape(G, K, N // 128, 128)],
                          axis=3).reshape(G, K, 2 * N)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_pack_gate_up_bit_exact(dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    g = np.random.default_rng(31)
    for E, K, N in [(1, 1, 128), (3, 64, 256), (5, 320, 1536)]:
        gate = g.integers(0, 65535, size=(E, K, N)).astype(np.uint16)
        up = g.integers(0, 65535, size=(E, K, N)).astype(np.uint16)
        say("pack gate/up", dtype, E, K, N)
        out = moe.pack_gate_up(dev16(gate, tdt), dev16(up, tdt))
        torch.cuda.synchronize()
        assert np.array_equal(host16(out), _interleave(gate, up))


@pytest.mark.parametrize("tile", [None, "128,32,4,4,2", "64,32,3,10"])
def test_gate_up_interleaved_layout(tile):
    # the interleaved weights give the same bits as the two separate matrices,
    # and the integer-exact result of the oracle, in every SiLU*up tile shape
    # (a tile whose rings are unsafe for the K is refused on both layouts)
    t = _tile(tile) if tile else None
    G, cap = 4, 11 * 128
    m_rows = 9 * 128
    bg = _groups(cap // 128, G, 23)
    for N, K in [(512, 320), (128, 64), (384, 128)]:
        A = syn.ternary_bits((cap, K), 11)
        B = syn.ternary_bits((G, K, N), 12)
        B2 = syn.ternary_bits((G, K, N), 13)
        say("gemm gate/up interleaved", tile, N, K)
        if t and 2 * (K // t[1]) < t[3] - 1:
            for kw in (dict(B2_bits=B2), dict(layout="kn_gate_up")):
                with pytest.raises(moe.MoeError):
                    _run(A, B if "B2_bits" in kw else _interleave(B, B2), bg, N=N, K=K, cap=cap,
                         m_rows=m_rows, dtype="bf16", epi="silu_mul", tile=t, **kw)
            continue
        D0 = _run(A, B, bg, N=N, K=K, cap=cap, m_rows=m_rows, dtype="bf16", B2_bits=B2, epi="silu_mul",
                  tile=t)
        D1 = _run(A, _interleave(B, B2), bg, N=N, K=K, cap=cap, m_rows=m_rows, dtype="bf16",
                  layout="kn_gate_up", epi="silu_mul", tile=t)
        assert torch.equal(D0[:m_rows].view(torch.int16), D1[:m_rows].view(torch.int16))
        ref = oracle.grouped_gemm(A, B, bg, N=N, K=K, B2_bits=B2, epilogue="silu_mul",
                                  rows=np.arange(m_rows, dtype=np.int32))
        assert_close(to_f64(D1)[:m_rows], ref, "interleaved", max_frac=8e-3, rel_fro=4e-3)
        assert np.all(np.isnan(to_f64(D1)[m_rows:]))
