"""Pins of the oracle to things other than itself: brute force on tiny
inputs, closed forms, invariants, hand-worked fixtures and special cases that
reduce to textbook or library routines.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from moe_expert_grouped_amd import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ORC = oracle  # the pin functions below take the oracle API as an argument


# ---------------------------------------------------------------- helpers

def brute_route(logits, k):
    T, E = logits.shape
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        idx[t] = order[:k]
    return idx


def brute_gemm_rows(A, B, groups_of_rows, src_of_rows, layout):
    """float64 numpy products, one 128-row block at a time."""
    out = np.full((len(src_of_rows), B.shape[2] if layout == "kn" else B.shape[1]), np.nan)
    for r, (src, g) in enumerate(zip(src_of_rows, groups_of_rows)):
        if src < 0 or g < 0:
            continue
        Bg = B[g] if layout == "kn" else B[g].T
        out[r] = A[src] @ Bg
    return out


def f32(bits):
    return syn.bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- pins as functions of an oracle API
# (so that the mutation tests can run the same pins against planted mistakes)

def pin_router_logits(O):
    rng = np.random.default_rng(21)
    # one-hot token rows pick out one hidden column of W exactly (non-square
    # T, H, E, so a transposed W or a wrong row stride shows)
    T, H, E = 7, 40, 5
    W = syn.bf16_bits(rng.standard_normal((E, H)).astype(np.float32))
    hs = rng.integers(0, H, size=T)
    x = np.zeros((T, H), np.uint16)
    x[np.arange(T), hs] = 0x3F80  # bf16 1.0
    lg = O.router_logits(x, W)
    assert np.array_equal(lg, f32(W)[:, hs].T)
    # entries in {-1, 0, 1}: integer logits, exact against an integer matrix product
    x = syn.ternary_bits((33, 96), 22)
    W = syn.ternary_bits((11, 96), 23)
    lg = O.router_logits(x, W)
    assert np.array_equal(lg, (f32(x).astype(np.int64) @ f32(W).astype(np.int64).T).astype(np.float64))
    # linear in x: doubling a row doubles its logits exactly
    x2 = x.copy()
    x2[0] = syn.bf16_bits(2.0 * f32(x[:1]).astype(np.float32))[0]
    assert np.array_equal(O.router_logits(x2, W)[0], 2.0 * lg[0])


def pin_route_bruteforce(O):
    rng = np.random.default_rng(1)
    for T, E, k in [(50, 8, 2), (40, 64, 4), (30, 257, 8), (20, 5, 5), (10, 1, 1), (33, 16, 1)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        idx, w = O.route(lg, k)
        assert np.array_equal(idx, brute_route(lg, k)), (T, E, k)
    # heavy ties: integer-valued logits
    lg = rng.integers(-2, 3, size=(200, 12)).astype(np.float32)
    for k in (1, 3, 12):
        idx, w = O.route(lg, k)
        assert np.array_equal(idx, brute_route(lg, k)), k


def pin_route_closed_forms(O):
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((64, 32)).astype(np.float32)
    # k = 1: the single weight is exactly 1
    idx, w = O.route(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    # all-equal logits: experts 0..k-1, weights exactly 1/k
    for k in (1, 2, 4, 8):
        idx, w = O.route(np.full((3, 16), 0.25, np.float32), k)
        assert np.array_equal(idx, np.tile(np.arange(k), (3, 1)))
        assert np.all(w == np.float32(1.0 / k))
    # invariants: weights sum to one, are non-increasing, and match an exp ratio
    for k in (2, 4, 8):
        idx, w = O.route(lg, k)
        assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
        assert np.all(np.diff(w, axis=1) <= 0)
        l_sel = np.take_along_axis(lg, idx, 1).astype(np.float64)
        # w_j / w_0 = exp(l_j - l_0)  (ratio form, independent of the normaliser)
        assert np.allclose(w[:, 1:] / w[:, :1], np.exp(l_sel[:, 1:] - l_sel[:, :1]), rtol=3e-7)
    # k = E: a permutation of all experts
    idx, _ = O.route(lg, 32)
    assert np.array_equal(np.sort(idx, 1), np.tile(np.arange(32), (64, 1)))


def pin_route_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "route_worked.json")))
    idx, w = O.route(np.array(g["logits"], np.float32), g["k"])
    assert np.array_equal(idx, np.array(g["idx"]))
    assert np.max(np.abs(w - np.array(g["w"]))) <= g["w_tol"]


def check_permutation(idx, E, P):
    T, k = idx.shape
    R = T * k
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(P["counts"], counts)
    assert P["counts"].sum() == R
    pad = (counts + 127) // 128 * 128
    assert np.array_equal(P["offsets"], np.concatenate([[0], np.cumsum(pad)]))
    assert np.all(P["offsets"] % 128 == 0)
    assert P["m_pad"] == P["offsets"][-1] <= R + min(E, R) * 127
    # brute force: rows of expert e hold its pairs in ascending pair order
    order = sorted(range(R), key=lambda p: (flat[p], p))
    expect_p2r = np.empty(R, np.int64)
    for e in range(E):
        mine = [p for p in order if flat[p] == e]
        for i, p in enumerate(mine):
            expect_p2r[p] = P["offsets"][e] + i
    assert np.array_equal(P["pair_to_row"], expect_p2r)
    r2p = P["row_to_pair"]
    assert np.array_equal(r2p[P["pair_to_row"]], np.arange(R))    # bijection
    assert (r2p >= 0).sum() == R
    assert np.all(r2p[r2p < 0] == -1)
    be = P["block_expert"]
    for b in range(len(be)):
        r = b * 128
        if r >= P["m_pad"]:
            assert be[b] == -1
        else:
            e = int(np.searchsorted(P["offsets"], r, side="right") - 1)
            assert be[b] == e


def pin_permute(O):
    rng = np.random.default_rng(3)
    cases = [
        rng.integers(0, 8, size=(100, 2)),                 # random
        np.zeros((300, 1), np.int64),                      # every pair on one expert
        np.array([[3]]),                                   # one token
        np.full((129, 1), 2),                              # 129 rows -> 2 blocks
        np.concatenate([np.zeros(127), np.ones(128), np.full(129, 2)]).reshape(-1, 1),
        rng.integers(0, 1, size=(64, 1)),                  # E = 1
    ]
    Es = [8, 4, 5, 3, 4, 1]
    for idx, E in zip(cases, Es):
        idx = idx.astype(np.int32)
        P = O.permute(idx, E)
        check_permutation(idx, E, P)
    # empty experts and top-k pairs from a real routing
    lg = rng.standard_normal((90, 16)).astype(np.float32)
    lg[:, [3, 7, 11]] = -50.0
    idx, _ = O.route(lg, 4)
    P = O.permute(idx, 16)
    assert P["counts"][3] == P["counts"][7] == P["counts"][11] == 0
    check_permutation(idx, 16, P)
    with pytest.raises(ValueError):
        O.permute(np.zeros((200, 1), np.int32), 1, cap=128)


def pin_gather(O):
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 4, size=(40, 2)).astype(np.int32)
    P = O.permute(idx, 4)
    x = rng.integers(0, 65535, size=(40, 24)).astype(np.uint16)
    xp = O.gather(x, P["row_to_pair"], 2)
    for r, p in enumerate(P["row_to_pair"]):
        if p < 0:
            assert np.all(xp[r] == 0)
        else:
            assert np.array_equal(xp[r], x[p // 2])


def pin_gemm_random(O):
    rng = np.random.default_rng(5)
    # ragged groups: block_group covers 5 blocks of 128 rows, one unused block at the end
    G, K, N = 3, 48, 40
    M = 5 * 128
    block_group = np.array([0, 2, 2, 1, -1], np.int32)
    T = 150
    A32 = rng.standard_normal((T, K)).astype(np.float32)
    A = syn.bf16_bits(A32)
    src = rng.integers(-1, T * 3, size=M).astype(np.int32)   # some rows without source
    for layout in ("kn", "nk"):
        shape = (G, K, N) if layout == "kn" else (G, N, K)
        B = syn.bf16_bits(rng.standard_normal(shape).astype(np.float32))
        D = O.grouped_gemm(A, B, block_group, N=N, K=K, b_layout=layout, a_src_row=src, a_src_div=3)
        groups = [block_group[r // 128] for r in range(M)]
        srcs = [s // 3 if s >= 0 else -1 for s in src]
        ref = brute_gemm_rows(f32(A), f32(B), groups, srcs, layout)
        nan = np.isnan(ref)
        assert np.array_equal(nan, np.isnan(D))
        assert np.max(np.abs(D[~nan] - ref[~nan])) <= 1e-12 * np.max(np.abs(ref[~nan]))
    # fp16 decode and identity row map, non-square to expose a transposed operand
    Ah = syn.fp16_bits(rng.uniform(-1, 1, (256, 72)).astype(np.float32))
    Bh = syn.fp16_bits(rng.uniform(-1, 1, (1, 40, 72)).astype(np.float32))
    D = O.grouped_gemm(Ah, Bh, np.zeros(2, np.int32), N=40, K=72, is_fp16=True, b_layout="nk")
    ref = Ah.view(np.float16).astype(np.float64) @ Bh[0].view(np.float16).astype(np.float64).T
    assert np.max(np.abs(D - ref)) <= 1e-12


def pin_gemm_integer_exact(O):
    # entries in {-1,0,1}: every partial sum is an exact integer
    K, N = 96, 56
    A = syn.ternary_bits((256, K), 6)
    B = syn.ternary_bits((2, K, N), 7)
    D = O.grouped_gemm(A, B, np.array([1, 0], np.int32), N=N, K=K)
    Ai = f32(A).astype(np.int64)
    Bi = f32(B).astype(np.int64)
    ref = np.concatenate([Ai[:128] @ Bi[1], Ai[128:] @ Bi[0]])
    assert np.array_equal(D, ref.astype(np.float64))


def pin_fp16_decode(O):
    # special half values through a 1x1x1 product with B = 1.0
    vals = np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 6.103515625e-05, 5.960464477539063e-08,
                     3.0517578125e-05, -1.1920928955078125e-07], np.float16)
    A = vals.view(np.uint16).reshape(-1, 1)
    A = np.concatenate([A, np.zeros((128 - len(vals), 1), np.uint16)])
    one = np.array([[[1.0]]], np.float16).view(np.uint16)
    D = O.grouped_gemm(A, one, np.zeros(1, np.int32), N=1, K=1, is_fp16=True)
    assert np.array_equal(D[:len(vals), 0], vals.astype(np.float64))


def _silu_of(O, zs, gate_w=1.0, up_w=1.0):
    """One token row [z, 1]; gate weights [gate_w, 0], up weights [0, up_w]:
    the output is SiLU(gate_w * z) * up_w."""
    zs = np.asarray(zs, np.float32)
    A = np.zeros((128, 2), np.uint16)
    A[: len(zs), 0] = syn.bf16_bits(zs)
    A[: len(zs), 1] = syn.bf16_bits(np.ones(len(zs), np.float32))
    Bg = syn.bf16_bits(np.array([[[gate_w], [0.0]]], np.float32))
    Bu = syn.bf16_bits(np.array([[[0.0], [up_w]]], np.float32))
    return O.grouped_gemm(A, Bg, np.zeros(1, np.int32), N=1, K=2, B2_bits=Bu,
                          epilogue="silu_mul")[: len(zs), 0]


def pin_silu(O):
    zs = np.array([0.0, 0.5, -0.5, 2.0, -2.0, 64.0, -64.0, 1.5, -1.5, 1.0], np.float32)
    s = _silu_of(O, zs)
    z = zs.astype(np.float64)
    assert s[0] == 0.0
    # SiLU(z) - SiLU(-z) = z for every z
    for a, b in [(1, 2), (3, 4), (5, 6), (7, 8)]:
        assert abs((s[a] - s[b]) - z[a]) <= 1e-15 * abs(z[a])
    # saturation: SiLU(z) -> z for large z, -> 0 from below for very negative z
    assert s[5] == 64.0
    assert -1e-20 < s[6] < 0.0
    # 0 < SiLU(z) < z for z > 0, increasing there
    assert 0 < s[1] < 0.5 and s[1] < s[9] < s[7] < s[3] < 2.0
    # gate and up play different roles: SiLU(2 * 1) * 1 versus SiLU(1) * 2
    g2 = _silu_of(O, [1.0], gate_w=2.0)[0]
    u2 = _silu_of(O, [1.0], up_w=2.0)[0]
    assert g2 == s[3]
    assert u2 == 2.0 * s[9]
    assert s[7] < u2 < s[3]  # SiLU(1.5) < 2 SiLU(1) < SiLU(2)


def pin_combine(O):
    rng = np.random.default_rng(8)
    T, k, E, H = 60, 3, 6, 32
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = O.route(lg, k)
    P = O.permute(idx, E)
    y = syn.bf16_bits(rng.standard_normal((P["cap"], H)).astype(np.float32))
    out = O.combine(y, P["pair_to_row"], w)
    yf = f32(y)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            ref[t] += float(w[t, j]) * yf[P["pair_to_row"][t * k + j]]
    assert np.max(np.abs(out - ref)) <= 1e-13
    # k = 1, weight 1: a pure un-permutation, bit for bit
    idx1, w1 = O.route(lg, 1)
    P1 = O.permute(idx1, E)
    y1 = syn.bf16_bits(rng.standard_normal((P1["cap"], H)).astype(np.float32))
    o1 = O.combine(y1, P1["pair_to_row"], w1)
    assert np.array_equal(o1, f32(y1)[P1["pair_to_row"]])
    # one-hot weights select one slot
    wh = np.zeros((T, k), np.float32)
    wh[:, 1] = 1.0
    oh = O.combine(y, P["pair_to_row"], wh)
    assert np.array_equal(oh, yf[P["pair_to_row"].reshape(T, k)[:, 1]])


def pin_weighted_scatter(O):
    rng = np.random.default_rng(12)
    T, k, E, N = 50, 3, 7, 24
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = O.route(lg, k)
    P = O.permute(idx, E)
    r2p = P["row_to_pair"]
    Y = rng.standard_normal((P["cap"], N))
    Y[r2p < 0] = np.nan  # padding rows carry no value and must add nothing
    out = O.weighted_scatter(Y, r2p, w, k, T)
    # brute force over rows
    ref = np.zeros((T, N))
    for r in range(P["cap"]):
        p = int(r2p[r])
        if p >= 0:
            ref[p // k] += float(w.reshape(-1)[p]) * Y[r]
    assert np.max(np.abs(out - ref)) <= 1e-13
    # the same sum as the gather-side combine over pair_to_row (k slots per token)
    ref2 = np.zeros((T, N))
    for t in range(T):
        for j in range(k):
            ref2[t] += float(w[t, j]) * Y[P["pair_to_row"][t * k + j]]
    assert np.max(np.abs(out - ref2)) <= 1e-13
    # k = 1, weight 1: a pure un-permutation, bit for bit
    idx1, w1 = O.route(lg, 1)
    P1 = O.permute(idx1, E)
    Y1 = rng.standard_normal((P1["cap"], N))
    o1 = O.weighted_scatter(Y1, P1["row_to_pair"], w1, 1, T)
    assert np.array_equal(o1, Y1[P1["pair_to_row"]])
    # one-hot weights select one slot
    wh = np.zeros((T, k), np.float32)
    wh[:, 2] = 1.0
    oh = O.weighted_scatter(Y, r2p, wh, k, T)
    assert np.array_equal(oh, Y[P["pair_to_row"].reshape(T, k)[:, 2]])


def _layer_inputs(T, H, E, k, I, seed):
    d = syn.make_moe(T, H, E, k, I, seed=seed)
    idx, w = ORC.route(d["logits"], k)
    return d, idx, w


def pin_layer_dense_special_case(O):
    # E = 1, k = 1, w = 1: exactly a dense SwiGLU FFN (torch float64 library ops)
    T, H, I = 40, 64, 48
    d = syn.make_moe(T, H, 1, 1, I, seed=9)
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out = O.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"])
    x = torch.from_numpy(f32(d["x"]))
    g = x @ torch.from_numpy(f32(d["wg"])[0])
    u = x @ torch.from_numpy(f32(d["wu"])[0])
    ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(f32(d["wd"])[0])
    assert np.max(np.abs(out - ref.numpy())) <= 1e-12 * float(ref.abs().max())


def pin_layer_bruteforce(O):
    T, H, E, k, I = 24, 32, 5, 2, 16
    d = syn.make_moe(T, H, E, k, I, seed=10)
    idx, w = O.route(d["logits"], k)
    out = O.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"])
    x, Wg, Wu, Wd = f32(d["x"]), f32(d["wg"]), f32(d["wu"]), f32(d["wd"])
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = x[t] @ Wg[e]
            u = x[t] @ Wu[e]
            a = g / (1.0 + np.exp(-g)) * u
            ref[t] += float(w[t, j]) * (a @ Wd[e])
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))
    # tokens are independent: a token subset in any order gives the same rows
    sub = np.array([7, 3, 19, 3], np.int32)
    o2 = O.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"], tokens=sub)
    assert np.array_equal(o2, out[sub])


def pin_layer_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "layer_worked.json")))
    bits = lambda a: syn.bf16_bits(np.array(a, np.float32))
    idx, w = O.route(np.array(g["logits"], np.float32), g["k"])
    out = O.moe_tokens(bits(g["x"]), idx, w, bits(g["wg"]), bits(g["wu"]), bits(g["wd"]))
    assert np.max(np.abs(out - np.array(g["out"]))) <= g["tol"]


def pin_pipeline_equals_definition(O):
    """route -> permute -> grouped gate/up (SiLU*up) -> grouped down -> combine
    reproduces the per-token definition (h and y rounded to bf16 as stored)."""
    T, H, E, k, I = 64, 64, 6, 2, 32
    d = syn.make_moe(T, H, E, k, I, seed=11)
    idx, w = O.route(d["logits"], k)
    P = O.permute(idx, E)
    be = P["block_expert"]
    h = O.grouped_gemm(d["x"], d["wg"], be, N=I, K=H, a_src_row=P["row_to_pair"], a_src_div=k,
                       B2_bits=d["wu"], epilogue="silu_mul")
    hb = syn.bf16_bits(np.nan_to_num(h).astype(np.float32))
    y = O.grouped_gemm(hb, d["wd"], be, N=H, K=I)
    yb = syn.bf16_bits(np.nan_to_num(y).astype(np.float32))
    out = O.combine(yb, P["pair_to_row"], w)
    ref = O.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"])
    err = out - ref
    assert np.sqrt((err ** 2).sum() / (ref ** 2).sum()) < 5e-3
    assert np.max(np.abs(err)) < 2e-2 * np.max(np.abs(ref))


PINS = [pin_router_logits, pin_route_bruteforce, pin_route_closed_forms, pin_route_golden, pin_permute, pin_gather,
        pin_gemm_random, pin_gemm_integer_exact, pin_fp16_decode, pin_silu, pin_combine, pin_weighted_scatter,
        pin_layer_dense_special_case, pin_layer_bruteforce, pin_layer_golden,
        pin_pipeline_equals_definition]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle)


def test_generator_properties():
    # the expert-parallel share: 4 of 16 experts empty, the top one above 25 % of rows
    d = syn.make_config("ep_skew", with_weights=False)
    counts = np.bincount(d["topk_idx"][:, 0], minlength=16)
    assert (counts == 0).sum() == 4
    assert counts.max() > 0.25 * 2048
    assert np.all(d["topk_w"] == 1.0)
    # RNE to bf16: ties to even, and exact values survive
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3.0e38], np.float32)
    b = syn.bf16_bits(f)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0x8000, 0x7F62]
    assert np.array_equal(syn.bf16_to_f32(syn.bf16_bits(np.float32([0.15625]))), [0.15625])
    # same seed, same bits
    a1 = syn.make_moe(8, 16, 4, 2, 8, seed=3)
    a2 = syn.make_moe(8, 16, 4, 2, 8, seed=3)
    assert all(np.array_equal(a1[k], a2[k]) for k in ("x", "wg", "wu", "wd", "logits"))
