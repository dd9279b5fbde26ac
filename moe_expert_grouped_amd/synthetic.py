"""Seeded synthetic inputs for the grouped-GEMM MoE layer.

This module holds only random-number generation and the rounding of fp32
draws to the 16-bit storage formats; none of the layer's arithmetic.  Both the
oracle-side tests and the GPU side draw their inputs from here, so the two
always see identical bits.

Workloads follow the shapes of the serial TP MoE layer in "Comm-compute
fusion (1)", section 1 (4 x 512 gathered tokens, hidden 4096, 64 experts, a
quarter weight slice per GPU) and of the dense fp16 4096^3 GEMM in "TIRx and
high-performance GEMM (part 2)", performance table; value distributions:
x ~ N(0,1), weights ~ N(0, 1/sqrt(fan_in)) (std), router logits ~ N(0,1).
The pages use no dataset; these seeded draws stand in for one.
"""
from __future__ import annotations

import numpy as np

# name -> shape.  "routing": "logits" = router logits are an input and the
# layer routes them; "zipf" = the (token, expert) assignment is given.
CONFIGS = {
    "tiny": dict(kind="moe", T=256, H=256, E=8, k=2, I=512, routing="logits"),
    "dense": dict(kind="dense", M=4096, N=4096, K=4096),
    "tp_share": dict(kind="moe", T=2048, H=4096, E=64, k=4, I=512, routing="logits"),
    "ep_skew": dict(kind="moe", T=2048, H=4096, E=16, k=1, I=2048, routing="zipf"),
    "ep_skew_small": dict(kind="moe", T=128, H=4096, E=16, k=1, I=2048, routing="zipf"),
    "prefill": dict(kind="moe", T=16384, H=4096, E=64, k=8, I=1536, routing="logits",
                    expert_bias=0.5),
}

ZIPF_S = 1.2          # skew exponent of the expert-parallel share
ZIPF_ACTIVE = 12      # experts that receive rows; the other 4 of 16 stay empty


def bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def fp16_bits(f: np.ndarray) -> np.ndarray:
    """Round fp32 to IEEE half (numpy's cast rounds to nearest even); uint16 bits."""
    return np.ascontiguousarray(f, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gens(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(8)]


def make_moe(T, H, E, k, I, routing="logits", expert_bias=0.0, seed=0, zipf_active=None,
             with_weights=True):
    """Inputs of one MoE layer share.

    Returns a dict with x [T,H], wg/wu [E,H,I], wd [E,I,H] (bf16 bits) and
    either logits [T,E] fp32 (routing == "logits") or a given assignment
    topk_idx [T,k] int32 / topk_w [T,k] fp32 (routing == "zipf", k == 1)."""
    g = _gens(seed)
    out = dict(T=T, H=H, E=E, k=k, I=I)
    if routing == "logits":
        logits = g[0].standard_normal((T, E), dtype=np.float32)
        if expert_bias:
            logits += g[5].normal(0.0, expert_bias, E).astype(np.float32)
        out["logits"] = logits
    elif routing == "zipf":
        assert k == 1
        act = zipf_active or min(ZIPF_ACTIVE, E)
        r = np.arange(1, act + 1, dtype=np.float64)
        p = r ** -ZIPF_S
        p /= p.sum()
        experts = g[6].permutation(E)[:act]
        out["topk_idx"] = experts[g[6].choice(act, size=T, p=p)].astype(np.int32).reshape(T, 1)
        out["topk_w"] = np.ones((T, 1), np.float32)
    elif routing == "uniform_idx":
        # distinct experts per token drawn uniformly, weights ~ softmax-like positive
        idx = np.argsort(g[6].random((T, E)), axis=1)[:, :k].astype(np.int32)
        w = g[7].random((T, k)).astype(np.float32) + np.float32(0.05)
        out["topk_idx"] = idx
        out["topk_w"] = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    else:
        raise ValueError(routing)
    out["x"] = bf16_bits(g[1].standard_normal((T, H), dtype=np.float32))
    if with_weights:
        out["wg"] = bf16_bits(g[2].standard_normal((E, H, I), dtype=np.float32) / np.float32(np.sqrt(H)))
        out["wu"] = bf16_bits(g[3].standard_normal((E, H, I), dtype=np.float32) / np.float32(np.sqrt(H)))
        out["wd"] = bf16_bits(g[4].standard_normal((E, I, H), dtype=np.float32) / np.float32(np.sqrt(I)))
    return out


def make_config(name: str, seed: int = 0, **over):
    c = dict(CONFIGS[name])
    c.update(over)
    kind = c.pop("kind")
    if kind == "dense":
        return make_dense(c["M"], c["N"], c["K"], seed=seed)
    return make_moe(seed=seed, **c)


def make_dense(M, N, K, seed=0):
    """D = A . B^T operands: A [M,K], B [N,K] fp16 bits, both ~ U(-1, 1)."""
    g = _gens(seed)
    A = fp16_bits(g[0].uniform(-1.0, 1.0, (M, K)).astype(np.float32))
    B = fp16_bits(g[1].uniform(-1.0, 1.0, (N, K)).astype(np.float32))
    return dict(A=A, B=B, M=M, N=N, K=K)


def ternary_bits(shape, seed, dtype="bf16", p_zero=1 / 3):
    """Entries in {-1, 0, +1}: every partial sum of a product of such matrices
    is a small integer, exact in fp32 in any order (used for bit-exact GEMM
    checks that expose any row/column mapping mistake)."""
    g = np.random.default_rng(seed)
    v = g.choice(np.array([-1.0, 0.0, 1.0], np.float32), size=shape,
                 p=[(1 - p_zero) / 2, p_zero, (1 - p_zero) / 2])
    return bf16_bits(v) if dtype == "bf16" else fp16_bits(v)


def sparse_ternary_bits(shape, seed, density, dtype="bf16"):
    """Entries in {-1, 0, +1}, each non-zero with probability `density`
    (rounded to a multiple of 1/128), +1 and -1 equally likely; uint16 bits.
    One byte drawn per entry and mapped through a table, so full-size weight
    tensors are quick to make.  Sparse enough, every product of such
    matrices stays a small integer: exact in fp32 in any summation order and
    exactly representable after the 16-bit store."""
    t = int(round(128 * density))
    if not 0 <= t <= 128:
        raise ValueError("density must be in [0, 1]")
    one = bf16_bits if dtype == "bf16" else fp16_bits
    pos, neg = (int(v) for v in one(np.array([1.0, -1.0], np.float32)))
    lut = np.zeros(256, np.uint16)
    lut[:t] = pos
    lut[256 - t:] = neg
    u = np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
    return lut[u]
