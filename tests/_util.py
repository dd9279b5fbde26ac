"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import sys

import numpy as np
import torch

# spec tolerances for bf16 inputs with fp32 accumulation
MAX_ABS_FRAC = 2e-2   # max |gpu - oracle| <= 2e-2 * max |oracle|
REL_FRO = 5e-3        # ||gpu - oracle||_F <= 5e-3 * ||oracle||_F


def say(*a):
    """Name the case before a GPU step, flushed, so a fault report names it."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev16(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> a GPU tensor of bf16 / fp16 with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(dtype).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def close_metrics(gpu: np.ndarray, ref: np.ndarray):
    err = gpu - ref
    max_abs = float(np.max(np.abs(err)))
    scale = float(np.max(np.abs(ref)))
    fro = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    return max_abs, scale, fro


def assert_close(gpu: np.ndarray, ref: np.ndarray, what="", max_frac=MAX_ABS_FRAC, rel_fro=REL_FRO):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output " + what
    max_abs, scale, fro = close_metrics(gpu, ref)
    assert max_abs <= max_frac * scale, "%s: max|err| %.3e > %.1e * %.3e" % (what, max_abs, max_frac, scale)
    assert fro <= rel_fro, "%s: rel Frobenius %.3e > %.1e" % (what, fro, rel_fro)
    return max_abs / max(scale, 1e-300), fro
