"""The C ABI on the host: the library loads, exports every entry point that
include/moe.h declares, and rejects bad arguments before touching a device.
No compute call is made (there may be no GPU)."""
import ctypes
import os
import re

import pytest

import moe_expert_grouped_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_gfx950.so not built: run __graft_entry__.build()")
    return moe.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 22, names
    for n in ["moe_route", "moe_router", "moe_permute", "grouped_gemm", "grouped_gemm_tuned", "moe_combine",
              "moe_finalize", "moe_layer", "moe_layer_ex", "moe_pack_gate_up", "moe_layer_workspace_size_ex",
              "grouped_gemm_noalloc", "moe_layer_router", "moe_layer_router_workspace_size"]:
        assert n in names
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"
    assert lib.moe_version().startswith(b"moe-grouped")


def test_padded_capacity(lib):
    # ceil128(R + min(E, R) * 127)
    for T, k, E in [(256, 2, 8), (2048, 4, 64), (2048, 1, 16), (128, 1, 16), (16384, 8, 64), (1, 1, 1), (3, 2, 1000)]:
        R = T * k
        cap = R + min(E, R) * 127
        cap = (cap + 127) // 128 * 128
        assert lib.moe_padded_capacity(T, k, E) == cap
    assert lib.moe_padded_capacity(0, 1, 1) == -1
    assert lib.moe_padded_capacity(1, 0, 1) == -1


def test_layer_workspace_layout(lib):
    T, H, E, k, I = 2048, 4096, 64, 4, 512
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    offs = [lay[n] for n in moe.LAYOUT_NAMES]
    assert offs == sorted(offs)
    assert all(o % 256 == 0 for o in offs)
    cap = moe.padded_capacity(T, k, E)
    assert lay["y"] - lay["h"] >= cap * I * 2
    assert lay["permute_scratch"] - lay["y"] >= cap * H * 2
    assert lay["total"] - lay["out_acc"] >= T * H * 4
    assert lib.moe_layer_workspace_size(T, H, E, k, I) == lay["total"]
    assert lib.moe_layer_workspace_size(T, H, E, 65, I) == 0  # k > E
    # the gather combine needs no fp32 token-row accumulator, which comes last
    assert lib.moe_layer_workspace_size_ex(T, H, E, k, I, 0) == lay["out_acc"]
    assert lib.moe_layer_workspace_size_ex(T, H, E, k, I, 1) == lay["total"]
    assert lib.moe_layer_workspace_size_ex(T, H, E, k, I, 2) == 0


FAKE = ctypes.c_void_p(4096)       # aligned non-null; never dereferenced
MISALIGNED = ctypes.c_void_p(4098)
NULL = None


def test_router_validation(lib):
    def call(x=FAKE, w=FAKE, T=4, H=256, E=8, k=2, lg=NULL, idx=FAKE, wo=FAKE, ws=FAKE, wsb=1 << 20,
             counts=NULL):
        return lib.moe_router(x, w, T, H, E, k, lg, idx, wo, counts, ws, wsb, NULL)
    assert call(x=NULL) == moe.MOE_ERR_INVALID
    assert call(w=NULL) == moe.MOE_ERR_INVALID
    assert call(idx=NULL) == moe.MOE_ERR_INVALID
    assert call(wo=NULL) == moe.MOE_ERR_INVALID
    assert call(x=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(w=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(T=0) == moe.MOE_ERR_INVALID
    assert call(k=9) == moe.MOE_ERR_INVALID          # k > E
    assert call(H=96) == moe.MOE_ERR_UNSUPPORTED     # H % 64
    assert call(E=129) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=64, k=17) == moe.MOE_ERR_UNSUPPORTED
    assert call(ws=NULL) == moe.MOE_ERR_WORKSPACE    # 4 tokens: the hidden dimension is split
    assert call(wsb=16) == moe.MOE_ERR_WORKSPACE
    assert call(ws=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(lg=FAKE) == moe.MOE_ERR_DEVICE       # valid arguments; no GPU here
    assert call(counts=FAKE) == moe.MOE_ERR_DEVICE
    # the slices: only a short routing needs the workspace, which holds S partial [T][E] tiles
    assert lib.moe_router_workspace_size(2048, 4096, 64) == 4 * 2048 * 64 * 4
    assert lib.moe_router_workspace_size(8192, 4096, 64) == 0
    assert lib.moe_router_workspace_size(300, 192, 128) == 0
    assert lib.moe_router_workspace_size(4, 256, 8) == 4 * 4 * 8 * 4
    assert lib.moe_router_workspace_size(4, 96, 8) == 0


def test_route_validation(lib):
    assert lib.moe_route(NULL, 4, 8, 2, FAKE, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, NULL) == moe.MOE_ERR_INVALID     # k > E
    assert lib.moe_route(FAKE, 0, 8, 2, FAKE, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_route(FAKE, 4, 2048, 2, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(FAKE, 4, 64, 17, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED


def test_permute_validation(lib):
    ws = lib.moe_permute_workspace_size(100, 2, 8)
    assert ws > 0
    cap = lib.moe_padded_capacity(100, 2, 8)
    args = lambda **kw: dict(dict(idx=FAKE, T=100, k=2, E=8, x=NULL, H=0, cap=cap, ws=FAKE, wsb=ws), **kw)

    def call(a):
        return lib.moe_permute(a["idx"], a["T"], a["k"], a["E"], a["x"], a["H"], FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, FAKE if a["x"] else NULL, a["cap"], a["ws"], a["wsb"], NULL)
    assert call(args(idx=NULL)) == moe.MOE_ERR_INVALID
    assert call(args(cap=cap - 128)) == moe.MOE_ERR_WORKSPACE
    assert call(args(cap=cap + 1)) == moe.MOE_ERR_INVALID
    assert call(args(wsb=ws - 1)) == moe.MOE_ERR_WORKSPACE
    assert call(args(E=2000)) == moe.MOE_ERR_UNSUPPORTED
    assert call(args(x=FAKE, H=12)) == moe.MOE_ERR_UNSUPPORTED
    assert call(args(x=MISALIGNED, H=16)) == moe.MOE_ERR_INVALID


def test_grouped_gemm_validation(lib):
    def call(dtype=0, N=128, K=128, cap=256, A=FAKE, src=NULL, div=1, B=FAKE, B2=NULL, lay=0,
             bg=FAKE, nr=FAKE, epi=0, rp=NULL, pw=NULL, k=0, D=FAKE, ws=FAKE, wsb=1 << 20):
        return lib.grouped_gemm(dtype, N, K, cap, A, src, div, B, B2, lay, bg, nr, epi, rp, pw, k, D,
                                ws, wsb, NULL)
    assert call(A=NULL) == moe.MOE_ERR_INVALID
    assert call(A=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(N=96) == moe.MOE_ERR_UNSUPPORTED
    assert call(K=100) == moe.MOE_ERR_UNSUPPORTED
    assert call(cap=200) == moe.MOE_ERR_INVALID
    assert call(dtype=5) == moe.MOE_ERR_UNSUPPORTED
    assert call(lay=3) == moe.MOE_ERR_UNSUPPORTED
    # gate/up interleaved in B: SiLU*up only, no B2, N a multiple of 128
    assert call(lay=2, epi=1, B2=FAKE) == moe.MOE_ERR_INVALID
    assert call(lay=2, epi=0) == moe.MOE_ERR_INVALID
    assert call(lay=2, epi=1, N=192) == moe.MOE_ERR_UNSUPPORTED
    # non-temporal weight loads: a flag on the [K][N] layouts only
    assert call(lay=1 | moe.MOE_B_STREAM) == moe.MOE_ERR_UNSUPPORTED
    assert call(lay=3 | moe.MOE_B_STREAM) == moe.MOE_ERR_UNSUPPORTED
    assert call(lay=2 | moe.MOE_B_STREAM, epi=1, B2=FAKE) == moe.MOE_ERR_INVALID
    assert call(lay=0x200) == moe.MOE_ERR_UNSUPPORTED
    assert call(epi=1) == moe.MOE_ERR_INVALID          # SiLU*up needs B2
    assert call(epi=7) == moe.MOE_ERR_UNSUPPORTED
    assert call(src=FAKE, div=0) == moe.MOE_ERR_INVALID
    assert call(ws=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(wsb=8) == moe.MOE_ERR_WORKSPACE
    # weighted scatter: needs the row -> pair map, the weights and k >= 1; [K][N] weights only
    assert call(epi=2) == moe.MOE_ERR_INVALID
    assert call(epi=2, rp=FAKE, pw=FAKE, k=0) == moe.MOE_ERR_INVALID
    assert call(epi=2, rp=FAKE, pw=NULL, k=2) == moe.MOE_ERR_INVALID
    assert call(epi=2, rp=FAKE, pw=FAKE, k=2, lay=1) == moe.MOE_ERR_UNSUPPORTED
    assert call(epi=3) == moe.MOE_ERR_UNSUPPORTED
    assert call(ws=NULL) == moe.MOE_ERR_WORKSPACE
    assert lib.grouped_gemm_workspace_size(256) > 0
    assert lib.grouped_gemm_workspace_size(0) == 0


def test_grouped_gemm_tuned_validation(lib):
    # the explicit launch shape of tests and sweeps: an instantiated tile that
    # fits the shape, or MOE_ERR_UNSUPPORTED (never a silent fallback)
    def call(tile=None, grid=0, N=512, K=256, epi=0, lay=0, B2=NULL, wsb=1 << 20, flags=0):
        t = None if tile is None else (ctypes.c_int32 * 6)(*tile)
        return lib.grouped_gemm_tuned(0, N, K, 256, FAKE, NULL, 1, FAKE, B2, lay, FAKE, FAKE, epi, NULL,
                                      NULL, 0, FAKE, t, grid, flags, FAKE, wsb, NULL)
    assert call(flags=1) == moe.MOE_ERR_DEVICE                          # plan ready; no GPU here
    assert call(flags=2) == moe.MOE_ERR_INVALID
    assert call(tile=(256, 32, 3, 6, 1, 8)) == moe.MOE_ERR_DEVICE      # valid; no GPU here
    assert call(tile=(256, 32, 3, 6, 1, 8), grid=8) == moe.MOE_ERR_DEVICE
    assert call(grid=-1) == moe.MOE_ERR_INVALID
    assert call(grid=65536) == moe.MOE_ERR_INVALID
    assert call(tile=(256, 32, 3, 7, 1, 4)) == moe.MOE_ERR_UNSUPPORTED  # not instantiated
    assert call(tile=(256, 64, 3, 6, 1, 4)) == moe.MOE_ERR_UNSUPPORTED  # 64-deep slices: not built
    assert call(tile=(256, 32, 3, 6, 1, 4), N=384) == moe.MOE_ERR_UNSUPPORTED  # 256 does not divide N
    assert call(tile=(256, 32, 3, 6, 1, 4), K=64) == moe.MOE_ERR_UNSUPPORTED  # ring unsafe for 2 slices
    assert call(tile=(256, 32, 3, 6, 0, 4)) == moe.MOE_ERR_UNSUPPORTED  # no row tasks per super-block
    assert call(tile=(128, 32, 3, 6, 1, 8), epi=1, B2=FAKE) == moe.MOE_ERR_DEVICE
    assert call(tile=(256, 32, 3, 6, 1, 8), epi=1, B2=FAKE) == moe.MOE_ERR_UNSUPPORTED  # SiLU*up: 128 max
    assert call(tile=(64, 32, 3, 10, 1, 4), epi=1, lay=2) == moe.MOE_ERR_DEVICE
    assert call(wsb=8) == moe.MOE_ERR_WORKSPACE


def test_grouped_gemm_noalloc_validation(lib):
    # the same checks as grouped_gemm, no workspace; the plan array holds up
    # to MOE_NOALLOC_MAX_CAP rows
    def call(cap=256, A=FAKE, epi=0, B2=NULL, lay=0):
        return lib.grouped_gemm_noalloc(0, 128, 128, cap, A, NULL, 1, FAKE, B2, lay, FAKE, FAKE, epi, NULL,
                                        NULL, 0, FAKE, NULL)
    assert call() == moe.MOE_ERR_DEVICE                      # valid; no GPU here
    assert call(cap=1 << 20) == moe.MOE_ERR_DEVICE
    assert call(cap=(1 << 20) + 128) == moe.MOE_ERR_WORKSPACE
    assert call(A=NULL) == moe.MOE_ERR_INVALID
    assert call(epi=1) == moe.MOE_ERR_INVALID               # SiLU*up needs B2
    assert call(lay=1 | moe.MOE_B_STREAM) == moe.MOE_ERR_UNSUPPORTED


def test_pack_gate_up_validation(lib):
    assert lib.moe_pack_gate_up(NULL, FAKE, 2, 64, 128, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_pack_gate_up(FAKE, FAKE, 2, 64, 128, NULL, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_pack_gate_up(FAKE, FAKE, 0, 64, 128, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_pack_gate_up(FAKE, MISALIGNED, 2, 64, 128, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_pack_gate_up(FAKE, FAKE, 2, 64, 64, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED


def test_finalize_validation(lib):
    assert lib.moe_finalize(NULL, 64, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_finalize(FAKE, 0, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_finalize(FAKE, 64, MISALIGNED, NULL) == moe.MOE_ERR_INVALID


def test_combine_and_layer_validation(lib):
    assert lib.moe_combine(NULL, 64, FAKE, FAKE, 4, 2, FAKE, NULL) == moe.MOE_ERR_INVALID
    assert lib.moe_combine(FAKE, 12, FAKE, FAKE, 4, 2, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(FAKE, 64, FAKE, FAKE, 4, 17, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    T, H, E, k, I = 64, 128, 8, 2, 64
    ws = lib.moe_layer_workspace_size(T, H, E, k, I)

    def call(x=FAKE, logits=FAKE, idx=NULL, w=NULL, H=H, I=I, k=k, wsb=ws):
        return lib.moe_layer(x, logits, idx, w, FAKE, FAKE, FAKE, T, H, E, k, I, FAKE, FAKE, wsb, NULL)
    assert call(x=NULL) == moe.MOE_ERR_INVALID
    assert call(logits=NULL) == moe.MOE_ERR_INVALID            # neither logits nor routing
    assert call(H=96) == moe.MOE_ERR_UNSUPPORTED
    assert call(I=80) == moe.MOE_ERR_UNSUPPORTED
    assert call(k=9) == moe.MOE_ERR_INVALID
    assert call(wsb=ws - 1) == moe.MOE_ERR_DEVICE               # the gather combine: no out_acc
    gather_ws = lib.moe_layer_workspace_size_ex(T, H, E, k, I, 0)
    assert call(wsb=gather_ws) == moe.MOE_ERR_DEVICE            # valid; no GPU here
    assert call(wsb=gather_ws - 1) == moe.MOE_ERR_WORKSPACE

    def call_ex(combine, wsb=ws, x=FAKE):
        return lib.moe_layer_ex(x, FAKE, NULL, NULL, FAKE, FAKE, FAKE, T, H, E, k, I, FAKE, combine,
                                FAKE, wsb, NULL)
    assert call_ex(2) == moe.MOE_ERR_UNSUPPORTED
    assert call_ex(-1) == moe.MOE_ERR_UNSUPPORTED
    assert call_ex(0x400) == moe.MOE_ERR_UNSUPPORTED           # an unknown flag
    # the flags take no workspace of their own: valid, and no GPU here
    for flags in (moe.MOE_LAYER_SEPARATE_PERMUTE, moe.MOE_LAYER_SPLIT_K,
                  moe.MOE_LAYER_SEPARATE_PERMUTE | moe.MOE_LAYER_SPLIT_K):
        assert call_ex(flags, wsb=gather_ws) == moe.MOE_ERR_DEVICE
        assert call_ex(1 | flags) == moe.MOE_ERR_DEVICE
        assert lib.moe_layer_workspace_size_ex(T, H, E, k, I, flags) == gather_ws
    assert call_ex(1, x=NULL) == moe.MOE_ERR_INVALID
    assert call_ex(1, wsb=ws - 1) == moe.MOE_ERR_WORKSPACE
    # w_up == NULL: packed gate/up weights, which need I % 128 == 0 (I = 64 here)
    assert lib.moe_layer(FAKE, FAKE, NULL, NULL, FAKE, NULL, FAKE, T, H, E, k, I, FAKE, FAKE, ws,
                         NULL) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_layer(FAKE, FAKE, NULL, NULL, NULL, NULL, FAKE, T, H, E, k, I, FAKE, FAKE, ws,
                         NULL) == moe.MOE_ERR_INVALID


def test_binding_constants_match_header():
    # the Python binding's status codes, enum values and layer flags are
    # the header's
    text = open(HEADER).read()
    defs = dict(re.findall(r"^#define\s+(MOE_[A-Z0-9_]+)\s+(0x[0-9a-fA-F]+|-?\d+)", text, re.M))
    names = [n for n in defs if hasattr(moe, n)]
    assert {"MOE_LAYER_SEPARATE_PERMUTE", "MOE_LAYER_SPLIT_K", "MOE_ERR_UNSUPPORTED"} <= set(names)
    for n in names:
        assert getattr(moe, n) == int(defs[n], 0), n


def test_layer_router_validation(lib):
    T, H, E, k, I = 64, 128, 8, 2, 64
    ws = lib.moe_layer_router_workspace_size(T, H, E, k, I, 0)
    lay = moe.layer_workspace_layout(T, H, E, k, I)
    # the layer's regions (without the scatter's accumulator), then the router's scratch
    assert ws == lay["out_acc"] + lib.moe_router_workspace_size(T, H, E)
    assert lib.moe_layer_router_workspace_size(T, H, E, k, I, 1) == \
        lay["total"] + lib.moe_router_workspace_size(T, H, E)
    assert lib.moe_layer_router_workspace_size(T, H, 200, k, I, 0) == 0   # E > 128: no router

    def call(x=FAKE, wr=FAKE, E=E, wsb=ws, combine=0):
        return lib.moe_layer_router(x, wr, FAKE, FAKE, FAKE, T, H, E, k, I, FAKE, combine, FAKE, wsb, NULL)
    assert call() == moe.MOE_ERR_DEVICE                 # valid; no GPU here
    assert call(wr=NULL) == moe.MOE_ERR_INVALID
    assert call(wr=MISALIGNED) == moe.MOE_ERR_INVALID
    assert call(x=NULL) == moe.MOE_ERR_INVALID
    assert call(E=200) == moe.MOE_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == moe.MOE_ERR_WORKSPACE
    assert call(combine=1) == moe.MOE_ERR_WORKSPACE      # the scatter needs its accumulator too
    assert call(combine=3) == moe.MOE_ERR_UNSUPPORTED


def test_valid_call_without_device_reports_device_error(lib):
    # only meaningful where no GPU is visible; on a GPU machine the call would launch
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.moe_route(FAKE, 4, 8, 2, FAKE, FAKE, NULL) == moe.MOE_ERR_DEVICE


def test_python_binding_fails_loudly_without_library(tmp_path):
    import importlib
    saved = moe._lib
    try:
        moe._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            moe.load_library(str(tmp_path / "missing.so"))
    finally:
        moe._lib = saved
