"""The heavy kernels' cross-tile paths against their single-tile runs.

A block of the heavy grouped GEMM runs the work items wi, wi + stride, ...
of its XCD slice.  With one block per CU and the small shapes of the other
tests each block runs one item, so two paths would only run at full size:
the chaining of same-height tiles (the next tile's first loads overlap this
tile's stores) and the down GEMM's prefetch of the next tile's first stages
into the ring slots a tile frees (128- to 224-row tiles with I % 64 == 0,
in builds that write the down GEMM's y from registers; the default build
stages y through LDS instead, which the prefetch would need).
``libmoe_grid16.so`` is the same source built with the heavy grid capped at
16 blocks, so every block runs several items in a row, and
``libmoe_grid16_ns.so`` the same again with y unstaged (the prefetch on).
Their h, y and layer output must equal the default build's bit for bit (the
MFMA chains are the same whatever block runs a tile and however y is
written), and the capped builds meet the bar against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import build, moe, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

# (name, sizes): heavy experts of several tiles, N blocks per GEMM > 1, a
# ragged last tile; I % 64 == 0 (the down prefetch runs) and I % 64 == 32
# (a half-full last down stage), a shared expert (dense group, split h:
# K = 2 I for its down GEMM) and mixed light/heavy routing.
CASES = {
    "i128": dict(T=1200, H=768, E=6, k=2, I=256, I_shared=256),
    "i160": dict(T=1000, H=512, E=5, k=2, I=160, I_shared=96),
    "mixed": dict(T=900, H=384, E=40, k=6, I=128, zipf_s=1.2, zipf_alpha=1.5),
}


def _grouped(layer, shape):
    """Router, permute and grouped FFN of the active library: (h, y)."""
    c = layer.cfg
    A = c.T * c.k
    ws = moe.alloc_workspace(shape)
    ids = torch.empty((c.T, c.k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((c.T, c.k), dtype=torch.float32, device=gh.DEV)
    moe.router(shape, layer.x, layer.wg, layer.bias, ids, w, None, ws)
    t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
    counts, offsets, srt, inv = t(c.E), t(c.E + 1), t(A), t(A)
    moe.permute(shape, ids, counts, offsets, srt, inv, ws)
    h = torch.empty((A, c.I), dtype=torch.bfloat16, device=gh.DEV)
    y = torch.empty((A, c.H), dtype=moe.y_dtype(shape), device=gh.DEV)
    moe.grouped_ffn(shape, layer.x, srt, offsets, layer.w_gu, layer.w_dn, h, y, ws)
    torch.cuda.synchronize()
    yi = y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16)
    return h.view(torch.int16).cpu().numpy(), yi.cpu().numpy()


VARIANTS = {"staged": build.GRID16_LIB, "unstaged": build.GRID16_NS_LIB}


def _both(fn, lib=build.GRID16_LIB):
    """fn() under the default library and under a grid-capped one."""
    a = fn()
    with moe.using_library(lib):
        b = fn()
    return a, b


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("tm", [0, 128, 160, 192, 224, 256])
@pytest.mark.parametrize("yf", ["fp32", "bf16"])
def test_grid16_bitwise(name, tm, yf, variant):
    print(f"[case] grid16 {variant} {name} tm={tm} y={yf}", flush=True)
    lib = VARIANTS[variant]
    cfg = synth.custom_config(f"g16_{name}", **CASES[name])
    layer = synth.make_layer(cfg, seed=3, device=gh.DEV)
    yb = yf == "bf16"
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, light_max_rows=0,
                       heavy_tile_rows=tm, y_bf16=yb)
    (h0, y0), (h1, y1) = _both(lambda: _grouped(layer, s), lib)
    assert np.array_equal(h0, h1), "h differs with the capped grid"
    assert np.array_equal(y0, y1), "y differs with the capped grid"

    def fwd(packed):
        m = moe.MoELayer(layer, light_max_rows=-1, heavy_tile_rows=tm, y_bf16=yb, packed=packed)
        out = m()[0]
        torch.cuda.synchronize()
        return out.view(torch.int32).cpu().numpy()

    for packed in (False, True):
        o0, o1 = _both(lambda: fwd(packed), lib)
        assert np.array_equal(o0, o1), f"layer output differs with the capped grid (packed={packed})"
    if tm <= 192:  # MXFP8 heavy tiles are at most 192 rows high

        def fwd8():
            out = moe.MoELayer(layer, light_max_rows=-1, heavy_tile_rows=tm, y_bf16=yb,
                               weights="mxfp8")()[0]
            torch.cuda.synchronize()
            return out.view(torch.int32).cpu().numpy()

        o0, o1 = _both(fwd8, lib)
        assert np.array_equal(o0, o1), "MXFP8 layer output differs with the capped grid"


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_grid16_oracle(oracle_lib, variant):
    """The capped builds against the oracle on one case (the bitwise tests
    above tie them to the default build everywhere else)."""
    cfg = synth.custom_config("g16_oracle", **CASES["i128"])
    layer = synth.make_layer(cfg, seed=3, device=gh.DEV)
    with moe.using_library(VARIANTS[variant]):
        rep = gh.check_layer(oracle_lib, layer, heavy_tile_rows=128)
    ma, rel = rep["err"]
    print(f"[parity] grid16 {variant} i128/128: max_abs={ma:.3e} relL2={rel:.3e}", flush=True)
