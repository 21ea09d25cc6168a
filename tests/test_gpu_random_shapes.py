"""Seeded random layers within the ABI's limits against the oracle.

Each case draws its sizes from a fixed seed (so a failure names a
reproducible case): T 1..400, H a multiple of 64 up to 512, E 1..96, k up to
min(E, 12), I a multiple of 32 up to 320, an optional shared expert, optional
Zipf routing skew, the light threshold (default rule, all heavy, 16, 64),
the heavy tile height (chosen, 128..256) and the y storage; odd cases read
the packed weight records (and must equal the plain layout bit for bit).  Routing
must match exactly (near-ties flagged) and the output meet the 2e-2 /
5e-3 bar.
"""
from __future__ import annotations

import numpy as np
import pytest

from expert_ffn_layer_amd import synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_case(i):
    r = np.random.default_rng(1000 + i)
    E = int(r.integers(1, 97))
    kw = dict(T=int(r.integers(1, 401)), H=64 * int(r.integers(1, 9)), E=E,
              k=int(r.integers(1, min(E, 12) + 1)), I=32 * int(r.integers(1, 11)))
    if r.random() < 0.25:
        kw["I_shared"] = 32 * int(r.integers(1, 11))
    if r.random() < 0.35:
        kw.update(zipf_s=1.2, zipf_alpha=float(r.choice([0.6, 1.5, 3.0])))
    if r.random() < 0.15:
        kw["renorm"] = 0
    lm = int(r.choice([-1, -1, 0, 16, 64]))
    tm = int(r.choice([0, 0, 128, 160, 192, 224, 256]))
    yf = str(r.choice(["fp32", "bf16", "fp16"]))
    return kw, lm, tm, yf


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer(oracle_lib, i):
    kw, lm, tm, yf = draw_case(i)
    packed = i % 2 == 1
    print(f"[case] random {i}: {kw} light_max={lm} tm={tm} y={yf} packed={packed}", flush=True)
    cfg = synth.custom_config(f"rand{i}", **kw)
    layer = synth.make_layer(cfg, seed=i, device=gh.DEV)
    rep = gh.check_layer(oracle_lib, layer, light_max_rows=lm, heavy_tile_rows=tm,
                         y_bf16=yf == "bf16", y_fp16=yf == "fp16", packed=packed)
    if packed:  # the packed records give the plain layout's bits
        import torch

        from expert_ffn_layer_amd import moe
        outs = [moe.MoELayer(layer, lm, tm, y_bf16=yf == "bf16", y_fp16=yf == "fp16",
                             packed=pk)()[0] for pk in (False, True)]
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    ma, rel = rep["err"]
    print(f"[parity] random {i}: near_ties={rep['near_ties']} max_abs={ma:.3e} relL2={rel:.3e}",
          flush=True)


N_MX_CASES = 8


@pytest.mark.parametrize("i", range(N_MX_CASES))
def test_random_layer_mxfp8(oracle_lib, i):
    """MXFP8 expert weights on random layers: the layer equals, bit for bit,
    the bf16 layer on the oracle's dequantisation of the same weights, and
    that layer meets the bar against the oracle."""
    import torch

    from expert_ffn_layer_amd import moe
    from tests.test_gpu_mxfp8 import dequant_layer

    kw, lm, tm, yf = draw_case(500 + i)
    tm = 0 if tm > 192 else tm  # MXFP8 tiles are at most 192 rows high
    print(f"[case] random mxfp8 {i}: {kw} light_max={lm} tm={tm} y={yf}", flush=True)
    cfg = synth.custom_config(f"randmx{i}", **kw)
    layer = synth.make_layer(cfg, seed=500 + i, device=gh.DEV)
    ref = dequant_layer(oracle_lib, layer)
    yb, yh = yf == "bf16", yf == "fp16"
    out_mx = moe.MoELayer(layer, lm, tm, y_bf16=yb, y_fp16=yh, weights="mxfp8")()
    out_16 = moe.MoELayer(ref, lm, tm, y_bf16=yb, y_fp16=yh)()
    torch.cuda.synchronize()
    assert torch.equal(out_mx[1], out_16[1])
    assert torch.equal(out_mx[0].view(torch.int32), out_16[0].view(torch.int32)), \
        "MXFP8 layer differs from the bf16 layer on dequantised weights"
    rep = gh.check_layer(oracle_lib, ref, light_max_rows=lm, heavy_tile_rows=tm, y_bf16=yb,
                         y_fp16=yh)
    ma, rel = rep["err"]
    print(f"[parity] random mxfp8 {i}: near_ties={rep['near_ties']} max_abs={ma:.3e} "
          f"relL2={rel:.3e}", flush=True)
