"""The fused light loop (one persistent gate|up -> down launch with
per-expert readiness counters) against the default two launches.

``libmoe_fusedlight.so`` is the same source built with MOE_FUSED_LIGHT=1:
its light experts run as tickets of one kernel, gate|up items first, and a
down item waits until its expert's h is complete.  It runs the same item
code, so h, y and the layer output must equal the default build's bit for
bit; one case also meets the bar against the oracle.  It is kept out of the
default build because it is slower on MI355X (every item pays a write-back
or an invalidation of its XCD's L2 to pass h between XCDs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import build, moe, synth
from tests import gpu_helpers as gh
from tests.test_gpu_grid16 import _grouped

pytestmark = pytest.mark.gpu

# light-only layers (decode-like, one with 17..64-row experts), a mixed
# light/heavy one, and a k == E one where every expert is shared by all
# tokens; ragged I (I % 64 == 32) and H (H % 128 == 64)
CASES = {
    "decode": dict(T=64, H=1024, E=128, k=8, I=256),
    "wide": dict(T=48, H=320, E=4, k=2, I=96),
    "mixed": dict(T=400, H=384, E=64, k=6, I=160, zipf_s=1.2, zipf_alpha=1.5),
    "k_eq_e": dict(T=40, H=192, E=6, k=6, I=64),
}


def _both(fn):
    a = fn()
    with moe.using_library(build.FUSED_LIB):
        b = fn()
    return a, b


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("yf", ["fp32", "bf16"])
def test_fused_light_bitwise(name, yf):
    print(f"[case] fused light {name} y={yf}", flush=True)
    cfg = synth.custom_config(f"fl_{name}", **CASES[name])
    layer = synth.make_layer(cfg, seed=5, device=gh.DEV)
    yb = yf == "bf16"
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, light_max_rows=64, y_bf16=yb)
    (h0, y0), (h1, y1) = _both(lambda: _grouped(layer, s))
    assert np.array_equal(h0, h1), "h differs in the fused light loop"
    assert np.array_equal(y0, y1), "y differs in the fused light loop"

    def fwd(packed):
        outs = []
        m = moe.MoELayer(layer, light_max_rows=-1, y_bf16=yb, packed=packed)
        for _ in range(3):  # the counters start over on every call
            outs.append(m()[0].view(torch.int32).cpu().numpy())
        torch.cuda.synchronize()
        return outs

    for packed in (False, True):
        o0, o1 = _both(lambda: fwd(packed))
        for a, b in zip(o0, o1):
            assert np.array_equal(a, b), f"layer output differs (packed={packed})"


def test_fused_light_oracle(oracle_lib):
    cfg = synth.custom_config("fl_oracle", **CASES["decode"])
    layer = synth.make_layer(cfg, seed=5, device=gh.DEV)
    with moe.using_library(build.FUSED_LIB):
        rep = gh.check_layer(oracle_lib, layer, packed=True)
    ma, rel = rep["err"]
    print(f"[parity] fused light decode: max_abs={ma:.3e} relL2={rel:.3e}", flush=True)
