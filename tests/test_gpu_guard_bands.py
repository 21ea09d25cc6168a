"""Guard bands around every buffer the library writes.

Each output (and the workspace) is placed between two 4 KB bands of a poison
byte; after the call the bands must be untouched.  The shapes are ragged on
purpose: a last heavy tile with few rows, H not a multiple of the 256-column
tile, I % 64 == 32 (a half-full last K stage in the down GEMM), token counts
that are not multiples of the combine's row groups, and a layer with both
light and heavy experts.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import moe, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

BAND = 4096
POISON = 0xA5


class Guarded:
    """A device buffer of `n` elements of `dtype` between two poison bands."""

    def __init__(self, n, dtype):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((nbytes + 2 * BAND,), POISON, dtype=torch.uint8, device=gh.DEV)
        self.nbytes = nbytes
        self.t = self.raw[BAND:BAND + nbytes].view(dtype)

    def check(self, what):
        r = self.raw.cpu().numpy()
        lo, hi = r[:BAND], r[BAND + self.nbytes:]
        assert np.all(lo == POISON), f"{what}: write before the buffer at byte {np.nonzero(lo != POISON)[0][-1] - BAND}"
        assert np.all(hi == POISON), f"{what}: write past the buffer at byte +{np.nonzero(hi != POISON)[0][0]}"


def guarded_ws(shape):
    g = Guarded(moe.workspace_bytes(shape), torch.uint8)
    return g


SHAPES = {
    # light and heavy experts, ragged tiles, I % 64 == 32
    "mixed": dict(T=203, H=320, E=48, k=10, I=96, zipf_s=1.2, zipf_alpha=0.6),
    # every expert light (T <= 64)
    "light": dict(T=33, H=192, E=64, k=6, I=160),
    # a shared expert and heavy tiles of every height
    "shared": dict(T=290, H=448, E=6, k=3, I=128, I_shared=96),
}


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("yf", ["fp32", "bf16"])
def test_stage_guard_bands(name, yf):
    print(f"[case] guard bands stages {name} y={yf}", flush=True)
    cfg = synth.custom_config(f"gb_{name}", **SHAPES[name])
    lay = synth.make_layer(cfg, seed=7, device=gh.DEV)
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    A = T * k
    s = moe.make_shape(T, H, E, k, I, cfg.I_shared, y_bf16=yf == "bf16")
    ws = guarded_ws(s)
    ids, w, probs = Guarded(A, torch.int32), Guarded(A, torch.float32), Guarded(T * E, torch.float32)
    moe.router(s, lay.x, lay.wg, lay.bias, ids.t, w.t, probs.t, ws.t)
    counts, offsets = Guarded(E, torch.int32), Guarded(E + 1, torch.int32)
    srt, inv = Guarded(A, torch.int32), Guarded(A, torch.int32)
    moe.permute(s, ids.t, counts.t, offsets.t, srt.t, inv.t, ws.t)
    h, y = Guarded(A * I, torch.bfloat16), Guarded(A * H, moe.y_dtype(s))
    moe.grouped_ffn(s, lay.x, srt.t, offsets.t, lay.w_gu, lay.w_dn, h.t, y.t, ws.t)
    out = Guarded(T * H, torch.float32)
    moe.combine(s, y.t, inv.t, w.t, 0, out.t)
    if cfg.I_shared:
        sh = Guarded(T * H, torch.float32)
        moe.shared_ffn(s, lay.x, lay.ws_gu, lay.ws_dn, sh.t, ws.t)
    torch.cuda.synchronize()
    for g, what in [(ws, "workspace"), (ids, "topk_ids"), (w, "topk_w"), (probs, "probs"),
                    (counts, "counts"), (offsets, "offsets"), (srt, "sorted_token_ids"),
                    (inv, "inv_pos"), (h, "h"), (y, "y"), (out, "out")]:
        g.check(what)
    if cfg.I_shared:
        sh.check("shared out")
    # the guarded run computed the same layer as moe_forward
    ref = moe.MoELayer(lay, y_bf16=yf == "bf16")()[0]
    torch.cuda.synchronize()
    if not cfg.I_shared:
        assert torch.equal(out.t.view(T, H), ref)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("packed", [False, True])
def test_forward_guard_bands(name, packed):
    print(f"[case] guard bands forward {name} packed={packed}", flush=True)
    cfg = synth.custom_config(f"gbf_{name}", **SHAPES[name])
    lay = synth.make_layer(cfg, seed=8, device=gh.DEV)
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    s = moe.make_shape(T, H, E, k, cfg.I, cfg.I_shared, y_bf16=1)
    ws = guarded_ws(s)
    pk = moe.pack_weights(s, lay.w_gu, lay.w_dn) if packed else None
    out, ids = Guarded(T * H, torch.float32), Guarded(T * k, torch.int32)
    w, counts = Guarded(T * k, torch.float32), Guarded(E, torch.int32)
    moe.forward(s, lay.x, lay.wg, lay.bias, None if packed else lay.w_gu,
                None if packed else lay.w_dn, lay.ws_gu, lay.ws_dn, out.t, ws.t, ids.t, w.t,
                counts.t, packed_weights=pk)
    torch.cuda.synchronize()
    for g, what in [(ws, "workspace"), (out, "out"), (ids, "topk_ids_out"),
                    (w, "topk_w_out"), (counts, "counts_out")]:
        g.check(what)
