"""moe_forward_noalloc, the workspace-free entry point for callers that cannot
allocate, against moe_forward: the same kernels on the same inputs, so the
outputs and the routing must be equal bit for bit.  Two calls in a row on the
library's one scratch array, the second with a smaller layer (it runs on what
the first left behind), each with the plain and the packed weights; and a
shape whose scratch would not fit is refused before anything is written."""
from __future__ import annotations

import ctypes

import pytest
import torch

from expert_ffn_layer_amd import moe, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
# heavy tiles, a shared expert; then a smaller all-light layer
BIG = synth.custom_config("na_big", T=300, H=512, E=16, k=8, I=256, I_shared=128)
SMALL = synth.custom_config("na_small", T=40, H=256, E=32, k=4, I=128)


def _run(layer, shape, noalloc, packed):
    c = layer.cfg
    out = torch.full((c.T, c.H), float("nan"), dtype=torch.float32, device=DEV)
    ids = torch.full((c.T, c.k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((c.T, c.k), float("nan"), dtype=torch.float32, device=DEV)
    counts = torch.full((c.E,), -7, dtype=torch.int32, device=DEV)
    wgu, wdn = (None, None) if packed is not None else (layer.w_gu, layer.w_dn)
    if noalloc:
        moe.forward_noalloc(shape, layer.x, layer.wg, layer.bias, wgu, wdn, layer.ws_gu,
                            layer.ws_dn, out, ids, w, counts, packed_weights=packed)
    else:
        ws = moe.alloc_workspace(shape)
        moe.forward(shape, layer.x, layer.wg, layer.bias, wgu, wdn, layer.ws_gu, layer.ws_dn,
                    out, ws, ids, w, counts, packed_weights=packed)
    torch.cuda.synchronize()
    return out, ids, w, counts


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_forward(packed):
    for cfg, yb in ((BIG, True), (SMALL, False)):
        print(f"[case] noalloc {cfg.name} packed={packed}", flush=True)
        layer = synth.make_layer(cfg, seed=5, device=DEV)
        s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, y_bf16=yb)
        assert moe.workspace_bytes(s) <= moe.NOALLOC_SCRATCH_BYTES
        pk = moe.pack_weights(s, layer.w_gu, layer.w_dn) if packed else None
        got = _run(layer, s, True, pk)
        ref = _run(layer, s, False, pk)
        for g, r, name in zip(got, ref, ("out", "topk_ids", "topk_w", "counts")):
            gi = g.view(torch.int32) if g.dtype == torch.float32 else g
            ri = r.view(torch.int32) if r.dtype == torch.float32 else r
            assert torch.equal(gi, ri), f"{cfg.name}: {name} differs from moe_forward"


def test_noalloc_refuses_oversized_shape():
    """A shape needing more scratch than the fixed array: MOE_ERR_WORKSPACE
    before anything is enqueued (the output keeps its contents; the weight
    pointers, never read, stand in for a layer of that size)."""
    T, H, E, k, I = 4096, 4096, 512, 10, 1024
    s = moe.make_shape(T, H, E, k, I)
    assert moe.workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros((H, E), dtype=torch.float32, device=DEV)
    out = torch.full((T, H), 3.0, dtype=torch.float32, device=DEV)
    p = out.data_ptr()
    rc = moe.lib().moe_forward_noalloc(ctypes.byref(s), x.data_ptr(), wg.data_ptr(), None, p, p,
                                       None, None, None, p, None, None, None,
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == moe.MOE_ERR_WORKSPACE
    assert "MOE_NOALLOC_SCRATCH_BYTES" in moe.last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
