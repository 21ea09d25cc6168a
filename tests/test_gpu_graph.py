"""The layer under HIP graph capture: moe_forward makes no host synchronisation,
no allocation and no memset, so a captured forward replays on the stream it
was captured from.  Each replay is checked bit for bit against an eager call
on the same inputs, with eager calls and synchronisations between replays,
and once more after new inputs are copied into the captured buffer."""
from __future__ import annotations

import pytest
import torch

from expert_ffn_layer_amd import moe, synth

pytestmark = pytest.mark.gpu

CASES = {
    # every expert light (T <= 64): router, one-block permute, light loops, combine
    "light": synth.custom_config("g_light", T=40, H=256, E=64, k=4, I=192),
    # light and heavy experts: plan kernel, both loops, ragged tiles
    "mixed": synth.custom_config("g_mixed", T=203, H=256, E=48, k=10, I=128, zipf_s=1.2,
                                 zipf_alpha=0.6),
    # heavy tiles with ragged tails and a shared expert
    "shared": synth.custom_config("g_shared", T=300, H=320, E=16, k=4, I=96, I_shared=160),
}


def _run(m, x, out):
    o, ids, w, counts = m(x=x, out=out)
    return out, ids, w, counts


def _same(got, ref):
    return all(torch.equal(a, b) for a, b in zip(got, ref))


@pytest.mark.parametrize("weights", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays(name, weights):
    print(f"[case] graph {name} {weights}", flush=True)
    cfg = CASES[name]
    layer = synth.make_layer(cfg, seed=11, device="cuda")
    m = moe.MoELayer(layer, packed=True, weights=weights)
    x = layer.x.clone()  # the captured input buffer
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    eager = [t.clone() for t in _run(m, x, torch.empty_like(out))]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            _run(m, x, out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _run(m, x, out)

    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert _same(captured, eager), f"replay {rep} differs from the eager forward"
        # eager work between replays, on the same buffers' neighbours
        _run(m, x, torch.empty_like(out))
        torch.cuda.synchronize()

    # new activations in the captured buffer: the replay follows them
    x_new = synth.make_layer(cfg, seed=12, device="cuda", router_only=True).x
    x.copy_(x_new)
    g.replay()
    torch.cuda.synchronize()
    eager_new = [t.clone() for t in _run(m, x_new.clone(), torch.empty_like(out))]
    torch.cuda.synchronize()
    assert _same(captured, eager_new), "replay on new inputs differs from the eager forward"
    assert not torch.equal(eager_new[0], eager[0])
    del g
