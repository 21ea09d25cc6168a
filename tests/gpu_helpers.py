"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same inputs, compare to the stated bar.

Bar (floating point, bf16 inputs and intermediates, fp32 accumulation):
max |out_gpu - out_oracle| <= 2e-2 and ||diff||_2 / ||out_oracle||_2 <= 5e-3.
Routing ids, counts and the permutation are integers and must match exactly,
except where the oracle's own fp32 probabilities are within 1e-6 of a tie
(the k-th and (k+1)-th, or two adjacent ranks among the first k+1); such
tokens are counted, their ids compared as sets where only the order inside
the top-k is in doubt, and their outputs compared against the oracle re-run
with the GPU's ids.
"""
from __future__ import annotations

import numpy as np
import torch

from expert_ffn_layer_amd import moe

# (case, max_abs, relL2, largest relative routing-weight error, near-ties)
# of the parity checks run in this session; printed at the end of the run.
RESULTS = []

MAX_ABS = 2e-2
REL_L2 = 5e-3
NEAR_TIE = 1e-6
# Routing weights / probabilities: the GPU sums the H-term logits in another
# fp32 order than the oracle (MFMA blocks, split-K partials), so logits
# differ by up to about 1e-5 at H = 4096..8192 and each renormalised weight
# moves by about 2*w*|dlogit|.  Measured largest relative weight error on the
# clear tokens of the full-size layers: 2.3e-5 (Ling-like, H = 8192), 1.4e-5
# (prefill), 9e-6 (skew), 3.3e-6 (decode); 0 on the small layers.  The bound
# is twice the largest.
W_RTOL = 5e-5
W_ATOL = 1e-6
DEV = "cuda"


def gpu_forward(layer, light_max_rows: int = -1, heavy_tile_rows: int = 0, y_bf16: bool = False,
                y_fp16: bool = False, packed: bool = False):
    """moe_forward on the layer; with ``packed`` the weights are handed over
    only as the packed copy (the plain layout is not passed)."""
    m = moe.MoELayer(layer, light_max_rows, heavy_tile_rows, y_bf16=y_bf16, y_fp16=y_fp16,
                     packed=packed)
    out, ids, w, counts = m()
    del m
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy(),
                counts=counts.cpu().numpy())


def err_stats(got, ref):
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(np.asarray(ref, np.float64)))
    rel = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, what=""):
    max_abs, rel = err_stats(got, ref)
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} relL2={rel:.3e}"
    return max_abs, rel


def routing_flags(ref):
    """(order_or_set_in_doubt, only_order_in_doubt) masks from the oracle gaps."""
    set_doubt = ref["gap_k"] < NEAR_TIE
    order_doubt = (ref["gap_in"] < NEAR_TIE) & ~set_doubt
    return set_doubt, order_doubt


def check_routing(gpu_ids, gpu_w, ref):
    set_doubt, order_doubt = routing_flags(ref)
    clean = ~(set_doubt | order_doubt)
    assert np.array_equal(gpu_ids[clean], ref["ids"][clean]), "routing ids differ on clear tokens"
    if order_doubt.any():
        assert np.array_equal(np.sort(gpu_ids[order_doubt], 1), np.sort(ref["ids"][order_doubt], 1))
    diff = np.abs(gpu_w[clean] - ref["w"][clean])
    tol = W_ATOL + W_RTOL * np.abs(ref["w"][clean])
    assert diff.size == 0 or np.all(diff <= tol), f"routing weights differ by {diff.max():.2e}"
    for row in gpu_ids:
        assert len(set(row.tolist())) == row.size
    return int(set_doubt.sum()), int(order_doubt.sum())


def weight_error(gpu_w, ref):
    """Largest |dw| - W_ATOL over |w| on the tokens whose routing is clear:
    the relative weight error the W_RTOL bound has to cover."""
    set_doubt, order_doubt = routing_flags(ref)
    clean = ~(set_doubt | order_doubt)
    if not clean.any():
        return 0.0
    d = np.abs(gpu_w[clean].astype(np.float64) - ref["w"][clean])
    return float(np.max(np.maximum(d - W_ATOL, 0.0) / np.maximum(np.abs(ref["w"][clean]), 1e-30)))


def check_layer(o, layer, tokens=None, light_max_rows: int = -1, full_routing=True,
                heavy_tile_rows: int = 0, y_bf16: bool = False, y_fp16: bool = False,
                packed: bool = False):
    """Run the layer on the GPU and compare with the oracle.  ``tokens``
    restricts the FFN/combine comparison to a sample of token rows; routing
    is compared on every token when ``full_routing``."""
    c = layer.cfg
    g = gpu_forward(layer, light_max_rows, heavy_tile_rows, y_bf16, y_fp16, packed)
    report = {}
    if full_routing:
        r_all = o.route(o.logits(layer.x, layer.wg, layer.bias), c.k, c.renorm)
        report["near_ties"] = check_routing(g["ids"], g["w"], r_all)
        report["w_rel"] = weight_error(g["w"], r_all)
        perm = o.permute(g["ids"], c.E)
        assert np.array_equal(g["counts"], perm["counts"]), "counts differ from oracle permute"
        assert int(g["counts"].sum()) == c.T * c.k
    tok = np.arange(c.T) if tokens is None else np.asarray(tokens)
    tok_t = torch.as_tensor(tok, device=layer.x.device)
    ref = o.forward(layer.x, layer.wg, layer.bias, layer.w_gu, layer.w_dn, c.k, c.renorm,
                    layer.ws_gu, layer.ws_dn, tokens=tok_t, permute=False)
    if not full_routing:
        report["near_ties"] = check_routing(g["ids"][tok], g["w"][tok], ref)
        report["w_rel"] = weight_error(g["w"][tok], ref)
    set_doubt, order_doubt = routing_flags(ref)
    flagged = set_doubt | order_doubt
    clean = ~flagged
    report["err"] = assert_close(g["out"][tok][clean], ref["out"][clean], "layer output")
    tag = (f"{c.name}[T={c.T} tokens={tok.size} light={light_max_rows} tm={heavy_tile_rows} "
           f"y={'bf16' if y_bf16 else ('fp16' if y_fp16 else 'fp32')}"
           f"{' packed' if packed else ''}]")
    RESULTS.append((tag, *report["err"], report.get("w_rel", 0.0), report["near_ties"]))
    if flagged.any():
        ft = torch.as_tensor(tok[flagged], device=layer.x.device)
        ref2 = o.forward(layer.x, layer.wg, layer.bias, layer.w_gu, layer.w_dn, c.k, c.renorm,
                         layer.ws_gu, layer.ws_dn, tokens=ft, ids=g["ids"][tok[flagged]],
                         permute=False)
        assert_close(g["out"][tok[flagged]], ref2["out"], "near-tie tokens")
    report["gpu"] = g
    return report
