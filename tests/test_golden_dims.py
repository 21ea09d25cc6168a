"""The workloads' dimensions against the numbers the pages print
(tests/golden/pages_dims.json, each entry citing its page and section)."""
import json
import os

import numpy as np

from expert_ffn_layer_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_dims.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def test_qwen_dims():
    g = _g()["qwen35_moe"]
    for name in ("decode", "prefill", "prefill_long", "skew"):
        c = synth.CONFIGS[name]
        assert (c.H, c.E, c.k) == (g["hidden"], g["routed_experts"], g["top_k"])


def test_prefill_rows_match_pages(oracle_lib):
    """The prefill workload permutes exactly the pages' 81920 rows of width
    4096: T*k routed rows come out of the oracle's permutation."""
    g = _g()["prefill_permuted_rows"]
    c = synth.CONFIGS["prefill"]
    assert g["batched_tokens_per_rank"] * g["data_parallel"] * c.k == g["rows"]
    assert c.T * c.k == g["rows"] and c.H == g["hidden"]
    rng = np.random.default_rng(0)
    ids = np.argsort(rng.random((c.T, c.E)), axis=1)[:, :c.k].astype(np.int32)
    pm = oracle_lib.permute(ids, c.E)
    assert pm["sorted_token_ids"].shape == (g["rows"],) and pm["offsets"][-1] == g["rows"]


def test_experts_per_device():
    g = _g()["experts_per_device"]
    assert synth.CONFIGS["decode"].E // g["expert_parallel"] == g["value"]


def test_ling_dims():
    g = _g()["ling"]
    c = synth.CONFIGS["ling"]
    assert (c.E, c.k) == (g["routed_experts"], g["top_k"]) and c.I_shared > 0
