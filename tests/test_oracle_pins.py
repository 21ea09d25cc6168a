"""The CPU oracle against its pins (library routines, closed forms,
invariants, brute force).  Runs without a GPU."""
import numpy as np
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_thread_count_independence(oracle_lib):
    """OpenMP splits only independent rows: 1 thread and many agree bitwise."""
    x, wg, w_gu, w_dn = oracle_pins.rand_layer(21, 33, 64, 8, 3, 32)
    n = oracle_lib.max_threads()
    try:
        oracle_lib.set_threads(1)
        a = oracle_lib.forward(x, wg, None, w_gu, w_dn, 3)
        oracle_lib.set_threads(max(n, 4))
        b = oracle_lib.forward(x, wg, None, w_gu, w_dn, 3)
    finally:
        oracle_lib.set_threads(n)
    for key in ("logits", "ids", "w", "out", "sorted_token_ids", "inv_pos"):
        assert np.array_equal(a[key], b[key]), key


def test_expert_major_equals_row_by_row(oracle_lib):
    """Evaluating the routed rows expert by expert gives the same bits as
    evaluating each (token, slot) row on its own."""
    x, wg, w_gu, w_dn = oracle_pins.rand_layer(22, 9, 64, 5, 2, 32)
    res = oracle_lib.forward(x, wg, None, w_gu, w_dn, 2)
    for t in range(9):
        for j in range(2):
            e = res["ids"][t, j]
            y = oracle_lib.expert_ffn(x[t:t + 1], w_gu[e], w_dn[e])
            assert np.array_equal(y[0], res["y"][t * 2 + j])


def test_forced_ids_weights(oracle_lib):
    """weights_for_ids on the oracle's own ids reproduces its weights."""
    rng = np.random.default_rng(23)
    lg = rng.standard_normal((20, 64)).astype(np.float32)
    r = oracle_lib.route(lg, 10, 1)
    assert np.array_equal(oracle_lib.weights_for_ids(lg, r["ids"], 1), r["w"])
