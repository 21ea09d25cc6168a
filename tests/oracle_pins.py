"""Pins of the CPU oracle to facts other than itself.

Each pin checks the oracle against something it does not compute itself:
a library routine (numpy's stable sort and float64 matmul), a closed form,
an invariant of the permutation, an exact special case, or brute force on a
tiny layer.  They are chosen so that a plausible mistake anywhere in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a broken
tie rule) fails at least one of them; ``tests/test_oracle_mutants.py`` plants
such mistakes in copies of the oracle and checks exactly that.

Every pin takes an ``oracle.Oracle`` and raises AssertionError on failure.
Inputs are numpy-only so the battery also runs in a bare subprocess.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- helpers
def silu64(z):
    return z / (1.0 + np.exp(-z))


def softmax64(l):
    l = np.asarray(l, np.float64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def ffn64(x, w_gu, w_dn):
    """One expert's SwiGLU FFN in float64 with library matmuls."""
    x = np.asarray(x, np.float64)
    w_gu = np.asarray(w_gu, np.float64)
    w_dn = np.asarray(w_dn, np.float64)
    I = w_gu.shape[0] // 2
    g = x @ w_gu[:I].T
    u = x @ w_gu[I:].T
    return (silu64(g) * u) @ w_dn.T


def topk_by_sort(p, k):
    """First k of a stable sort by descending p; equal p keep ascending id."""
    order = np.argsort(-np.asarray(p, np.float64), axis=-1, kind="stable")
    return order[..., :k]


def rand_layer(seed, T, H, E, k, I, gstd=0.1, wstd=0.05):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((H, E)) * gstd).astype(np.float32)
    w_gu = (rng.standard_normal((E, 2 * I, H)) * wstd).astype(np.float32)
    w_dn = (rng.standard_normal((E, H, I)) * wstd).astype(np.float32)
    return x, wg, w_gu, w_dn


def rel_max(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


# ------------------------------------------------------------------- pins
def pin_logits_vs_library(o):
    """Router projection against float64 matmul (+ bias)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 96)).astype(np.float32)
    wg = (rng.standard_normal((96, 33)) * 0.1).astype(np.float32)
    b = rng.standard_normal(33).astype(np.float32)
    ref = x.astype(np.float64) @ wg.astype(np.float64) + b
    got = o.logits(x, wg, b)
    scale = np.abs(x).astype(np.float64) @ np.abs(wg).astype(np.float64) + np.abs(b)
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-7), "logits != x@wg+b"


def pin_topk_full_sort(o):
    """Top-k ids are the first k of a full stable sort by probability, with
    exact ties (quantised logits) going to the lower id; probabilities and
    renormalised weights match float64."""
    rng = np.random.default_rng(2)
    for T, E, k, quant in [(40, 8, 2, False), (40, 512, 10, False), (30, 256, 8, False),
                           (20, 7, 7, False), (10, 1000, 32, False), (40, 64, 10, True),
                           (40, 13, 5, True)]:
        l = rng.standard_normal((T, E)).astype(np.float32)
        if quant:
            l = (rng.integers(0, 4, (T, E)) * 0.5).astype(np.float32)
        r = o.route(l, k, 1)
        assert np.array_equal(r["ids"], topk_by_sort(r["probs"], k)), f"top-k order {T,E,k}"
        p64 = softmax64(l)
        assert rel_max(r["probs"], p64) < 1e-6, "softmax"
        # ids agree with a sort of the float64 probabilities wherever the
        # float64 k-th/k+1-th gap is clear of fp32 rounding
        order64 = np.argsort(-p64, axis=-1, kind="stable")
        if k < E:
            srt = -np.sort(-p64, axis=-1)
            clear = (srt[:, k - 1] - srt[:, k]) > 1e-6
            for t in np.nonzero(clear)[0]:
                assert set(order64[t, :k]) == set(r["ids"][t]), "top-k set vs float64"
        psel = np.take_along_axis(p64, r["ids"].astype(np.int64), axis=1)
        w64 = psel / psel.sum(axis=1, keepdims=True)
        assert np.abs(r["w"] - w64).max() < 2e-6, "renormalised weights"
        assert np.all(np.abs(r["w"].astype(np.float64).sum(1) - 1) < 1e-5)


def pin_tie_rule(o):
    """All-equal logits: ids 0..k-1 and w = 1/k exactly (E a power of 2)."""
    for E, k in [(8, 2), (512, 10), (256, 8), (64, 64)]:
        r = o.route(np.zeros((3, E), np.float32), k, 1)
        assert np.array_equal(r["ids"], np.tile(np.arange(k, dtype=np.int32), (3, 1)))
        assert np.all(r["w"] == np.float32(1.0) / np.float32(k)), "w = 1/k"


def pin_bias_only(o):
    """x = 0: the logits are the bias exactly; ids are the top-k of the bias."""
    rng = np.random.default_rng(3)
    E, k, H = 40, 6, 32
    b = rng.permutation(E).astype(np.float32) * 0.25 - 3.0
    x = np.zeros((4, H), np.float32)
    wg = rng.standard_normal((H, E)).astype(np.float32)
    lg = o.logits(x, wg, b)
    assert np.array_equal(lg, np.tile(b, (4, 1))), "bias not added exactly"
    r = o.route(lg, k, 1)
    assert np.array_equal(r["ids"][0], np.argsort(-b, kind="stable")[:k])


def pin_nonfinite(o):
    """NaN counts as -inf; +inf entries share all mass; all -inf is uniform.
    Ids stay distinct and in range."""
    E, k = 16, 4
    l = np.zeros((5, E), np.float32)
    l[0, :] = np.nan
    l[1, 5] = np.inf
    l[1, 9] = np.nan
    l[2, :] = -np.inf
    l[3, :] = np.arange(E, dtype=np.float32)
    l[3, 2] = np.nan
    l[3, 11] = np.inf
    l[3, 12] = np.inf
    l[4, :] = np.arange(E, dtype=np.float32) * 0.125
    l[4, 15] = np.nan
    r = o.route(l, k, 1)
    assert np.array_equal(r["ids"][0], np.arange(k)), "all-NaN row"
    assert r["ids"][1][0] == 5 and r["w"][1][0] == 1.0 and np.all(r["w"][1][1:] == 0)
    assert np.array_equal(r["ids"][1][1:], [0, 1, 2])
    assert np.array_equal(r["ids"][2], np.arange(k)), "all -inf row"
    assert np.all(r["w"][2] == np.float32(0.25))
    assert np.array_equal(r["ids"][3][:2], [11, 12]) and np.all(r["w"][3][:2] == 0.5)
    assert np.array_equal(r["ids"][3][2:], [0, 1])
    assert np.array_equal(r["ids"][4], [14, 13, 12, 11]) and r["probs"][4][15] == 0
    ref = softmax64(l[4, :15])
    assert rel_max(r["probs"][4][:15], ref) < 1e-6, "NaN row softmax"
    for row in r["ids"]:
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < E


def pin_large_logits(o):
    """Softmax of logits near 500 stays finite and exact (needs the max shift)."""
    rng = np.random.default_rng(4)
    l = (500.0 + rng.standard_normal((5, 32))).astype(np.float32)
    r = o.route(l, 3, 1)
    assert np.all(np.isfinite(r["probs"])) and rel_max(r["probs"], softmax64(l)) < 1e-5


def pin_renorm_off(o):
    """renorm = 0: the weights are the softmax probabilities of the ids."""
    rng = np.random.default_rng(5)
    l = rng.standard_normal((6, 20)).astype(np.float32)
    r = o.route(l, 5, 0)
    assert np.array_equal(r["w"], np.take_along_axis(r["probs"], r["ids"].astype(np.int64), 1))


def pin_weights_for_ids(o):
    """Routing weights of ids that are not the oracle's own top-k (the k-th
    and (k+1)-th ranks swapped, the order reversed, random distinct ids):
    the float64 softmax probabilities of exactly those ids, renormalised over
    them (renorm 1) or raw (renorm 0)."""
    rng = np.random.default_rng(24)
    for T, E, k in [(30, 64, 10), (12, 512, 10), (10, 16, 4), (6, 9, 8)]:
        l = (rng.standard_normal((T, E)) * 2.0).astype(np.float32)
        p64 = softmax64(l)
        top = topk_by_sort(p64, k + 1)
        swapped = top[:, :k].copy()
        swapped[:, k - 1] = top[:, k]
        variants = {
            "swapped": swapped,
            "reversed": top[:, :k][:, ::-1],
            "random": np.stack([rng.permutation(E)[:k] for _ in range(T)]),
        }
        for name, ids in variants.items():
            ids = np.ascontiguousarray(ids, dtype=np.int32)
            psel = np.take_along_axis(p64, ids.astype(np.int64), axis=1)
            w1 = o.weights_for_ids(l, ids, 1)
            want1 = psel / psel.sum(axis=1, keepdims=True)
            assert np.abs(w1 - want1).max() < 2e-6, f"renormalised weights of {name} ids"
            w0 = o.weights_for_ids(l, ids, 0)
            assert rel_max(w0, psel) < 1e-6, f"raw probabilities of {name} ids"


def pin_permute(o):
    """Counts sum to T*k, every token appears exactly k times, each expert's
    segment lists its tokens in increasing order, inv_pos is a bijection that
    points back at the token and lies in its expert's segment, and the whole
    equals numpy's stable argsort of the flattened ids."""
    rng = np.random.default_rng(6)
    for T, E, k in [(1, 4, 1), (37, 16, 3), (64, 512, 10), (300, 8, 8), (5, 1024, 32)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        pm = o.permute(ids, E)
        flat = ids.reshape(-1)
        A = T * k
        assert pm["counts"].sum() == A
        assert np.array_equal(pm["counts"], np.bincount(flat, minlength=E))
        assert pm["offsets"][0] == 0 and pm["offsets"][-1] == A
        assert np.array_equal(np.diff(pm["offsets"]), pm["counts"])
        srt = pm["sorted_token_ids"]
        assert np.array_equal(np.bincount(srt, minlength=T), np.full(T, k))
        for e in range(E):
            seg = srt[pm["offsets"][e]:pm["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)
        inv = pm["inv_pos"]
        assert np.array_equal(np.sort(inv), np.arange(A))
        a = np.arange(A)
        assert np.array_equal(srt[inv], a // k)
        assert np.all(inv >= pm["offsets"][flat]) and np.all(inv < pm["offsets"][flat + 1])
        ref = np.argsort(flat, kind="stable")
        assert np.array_equal(srt, ref // k) and np.array_equal(inv[ref], a)


def pin_k1_single_expert(o):
    """k = 1: the weight is 1 and the layer is the selected expert's FFN."""
    x, wg, w_gu, w_dn = rand_layer(7, 12, 64, 6, 1, 48)
    res = o.forward(x, wg, None, w_gu, w_dn, 1)
    assert np.all(res["w"] == 1.0)
    lg64 = x.astype(np.float64) @ wg.astype(np.float64)
    srt = -np.sort(-lg64, axis=1)
    assert np.all(srt[:, 0] - srt[:, 1] > 1e-4), "seed has a near-tie"
    assert np.array_equal(res["ids"][:, 0], lg64.argmax(1))
    ref = np.stack([ffn64(x[t:t + 1], w_gu[e], w_dn[e])[0]
                    for t, e in enumerate(res["ids"][:, 0])])
    assert rel_max(res["out"], ref) < 1e-5


def pin_identical_experts(o):
    """All experts equal: the output is one dense FFN whatever the routing."""
    x, wg, w_gu, w_dn = rand_layer(8, 10, 64, 8, 3, 32)
    w_gu[:] = w_gu[0]
    w_dn[:] = w_dn[0]
    res = o.forward(x, wg, None, w_gu, w_dn, 3)
    assert rel_max(res["out"], ffn64(x, w_gu[0], w_dn[0])) < 1e-5


def pin_zero_weights(o):
    """W_down = 0 or W_gate = 0 gives exactly zero output."""
    x, wg, w_gu, w_dn = rand_layer(9, 8, 64, 4, 2, 32)
    res = o.forward(x, wg, None, w_gu, np.zeros_like(w_dn), 2)
    assert np.all(res["out"] == 0)
    g0 = w_gu.copy()
    g0[:, :32] = 0
    res = o.forward(x, wg, None, g0, w_dn, 2)
    assert np.all(res["out"] == 0)


def pin_identity_weights(o):
    """I = H with W_gate = W_up = W_down = identity: out = silu(x) * x."""
    H = 32
    x, wg, _, _ = rand_layer(10, 7, H, 5, 2, H)
    eye = np.eye(H, dtype=np.float32)
    w_gu = np.tile(np.concatenate([eye, eye])[None], (5, 1, 1))
    w_dn = np.tile(eye[None], (5, 1, 1))
    res = o.forward(x, wg, None, w_gu, w_dn, 2)
    x64 = x.astype(np.float64)
    assert rel_max(res["out"], silu64(x64) * x64) < 1e-6


def pin_dense_bruteforce(o):
    """Tiny layer against a float64 dense brute force: every expert applied
    to every token, masked by the renormalised top-k gate."""
    T, H, E, k, I = 16, 64, 8, 2, 32
    x, wg, w_gu, w_dn = rand_layer(11, T, H, E, k, I)
    b = (np.random.default_rng(12).standard_normal(E) * 0.3).astype(np.float32)
    res = o.forward(x, wg, b, w_gu, w_dn, k)
    lg = x.astype(np.float64) @ wg.astype(np.float64) + b
    p = softmax64(lg)
    srt = -np.sort(-p, axis=1)
    assert np.all(srt[:, k - 1] - srt[:, k] > 1e-5), "seed has a near-tie"
    ids = topk_by_sort(p, k)
    gate = np.zeros((T, E))
    for t in range(T):
        gate[t, ids[t]] = p[t, ids[t]] / p[t, ids[t]].sum()
    dense = np.stack([ffn64(x, w_gu[e], w_dn[e]) for e in range(E)], axis=1)  # [T,E,H]
    ref = np.einsum("te,teh->th", gate, dense)
    assert np.array_equal(np.sort(res["ids"], 1), np.sort(ids, 1))
    assert rel_max(res["out"], ref) < 1e-5


def pin_shared_expert(o):
    """With a shared expert, out = shared FFN + routed sum."""
    x, wg, w_gu, w_dn = rand_layer(13, 9, 64, 6, 2, 32)
    rng = np.random.default_rng(14)
    s_gu = (rng.standard_normal((2 * 48, 64)) * 0.05).astype(np.float32)
    s_dn = (rng.standard_normal((64, 48)) * 0.05).astype(np.float32)
    with_s = o.forward(x, wg, None, w_gu, w_dn, 2, ws_gu=s_gu, ws_dn=s_dn)
    without = o.forward(x, wg, None, w_gu, w_dn, 2)
    assert rel_max(with_s["out"] - without["out"], ffn64(x, s_gu, s_dn)) < 1e-5
    only_s = o.forward(x, wg, None, w_gu, np.zeros_like(w_dn), 2, ws_gu=s_gu, ws_dn=s_dn)
    assert rel_max(only_s["out"], ffn64(x, s_gu, s_dn)) < 1e-5


def pin_exact_scaling(o):
    """Doubling W_down doubles the output bitwise (power-of-2 scaling)."""
    x, wg, w_gu, w_dn = rand_layer(15, 11, 64, 8, 3, 32)
    a = o.forward(x, wg, None, w_gu, w_dn, 3)["out"]
    b = o.forward(x, wg, None, w_gu, 2 * w_dn, 3)["out"]
    assert np.array_equal(2 * a, b)


def pin_token_permutation(o):
    """Permuting the tokens permutes the output rows bitwise."""
    x, wg, w_gu, w_dn = rand_layer(16, 13, 64, 8, 3, 32)
    perm = np.random.default_rng(17).permutation(13)
    a = o.forward(x, wg, None, w_gu, w_dn, 3)
    b = o.forward(x[perm], wg, None, w_gu, w_dn, 3)
    assert np.array_equal(a["out"][perm], b["out"])
    assert np.array_equal(a["ids"][perm], b["ids"])


def pin_ffn_closed_form(o):
    """H = I = 1: FFN(x) = w_d * silu(w_g x) * (w_u x) evaluated by hand."""
    xs = np.array([[-3.0], [-0.5], [0.0], [0.75], [4.0]], np.float32)
    w_gu = np.array([[1.5], [-2.0]], np.float32)
    w_dn = np.array([[0.25]], np.float32)
    y = o.expert_ffn(xs, w_gu, w_dn)
    for v, got in zip(xs[:, 0].astype(np.float64), y[:, 0]):
        g, u = 1.5 * v, -2.0 * v
        ref = 0.25 * (g / (1.0 + np.exp(-g))) * u
        assert abs(got - ref) <= 1e-6 * max(1.0, abs(ref))


# ------------------------------------------------------- MXFP8 weights
def _e4m3_library_table():
    """Values of the 256 FP8 E4M3 codes from torch's float8_e4m3fn (a
    library's decoding of the same OCP format), float64."""
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy() \
        .astype(np.float64)


def _e4m3_library_round(v):
    """torch's round-to-nearest-even cast of fp32 values to E4M3 codes (it is
    not saturating: only |v| < 464 is meaningful)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def pin_mxfp8_decode_table(o):
    """Every code, at scale 2^0, decodes to the library's E4M3 value (NaN
    codes included); a scale code c multiplies by 2^(c-127)."""
    tab = _e4m3_library_table()
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    got = o.mxfp8_dequantize(codes, np.full((8, 1), 127, np.uint8)).astype(np.float64)
    assert np.array_equal(got.reshape(-1), tab, equal_nan=True)
    for sc in (100, 127 - 9, 131, 140):
        got = o.mxfp8_dequantize(codes, np.full((8, 1), sc, np.uint8)).astype(np.float64)
        assert np.array_equal(got.reshape(-1), tab * 2.0 ** (sc - 127), equal_nan=True)


def pin_mxfp8_rounding_vs_library(o):
    """With the block scale at 2^0 (an anchor of 300 in every block), element
    codes equal the library's nearest-even cast: random magnitudes over the
    subnormal and normal ranges, every representable value, every midpoint
    between neighbours (ties), both signs, signed zeros."""
    tab = _e4m3_library_table()[:127]           # codes 0..126: 0 .. 448 ascending
    mids = (tab[:-1] + tab[1:]) / 2
    rng = np.random.default_rng(21)
    mags = 2.0 ** rng.uniform(-12.0, np.log2(463.0), size=31 * 40)
    vals = np.concatenate([mags * rng.choice([-1.0, 1.0], mags.size), mids, -mids, tab, -tab,
                           [0.0, -0.0, 463.0, -463.0]])
    vals = np.concatenate([vals, np.zeros((-vals.size) % 31)])
    blocks = np.concatenate([vals.reshape(-1, 31), np.full((vals.size // 31, 1), 300.0)], 1)
    blocks = blocks.astype(np.float32)
    codes, scales = o.mxfp8_quantize(blocks)
    assert np.all(scales == 127)
    assert np.array_equal(codes, _e4m3_library_round(blocks))


def pin_mxfp8_saturation(o):
    """Past 448 (after scaling) elements saturate to +-448 (codes 0x7E/0xFE);
    a block maximum of 512 moves the scale up one binade instead."""
    b = np.zeros((2, 32), np.float32)
    b[0, :6] = [511.0, 500.0, -470.0, 449.0, -448.5, 1.0]
    b[1, :3] = [512.0, -300.0, 1.0]
    codes, scales = o.mxfp8_quantize(b)
    assert scales[0, 0] == 127 and scales[1, 0] == 128
    assert list(codes[0, :6]) == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x38]
    d = o.mxfp8_dequantize(codes, scales)
    assert list(d[0, :5]) == [448.0, 448.0, -448.0, 448.0, -448.0]
    assert list(d[1, :3]) == [512.0, -288.0, 1.0]      # -150 -> -144 (spacing 16), x 2


def pin_mxfp8_scale_rule(o):
    """Block scale = floor(log2 max|v|) - 8 (numpy's log2), clamped at -127
    (zero blocks and tiny blocks): max |v| / X then lies in [256, 512)."""
    rng = np.random.default_rng(22)
    nb = 400
    e = rng.integers(-40, 40, size=nb)
    b = rng.standard_normal((nb, 32)) * 2.0 ** e[:, None]
    b[::7, 5] = 2.0 ** e[::7]                              # exact powers of two as maxima
    b[::7] = np.where(np.arange(32) == 5, b[::7], b[::7] * 1e-3)
    b[3] = 0.0
    b[4] = 0.0
    b[4, 9] = -(2.0 ** -140)
    b = b.astype(np.float32)
    codes, scales = o.mxfp8_quantize(b)
    amax = np.abs(b.astype(np.float64)).max(1)
    with np.errstate(divide="ignore"):
        want = np.where(amax > 0, np.floor(np.log2(amax)) - 8, -127)
    want = np.clip(want, -127, 127)
    assert np.array_equal(scales[:, 0].astype(np.int64) - 127, want.astype(np.int64))
    ok = want > -127
    ratio = amax[ok] / 2.0 ** want[ok]
    assert np.all((ratio >= 256) & (ratio < 512))
    assert np.all(codes[3] == 0)


def pin_mxfp8_nearest_bruteforce(o):
    """Each element is the finite E4M3 value nearest to v / X by exhaustive
    search over the library's table (ties to the even code), or +-448 past
    the range; bf16-valued weights as the layer uses them."""
    tab = _e4m3_library_table()[:127]
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    w[5, :32] *= 1e-3
    w[6, 32:] = np.round(w[6, 32:] * 4096) / 4096          # many exact ties after scaling
    w = (w.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # bf16 values
    codes, scales = o.mxfp8_quantize(w)
    X = 2.0 ** (scales.astype(np.float64) - 127)
    t = w.astype(np.float64) / np.repeat(X, 32, axis=1)
    for (r, c), tv in np.ndenumerate(t):
        a = abs(tv)
        dist = np.abs(tab - a)
        best = np.flatnonzero(dist == dist.min())
        code = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        if a > 448.0:
            code = 0x7E
        if np.signbit(tv):
            code |= 0x80
        assert codes[r, c] == code, (r, c, tv, codes[r, c], code)


def pin_mxfp8_golden_block(o):
    """A block worked by hand from the MX conversion rule
    (tests/golden/mxfp8_block.json)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "mxfp8_block.json")) as f:
        g = json.load(f)
    codes, scales = o.mxfp8_quantize(np.array([g["values"]], np.float32))
    assert int(scales[0, 0]) == g["scale_code"]
    assert codes[0].tolist() == g["codes"]
    d = o.mxfp8_dequantize(codes, scales)[0]
    assert np.array_equal(d, np.array(g["dequantized"], np.float32))
    assert np.array_equal(np.signbit(d), np.signbit(np.array(g["dequantized"])))


ALL_PINS = [pin_logits_vs_library, pin_topk_full_sort, pin_tie_rule, pin_bias_only,
            pin_nonfinite, pin_large_logits, pin_renorm_off, pin_weights_for_ids, pin_permute,
            pin_k1_single_expert, pin_identical_experts, pin_zero_weights,
            pin_identity_weights, pin_dense_bruteforce, pin_shared_expert,
            pin_exact_scaling, pin_token_permutation, pin_ffn_closed_form,
            pin_mxfp8_decode_table, pin_mxfp8_rounding_vs_library, pin_mxfp8_saturation,
            pin_mxfp8_scale_rule, pin_mxfp8_nearest_bruteforce, pin_mxfp8_golden_block]


def run_all(o) -> dict:
    """name -> None (passed) or the failure text."""
    out = {}
    for pin in ALL_PINS:
        try:
            pin(o)
            out[pin.__name__] = None
        except Exception as ex:  # noqa: BLE001 - any failure counts
            out[pin.__name__] = f"{type(ex).__name__}: {ex}"
    return out
