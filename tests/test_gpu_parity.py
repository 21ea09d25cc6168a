"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Sizes span several tiles and ragged tails; full-size
workloads compare every token's routing and a sample of tokens' outputs."""
import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import moe, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def layer_on_gpu(cfg, seed=0):
    lay = synth.make_layer(cfg, seed=seed, device=gh.DEV)
    return lay.rounded_to_bf16() if cfg.fp32_values else lay


def custom(name, **kw):
    return synth.custom_config(name, **kw)


def log(name, rep):
    ma, rel = rep["err"]
    print(f"[parity] {name}: near_ties={rep['near_ties']} max_abs={ma:.3e} relL2={rel:.3e} "
          f"w_rel={rep.get('w_rel', 0.0):.2e}", flush=True)


# ------------------------------------------------------------ end to end
SMALL = {
    # tiny workload (fp32 values rounded to bf16 for the GPU; oracle gets the same)
    "tiny": synth.CONFIGS["tiny"],
    # light-row experts only (~2.5 rows each), several N blocks
    "light": custom("light", T=40, H=256, E=64, k=4, I=192),
    # heavy tiles with ragged tails (75 rows per expert, BM=128), K tail in down
    "heavy_ragged": custom("heavy_ragged", T=300, H=320, E=16, k=4, I=96),
    # mixed light / heavy experts, non-power-of-2 k
    "mixed": custom("mixed", T=203, H=256, E=48, k=10, I=128, zipf_s=1.2, zipf_alpha=0.6),
    # max sizes of the ABI: E=1024, k=32
    "max_e_k": custom("max_e_k", T=33, H=128, E=1024, k=32, I=64),
    # k == E
    "k_eq_e": custom("k_eq_e", T=17, H=64, E=8, k=8, I=32),
    # single token
    "one_token": custom("one_token", T=1, H=512, E=128, k=10, I=256),
    # shared expert
    "shared": custom("shared", T=150, H=256, E=32, k=8, I=128, I_shared=160),
    # raw (not renormalised) routing weights
    "no_renorm": custom("no_renorm", T=70, H=192, E=24, k=6, I=64, renorm=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(oracle_lib, name):
    print(f"[case] forward {name}", flush=True)
    rep = gh.check_layer(oracle_lib, layer_on_gpu(SMALL[name]))
    log(name, rep)


# y storage as (y_bf16, y_fp16)
YFMT = {"fp32": (False, False), "bf16": (True, False), "fp16": (False, True)}


@pytest.mark.parametrize("name", ["light", "heavy_ragged", "mixed", "shared", "max_e_k"])
@pytest.mark.parametrize("yf", ["bf16", "fp16"])
def test_forward_small_16bit_y(oracle_lib, name, yf):
    """Routed expert outputs stored as bf16 or fp16 (the shared expert stays
    fp32)."""
    print(f"[case] forward {yf} y {name}", flush=True)
    yb, yh = YFMT[yf]
    rep = gh.check_layer(oracle_lib, layer_on_gpu(SMALL[name]), y_bf16=yb, y_fp16=yh)
    log(f"{name}/{yf}y", rep)


@pytest.mark.parametrize("name", ["tiny", "light", "mixed"])
def test_forward_heavy_only(oracle_lib, name):
    """Every expert through the heavy tiles (light loop off)."""
    print(f"[case] forward heavy-only {name}", flush=True)
    rep = gh.check_layer(oracle_lib, layer_on_gpu(SMALL[name]), light_max_rows=0)
    log(name + "/heavy", rep)


# ------------------------------------------------------------ tile heights
# ~225 rows per expert: 1 tile of 256, 2 ragged tiles of 192 or 128; I % 64 ==
# 32 gives the down GEMM a half-full last K stage, and the shared expert's
# [hi | lo] K run straddles I inside one 64-wide stage.
TILES = custom("tiles", T=600, H=320, E=8, k=3, I=96, I_shared=96)


@pytest.mark.parametrize("y_bf16", [False, True])
def test_tile_heights_bitwise(oracle_lib, y_bf16):
    """Every heavy tile height gives the same output bits (each element's
    MFMA chain over K is the same), and matches the oracle."""
    print(f"[case] tile heights y_bf16={y_bf16}", flush=True)
    lay = layer_on_gpu(TILES)
    outs = {}
    for tm in (0, 256, 224, 192, 160, 128):
        g = gh.gpu_forward(lay, light_max_rows=0, heavy_tile_rows=tm, y_bf16=y_bf16)
        outs[tm] = g["out"].view(np.int32)
    for tm in (256, 224, 192, 160, 128):
        assert np.array_equal(outs[tm], outs[0]), f"tile height {tm} differs"
    rep = gh.check_layer(oracle_lib, lay, light_max_rows=0, heavy_tile_rows=192, y_bf16=y_bf16)
    log(f"tiles/192/bf16y={y_bf16}", rep)


@pytest.mark.parametrize("T,E,k,zipf,lm", [
    (300, 512, 10, 0.0, 64), (400, 512, 10, 3.0, 8),    # one-block permute decides
    (500, 1024, 10, 0.0, 64), (700, 1024, 10, 3.0, 8),  # plan kernel decides
    (1000, 512, 10, 0.0, 8), (300, 64, 10, 0.0, 8)])    # T*k > 8E: fixed on the host
def test_default_light_rule_bitwise(oracle_lib, T, E, k, zipf, lm):
    """The default's per-call light/heavy choice (decided on the device, in
    the one-block permute for T*k <= 4096 and in the plan kernel above, or
    on the host when T*k > 8E): experts with up to 64 rows take the light
    loop when the rows average at most 8 per touched expert, else those with
    up to 8 rows.  It gives the bits of both fixed choices and matches the
    oracle."""
    print(f"[case] default light rule T={T} E={E} k={k} zipf={zipf}", flush=True)
    kw = dict(zipf_s=1.2, zipf_alpha=zipf) if zipf else {}
    cfg = custom(f"rule{T}_{E}", T=T, H=256, E=E, k=k, I=64, **kw)
    lay = layer_on_gpu(cfg)
    outs = {lm: gh.gpu_forward(lay, light_max_rows=lm) for lm in (-1, 0, 64)}
    s = moe.make_shape(T, 256, E, k, 64)
    c = outs[-1]["counts"]
    assert np.array_equal(moe.light_experts(c, s), (c >= 1) & (c <= lm))
    mean = c.sum() / max(1, int((c > 0).sum()))
    assert (mean <= moe.LIGHT_MEAN_ROWS) == (lm == moe.LIGHT_MAX_ROWS)
    for lm in (0, 64):
        assert np.array_equal(outs[-1]["out"].view(np.int32), outs[lm]["out"].view(np.int32))
    rep = gh.check_layer(oracle_lib, lay)
    log(f"rule{T}_{E}", rep)


@pytest.mark.parametrize("tm", [128, 160, 192, 224, 256])
def test_forward_heavy_ragged_heights(oracle_lib, tm):
    print(f"[case] heavy_ragged tm={tm}", flush=True)
    rep = gh.check_layer(oracle_lib, layer_on_gpu(SMALL["heavy_ragged"]), heavy_tile_rows=tm)
    log(f"heavy_ragged/{tm}", rep)


# ------------------------------------------------------------ full size
# The benchmark's configuration (weights handed over only as the packed
# copy; y in bf16 without a shared expert, fp16 with one) is compared over
# 512 sampled tokens of each full-size layer (all 64 at decode); fp32 y and
# the plain weight layout over 64.
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,sample,yf,packed", [
    ("decode", None, "bf16", True), ("prefill", 512, "bf16", True), ("skew", 512, "bf16", True),
    ("ling", 512, "fp16", True),
    ("decode", None, "fp32", False), ("prefill", 64, "fp32", False), ("skew", 64, "fp32", False),
    ("ling", 64, "fp32", False)])
def test_forward_full_size(oracle_lib, name, sample, yf, packed):
    print(f"[case] full-size {name} y={yf} packed={packed} sample={sample}", flush=True)
    y_bf16, y_fp16 = YFMT[yf]
    cfg = synth.CONFIGS[name]
    lay = layer_on_gpu(cfg)
    tokens = None
    if sample:
        tokens = np.sort(np.random.default_rng(1).choice(cfg.T, sample, replace=False))
    rep = gh.check_layer(oracle_lib, lay, tokens=tokens, y_bf16=y_bf16, y_fp16=y_fp16,
                         packed=packed)
    log(f"{name}/y={yf}/packed={packed}/tokens={sample or cfg.T}", rep)
    counts = rep["gpu"]["counts"]
    assert counts.sum() == cfg.T * cfg.k
    if name == "prefill":
        assert counts.sum() == 81920  # the pages' [81920, 4096] permuted rows
    del lay
    torch.cuda.empty_cache()


# ------------------------------------------------------------ stages
@pytest.mark.parametrize("lm", [-1, 64, 0])
def test_repeated_ids_small_batch(oracle_lib, lm):
    """moe_permute accepts ids repeated within a token, so an expert can get
    more rows than there are tokens: with T <= 64 (every expert light by
    default) the grouped FFN must still run the over-full expert through the
    heavy tiles.  Every expert's y rows against the oracle's expert FFN, and
    the same bits for every light threshold."""
    cfg = custom("rep", T=40, H=256, E=8, k=4, I=128)
    lay = layer_on_gpu(cfg)
    rng = np.random.default_rng(11)
    ids_np = np.empty((cfg.T, cfg.k), np.int32)
    for t in range(cfg.T):
        ids_np[t] = [0, 0, 0, rng.integers(1, cfg.E)]  # expert 0: 120 rows
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, light_max_rows=lm)
    ws = moe.alloc_workspace(s)
    A = cfg.T * cfg.k
    t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
    counts, offsets, srt, inv = t(cfg.E), t(cfg.E + 1), t(A), t(A)
    moe.permute(s, torch.as_tensor(ids_np, device=gh.DEV), counts, offsets, srt, inv, ws)
    y = torch.full((A, cfg.H), float("nan"), dtype=torch.float32, device=gh.DEV)
    moe.grouped_ffn(s, lay.x, srt, offsets, lay.w_gu, lay.w_dn, None, y, ws)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    assert off[1] - off[0] == 3 * cfg.T
    srt_np = srt.cpu().numpy()
    y_np = y.cpu().numpy()
    assert np.all(np.isfinite(y_np)), "rows left unwritten"
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            ref = oracle_lib.expert_ffn(lay.x[torch.as_tensor(srt_np[rows], device=gh.DEV)],
                                        lay.w_gu[e], lay.w_dn[e])
            gh.assert_close(y_np[rows], ref, f"expert {e}")


def _ids_tensor(rng, T, E, k):
    return torch.as_tensor(np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32),
                           device=gh.DEV)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (4, 16, 4), (64, 512, 10), (300, 128, 13),
                                   (409, 64, 10), (500, 64, 10), (1000, 512, 10), (4096, 8, 2),
                                   (333, 1024, 32)])
def test_permute_stage(oracle_lib, T, E, k):
    """Bit-exact against the oracle's permutation: one-block path (T*k <=
    4096: 1, 16, 640, 3900, 4090 assignments) and several chunks, ragged."""
    print(f"[case] permute T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(T + E)
    ids = _ids_tensor(rng, T, E, k)
    s = moe.make_shape(T, 64, E, k, 32)
    ws = moe.alloc_workspace(s)
    counts = torch.empty(E, dtype=torch.int32, device=gh.DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=gh.DEV)
    srt = torch.empty(T * k, dtype=torch.int32, device=gh.DEV)
    inv = torch.empty(T * k, dtype=torch.int32, device=gh.DEV)
    moe.permute(s, ids, counts, offsets, srt, inv, ws)
    torch.cuda.synchronize()
    ref = oracle_lib.permute(ids.cpu().numpy(), E)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(srt.cpu().numpy(), ref["sorted_token_ids"])
    assert np.array_equal(inv.cpu().numpy(), ref["inv_pos"])


def test_permute_skips_invalid_ids():
    """Ids outside [0, E) are not counted and get inv_pos = -1; the rest keep
    their stable expert-major order (numpy stable argsort)."""
    rng = np.random.default_rng(5)
    T, E, k = 700, 40, 6
    ids_np = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.random(ids_np.shape) < 0.05
    ids_np[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    s = moe.make_shape(T, 64, E, k, 32)
    ws = moe.alloc_workspace(s)
    t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
    counts, offsets, srt, inv = t(E), t(E + 1), t(T * k), t(T * k)
    moe.permute(s, torch.as_tensor(ids_np, device=gh.DEV), counts, offsets, srt, inv, ws)
    torch.cuda.synchronize()
    flat = ids_np.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(flat[valid], minlength=E))
    inv_np = inv.cpu().numpy()
    assert np.all(inv_np[~valid] == -1)
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    n = valid.sum()
    assert np.array_equal(srt.cpu().numpy()[:n], order // k)
    assert np.array_equal(inv_np[order], np.arange(n))


# many tokens (one wave per token in the select), E not a multiple of 64
ROUTER_WIDE = custom("router_wide", T=1037, H=256, E=200, k=7, I=32)
# few tokens and 16 split-K partials (the grouped select), E <= 512 and E > 512
ROUTER_SPLIT = custom("router_split", T=10, H=1024, E=300, k=5, I=32)
ROUTER_SPLIT_WIDE_E = custom("router_split_wide_e", T=20, H=1024, E=1000, k=12, I=32)


@pytest.mark.parametrize("cfg", [SMALL["light"], SMALL["mixed"], SMALL["max_e_k"], ROUTER_WIDE,
                                 ROUTER_SPLIT, ROUTER_SPLIT_WIDE_E], ids=lambda c: c.name)
def test_router_stage(oracle_lib, cfg):
    print(f"[case] router {cfg.name}", flush=True)
    lay = layer_on_gpu(cfg)
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, renorm=cfg.renorm)
    ws = moe.alloc_workspace(s)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=gh.DEV)
    probs = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=gh.DEV)
    moe.router(s, lay.x, lay.wg, lay.bias, ids, w, probs, ws)
    torch.cuda.synchronize()
    ref = oracle_lib.route(oracle_lib.logits(lay.x, lay.wg, lay.bias), cfg.k, cfg.renorm)
    gh.check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref)
    rp = ref["probs"]
    assert np.all(np.abs(probs.cpu().numpy() - rp) <= gh.W_ATOL + gh.W_RTOL * rp)


def test_router_nonfinite(oracle_lib):
    """NaN and +/-inf in the bias: the same ids as the oracle, all distinct
    and in range (NaN counts as -inf; +inf entries share the mass)."""
    cfg = custom("nonfinite", T=8, H=64, E=96, k=6, I=32)
    lay = layer_on_gpu(cfg)
    b = torch.zeros(cfg.E)
    b[3] = float("nan")
    b[17] = float("inf")
    b[40] = float("inf")
    b[50:60] = float("-inf")
    lay.bias = b.to(gh.DEV)
    x0 = lay.x.clone()
    x0[0] = float("nan")  # a token whose every logit is NaN
    lay.x = x0
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
    ws = moe.alloc_workspace(s)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=gh.DEV)
    moe.router(s, lay.x, lay.wg, lay.bias, ids, w, None, ws)
    torch.cuda.synchronize()
    ref = oracle_lib.route(oracle_lib.logits(lay.x, lay.wg, lay.bias), cfg.k, 1)
    g = ids.cpu().numpy()
    assert np.array_equal(g[:, :2], ref["ids"][:, :2])
    assert np.array_equal(g[0], np.arange(cfg.k))
    for row in g:
        assert len(set(row.tolist())) == cfg.k and row.min() >= 0 and row.max() < cfg.E
    assert np.array_equal(g, ref["ids"])


@pytest.mark.parametrize("light_max", [16, 64])
@pytest.mark.parametrize("yf", ["fp32", "bf16", "fp16"])
def test_light_heavy_bitwise(light_max, yf):
    """The same expert rows through the light loop (both its 16-row and its
    wide 17..64-row branch) and through the heavy tiles give bitwise
    identical h and y (fp32, bf16 or fp16)."""
    y_bf16, y_fp16 = YFMT[yf]
    cfg = custom("lh", T=160, H=512, E=64, k=8, I=256)
    lay = layer_on_gpu(cfg)
    outs = []
    for lm in (light_max, 0):
        s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, light_max_rows=lm, y_bf16=y_bf16,
                           y_fp16=y_fp16)
        ws = moe.alloc_workspace(s)
        A = cfg.T * cfg.k
        ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=gh.DEV)
        w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=gh.DEV)
        moe.router(s, lay.x, lay.wg, None, ids, w, None, ws)
        t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
        counts, offsets, srt, inv = t(cfg.E), t(cfg.E + 1), t(A), t(A)
        moe.permute(s, ids, counts, offsets, srt, inv, ws)
        h = torch.empty((A, cfg.I), dtype=torch.bfloat16, device=gh.DEV)
        y = torch.empty((A, cfg.H), dtype=moe.y_dtype(s), device=gh.DEV)
        moe.grouped_ffn(s, lay.x, srt, offsets, lay.w_gu, lay.w_dn, h, y, ws)
        torch.cuda.synchronize()
        yi = y.view(torch.int16) if (y_bf16 or y_fp16) else y.view(torch.int32)
        outs.append((counts.cpu().numpy(), h.view(torch.int16).cpu().numpy(), yi.cpu().numpy()))
    (c0, h0, y0), (c1, h1, y1) = outs
    assert np.array_equal(c0, c1)
    assert ((c0 >= 1) & (c0 <= 16)).sum() > 0
    if light_max == 64:
        assert ((c0 > 16) & (c0 <= 64)).sum() > 0  # the wide branch ran
    assert np.array_equal(h0, h1), "h differs between light and heavy loops"
    assert np.array_equal(y0, y1), "y differs between light and heavy loops"


@pytest.mark.parametrize("yf", ["fp32", "bf16", "fp16"])
def test_ffn_stage_rows(oracle_lib, yf):
    """Grouped FFN rows (fp32, bf16 or fp16 y from bf16 h) against the
    oracle's per-row expert FFN."""
    cfg = SMALL["mixed"]
    lay = layer_on_gpu(cfg)
    y_bf16, y_fp16 = YFMT[yf]
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, y_bf16=y_bf16, y_fp16=y_fp16)
    ws = moe.alloc_workspace(s)
    A = cfg.T * cfg.k
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=gh.DEV)
    moe.router(s, lay.x, lay.wg, lay.bias, ids, w, None, ws)
    t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
    counts, offsets, srt, inv = t(cfg.E), t(cfg.E + 1), t(A), t(A)
    moe.permute(s, ids, counts, offsets, srt, inv, ws)
    y = torch.empty((A, cfg.H), dtype=moe.y_dtype(s), device=gh.DEV)
    moe.grouped_ffn(s, lay.x, srt, offsets, lay.w_gu, lay.w_dn, None, y, ws)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    srt_np = srt.cpu().numpy()
    y_np = y.float().cpu().numpy()
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        ref = oracle_lib.expert_ffn(lay.x[torch.as_tensor(srt_np[rows], device=gh.DEV)],
                                    lay.w_gu[e], lay.w_dn[e])
        gh.assert_close(y_np[rows], ref, f"expert {e}")


@pytest.mark.parametrize("lm", [64, 0])
def test_swiglu_extreme_gates(oracle_lib, lm):
    """Gate values out to about +-150: W_gate rows scaled by 128 and W_down by
    1/8 (both exact in bf16; outputs stay of order 1, so the usual bar
    applies).  Below g = -88.7 e^-g overflows fp32 and silu(g) is -0 (the
    oracle's quotient g / inf, the kernels' g * rcp(inf)); just above it
    1 / (1 + e^-g) falls below the normal range.  The light loop (lm = 64:
    every expert has 17..64 rows, its wide branch) and the heavy tiles
    (lm = 0) against the oracle's per-row expert FFN, fp32 y."""
    print(f"[case] swiglu extreme gates lm={lm}", flush=True)
    cfg = custom("gates", T=160, H=256, E=8, k=2, I=64)
    lay = layer_on_gpu(cfg)
    lay.w_gu[:, :cfg.I] *= 128
    lay.w_dn *= 0.125
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, light_max_rows=lm)
    ws = moe.alloc_workspace(s)
    A = cfg.T * cfg.k
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=gh.DEV)
    moe.router(s, lay.x, lay.wg, lay.bias, ids, w, None, ws)
    t = lambda n: torch.empty(n, dtype=torch.int32, device=gh.DEV)
    counts, offsets, srt, inv = t(cfg.E), t(cfg.E + 1), t(A), t(A)
    moe.permute(s, ids, counts, offsets, srt, inv, ws)
    y = torch.empty((A, cfg.H), dtype=moe.y_dtype(s), device=gh.DEV)
    moe.grouped_ffn(s, lay.x, srt, offsets, lay.w_gu, lay.w_dn, None, y, ws)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    srt_np = srt.cpu().numpy()
    y_np = y.float().cpu().numpy()
    assert ((np.diff(off) > 16) & (np.diff(off) <= 64)).all()
    overflow = 0
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        xr = lay.x[torch.as_tensor(srt_np[rows], device=gh.DEV)]
        # gate values of these rows (to count the overflow region only)
        g = xr.double() @ lay.w_gu[e, :cfg.I].double().T
        overflow += int((g < -88.73).sum())
        ref = oracle_lib.expert_ffn(xr, lay.w_gu[e], lay.w_dn[e])
        gh.assert_close(y_np[rows], ref, f"expert {e}")
    assert overflow > 50, overflow


@pytest.mark.parametrize("T", [77, 600])
@pytest.mark.parametrize("yf", ["fp32", "bf16", "fp16"])
def test_combine_stage(T, yf):
    """Combine against a float64 numpy weighted sum of the same rows (fp32,
    or bf16 / fp16 widened exactly), below and above the 512-token grid
    switch."""
    rng = np.random.default_rng(9)
    H, k, E = 320, 5, 20
    A = T * k
    y_bf16, y_fp16 = YFMT[yf]
    y = torch.randn((A, H), device=gh.DEV)
    if y_bf16:
        y = y.to(torch.bfloat16)
    if y_fp16:
        y = y.to(torch.float16)
    perm = rng.permutation(A).astype(np.int32)
    perm[3] = -1  # skipped row
    w = torch.rand((T, k), device=gh.DEV)
    s = moe.make_shape(T, H, E, k, 32, y_bf16=y_bf16, y_fp16=y_fp16)
    for acc in (0, 1):
        out = torch.randn((T, H), device=gh.DEV)
        prev = out.cpu().numpy().astype(np.float64)
        moe.combine(s, y, torch.as_tensor(perm, device=gh.DEV), w, acc, out)
        torch.cuda.synchronize()
        yv = y.float().cpu().numpy().astype(np.float64)
        wv = w.cpu().numpy().astype(np.float64)
        ref = np.zeros((T, H))
        for t in range(T):
            for j in range(k):
                p = perm[t * k + j]
                if p >= 0:
                    ref[t] += wv[t, j] * yv[p]
        if acc:
            ref += prev
        assert np.abs(out.cpu().numpy() - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


def test_profile_hook_per_launch():
    """With a shared expert the heavy GEMM kernels run twice per forward;
    the hook brackets either launch on its own, or every launch."""
    lay = layer_on_gpu(SMALL["shared"])
    m = moe.MoELayer(lay, light_max_rows=0)
    m()
    torch.cuda.synchronize()
    durs = []
    for launch in (-1, 0, 1, 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.profile_kernel("gateup_heavy", a, b, launch=launch)
        m()
        n = moe.profile_launches()
        moe.profile_kernel(None)
        torch.cuda.synchronize()
        assert n == 2
        if launch != 2:  # a launch index past the last one records nothing
            durs.append(a.elapsed_time(b))
    assert all(d > 0 for d in durs)


def test_shared_stage(oracle_lib):
    cfg = SMALL["shared"]
    lay = layer_on_gpu(cfg)
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared)
    ws = moe.alloc_workspace(s)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=gh.DEV)
    moe.shared_ffn(s, lay.x, lay.ws_gu, lay.ws_dn, out, ws)
    torch.cuda.synchronize()
    ref = oracle_lib.expert_ffn(lay.x, lay.ws_gu, lay.ws_dn)
    gh.assert_close(out.cpu().numpy(), ref, "shared expert")


OVERLAP = {
    "shared": custom("ovl", T=700, H=512, E=16, k=4, I=256, I_shared=512),
    # Zipf routing: the cold experts take the light loop, the rest heavy tiles
    "light": custom("ovl_light", T=600, H=384, E=48, k=6, I=128, zipf_s=1.2, zipf_alpha=1.5),
    "both": custom("ovl_both", T=600, H=384, E=48, k=6, I=128, I_shared=96, zipf_s=1.2,
                   zipf_alpha=1.5),
}


@pytest.mark.parametrize("name", list(OVERLAP))
def test_shared_overlap_back_to_back(name):
    """moe_forward runs the shared expert on a side stream that forks from
    the caller's stream before the router and joins before the combine.
    Four calls enqueued back to back on a non-default stream, each writing
    its own output (and the last two sharing one), with no host wait in
    between, must each equal the serial composition of the stages bit for
    bit: shared expert into `out`, routed FFN, then the combine adding to it.
    The layers: a shared expert with heavy experts only, and Zipf-routed
    layers whose cold experts take the light loop, with and without a shared
    expert."""
    cfg = OVERLAP[name]
    print(f"[case] overlap {name}", flush=True)
    lay = layer_on_gpu(cfg)
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared)
    ws = moe.alloc_workspace(s)
    T, H, k = cfg.T, cfg.H, cfg.k
    # serial reference from the stage calls, on the default stream
    ids = torch.empty((T, k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=gh.DEV)
    moe.router(s, lay.x, lay.wg, lay.bias, ids, w, None, ws)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=gh.DEV)
    offsets = torch.empty((cfg.E + 1,), dtype=torch.int32, device=gh.DEV)
    sorted_ids = torch.empty((T * k,), dtype=torch.int32, device=gh.DEV)
    inv = torch.empty((T * k,), dtype=torch.int32, device=gh.DEV)
    moe.permute(s, ids, counts, offsets, sorted_ids, inv, ws)
    if name != "shared":  # the layer really has experts of both kinds
        c = counts.cpu().numpy()
        light = moe.light_experts(c, s)
        assert light.any() and (~light & (c > 0)).any(), c
    y = torch.empty((T * k, H), dtype=torch.float32, device=gh.DEV)
    moe.grouped_ffn(s, lay.x, sorted_ids, offsets, lay.w_gu, lay.w_dn, None, y, ws)
    ref = torch.empty((T, H), dtype=torch.float32, device=gh.DEV)
    if cfg.I_shared:
        moe.shared_ffn(s, lay.x, lay.ws_gu, lay.ws_dn, ref, ws)
    moe.combine(s, y, inv, w, bool(cfg.I_shared), ref)
    torch.cuda.synchronize()
    ref = ref.view(torch.int32).cpu()
    st = torch.cuda.Stream()
    outs = [torch.full((T, H), float("nan"), device=gh.DEV) for _ in range(3)]
    wss = [moe.alloc_workspace(s) for _ in range(2)]
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for i, o in enumerate(outs + [outs[2]]):
            moe.forward(s, lay.x, lay.wg, lay.bias, lay.w_gu, lay.w_dn, lay.ws_gu, lay.ws_dn,
                        o, wss[i % 2], stream=st)
    st.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o.view(torch.int32).cpu(), ref), f"call {i} differs from the stages"


def test_shared_overlap_two_host_threads():
    """Two host threads call moe_forward at once (ctypes releases the GIL),
    each on its own stream with its own workspace and inputs, three calls
    each with no wait in between: the library's side stream and its fork and
    join events are shared per device, so the fork-to-join sections must
    not interleave.  Every output equals the same call made alone."""
    import threading

    cfg = OVERLAP["both"]
    lays = [layer_on_gpu(cfg, seed=s) for s in (11, 12)]
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared)

    def call(lay, ws, out, stream=None):
        moe.forward(s, lay.x, lay.wg, lay.bias, lay.w_gu, lay.w_dn, lay.ws_gu, lay.ws_dn, out, ws,
                    stream=stream)

    refs = []
    for lay in lays:
        ws = moe.alloc_workspace(s)
        out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=gh.DEV)
        call(lay, ws, out)
        torch.cuda.synchronize()
        refs.append(out.view(torch.int32).cpu())
    streams = [torch.cuda.Stream() for _ in lays]
    outs = [[torch.full((cfg.T, cfg.H), float("nan"), device=gh.DEV) for _ in range(3)]
            for _ in lays]
    wss = [moe.alloc_workspace(s) for _ in lays]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for o in outs[i]:
                    call(lays[i], wss[i], o, stream=streams[i])
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for st in streams:
        st.synchronize()
    for i in range(2):
        for j, o in enumerate(outs[i]):
            assert torch.equal(o.view(torch.int32).cpu(), refs[i]), f"thread {i} call {j} differs"


# ------------------------------------------------------------ properties
def test_determinism_and_equivariance():
    cfg = SMALL["mixed"]
    lay = layer_on_gpu(cfg)
    a = gh.gpu_forward(lay)
    b = gh.gpu_forward(lay)
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{key} not deterministic"
    perm = torch.as_tensor(np.random.default_rng(3).permutation(cfg.T), device=gh.DEV)
    lay_p = synth.Layer(cfg, lay.x[perm].contiguous(), lay.wg, lay.bias, lay.w_gu, lay.w_dn)
    c = gh.gpu_forward(lay_p)
    pn = perm.cpu().numpy()
    assert np.array_equal(a["out"][pn], c["out"]), "token permutation changed output bits"
    assert np.array_equal(a["ids"][pn], c["ids"])


def test_exact_scaling_and_zero():
    cfg = SMALL["mixed"]
    lay = layer_on_gpu(cfg)
    a = gh.gpu_forward(lay)
    lay2 = synth.Layer(cfg, lay.x, lay.wg, lay.bias, lay.w_gu, (lay.w_dn * 2).contiguous())
    b = gh.gpu_forward(lay2)
    assert np.array_equal(2 * a["out"], b["out"])
    lay0 = synth.Layer(cfg, lay.x, lay.wg, lay.bias, lay.w_gu, torch.zeros_like(lay.w_dn))
    z = gh.gpu_forward(lay0)
    assert np.all(z["out"] == 0)


def test_empty_batch():
    cfg = custom("empty", T=0, H=64, E=8, k=2, I=32)
    s = moe.make_shape(0, 64, 8, 2, 32)
    ws = moe.alloc_workspace(s)
    lay = layer_on_gpu(custom("e1", T=1, H=64, E=8, k=2, I=32))
    counts = torch.full((8,), 7, dtype=torch.int32, device=gh.DEV)
    out = torch.empty((0, 64), dtype=torch.float32, device=gh.DEV)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=gh.DEV)
    moe.forward(s, x, lay.wg, None, lay.w_gu, lay.w_dn, None, None, out, ws, counts_out=counts)
    torch.cuda.synchronize()
    assert cfg.T == 0 and np.all(counts.cpu().numpy() == 0)


# ------------------------------------------------------------ packed weights
@pytest.mark.parametrize("cfg,tm,lm", [(TILES, 0, 0), (TILES, 128, 0), (TILES, 192, 0),
                                       (TILES, 256, 0), (TILES, 0, -1), (SMALL["mixed"], 0, 0),
                                       (SMALL["mixed"], 0, -1), (SMALL["heavy_ragged"], 0, 0),
                                       (SMALL["light"], 0, -1), (SMALL["max_e_k"], 0, -1)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_packed_weights_bitwise(cfg, tm, lm):
    """Both loops reading the packed records give the same output bits as
    reading the plain layout (same data, same MFMA chains), at every heavy
    tile height and with the light loop on and off."""
    print(f"[case] packed {cfg.name} tm={tm} light_max={lm}", flush=True)
    lay = layer_on_gpu(cfg)
    outs = []
    for packed in (False, True):
        m = moe.MoELayer(lay, light_max_rows=lm, heavy_tile_rows=tm, packed=packed)
        out, ids, w, counts = m()
        torch.cuda.synchronize()
        outs.append(out.view(torch.int32).cpu().numpy())
    assert np.array_equal(outs[0], outs[1]), "packed weights change the output"


def test_packed_weights_layout():
    """Spot-check the packed records against their definition: record
    (e, nb, c) is 16 row blocks j of two 1 KB chunks h; lane L of chunk
    (j, h) holds K values 64c + 32h + 8(L//16) .. +7 of tile row
    rr = 16j + L%16, which is the gate|up row of h column
    nb*128 + 16*(rr//32) + rr%16 (gate where rr%32 < 16, else up) or W_down
    row nb*256 + rr, zero past the weights; W_gate|up's records first,
    nothing else in the buffer."""
    cfg = custom("pk", T=8, H=192, E=2, k=1, I=160)
    lay = layer_on_gpu(cfg)
    s = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
    pk = moe.pack_weights(s, lay.w_gu, lay.w_dn)
    torch.cuda.synchronize()
    words = pk.view(torch.int16).cpu().numpy()
    wgu = lay.w_gu.view(torch.int16).cpu().numpy()
    wdn = lay.w_dn.view(torch.int16).cpu().numpy()
    H, I, E = cfg.H, cfg.I, cfg.E
    rng = np.random.default_rng(3)
    nbg, nbd = -(-2 * I // 256), -(-H // 256)
    ncg, ncd = -(-H // 64), -(-I // 64)
    rec_gu = E * nbg * ncg * 256 * 64
    assert words.size == rec_gu + E * nbd * ncd * 256 * 64
    for _ in range(3000):
        gate_up = bool(rng.integers(2))
        nbk, nc = (nbg, ncg) if gate_up else (nbd, ncd)
        e, nb, c, j, h, L = (int(rng.integers(n)) for n in (E, nbk, nc, 16, 2, 64))
        rr = 16 * j + L % 16
        k0 = 64 * c + 32 * h + 8 * (L // 16)
        if gate_up:
            hc = nb * 128 + (rr // 32) * 16 + rr % 16
            ok, row, src, K = hc < I, (hc if rr % 32 < 16 else I + hc), wgu[e], H
        else:
            row = nb * 256 + rr
            ok, src, K = row < H, wdn[e], I
        want = src[row, k0:k0 + 8] if ok and k0 < K else np.zeros(8, np.int16)
        off = ((0 if gate_up else rec_gu) + ((e * nbk + nb) * nc + c) * 256 * 64
               + (2 * j + h) * 512 + L * 8)
        assert np.array_equal(words[off:off + 8], want), (gate_up, e, nb, c, j, h, L)
