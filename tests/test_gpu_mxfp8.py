"""GPU checks of the MXFP8 expert-weight variant, through the C ABI.

- The quantiser's codes and scales equal the oracle's bit for bit (integer
  outputs): random bf16 weights, every finite bf16 bit pattern class
  (subnormals, huge values, signed zeros), ties and saturating blocks.
- The packed layout matches its definition (spot checks).
- The layer on MXFP8 weights -- light loop and heavy tiles -- gives the
  bits of the bf16 layer run on the dequantised weights (same MFMA chains on
  the same operands).
- Against the oracle run on its own quantisation of the same weights: the
  bar of the bf16 path (max_abs 2e-2, relL2 5e-3).
"""
import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import moe, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def custom(name, **kw):
    return synth.custom_config(name, **kw)


def layer_on_gpu(cfg, seed=0):
    lay = synth.make_layer(cfg, seed=seed, device=gh.DEV)
    return lay.rounded_to_bf16() if cfg.fp32_values else lay


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def quantize_gpu(w_bf16_bits_np):
    w = torch.as_tensor(w_bf16_bits_np.astype(np.int16), device=gh.DEV).view(torch.bfloat16)
    codes, scales = moe.quantize_mxfp8(w)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def edge_blocks(rng):
    """bf16 bit patterns [rows, 64]: random finite patterns over the whole
    exponent range, subnormal-only blocks, zero and -0 blocks, blocks whose
    maximum saturates, exact ties after scaling."""
    rows = []
    # random finite bf16 patterns (exponent field 0..254), any sign
    e = rng.integers(0, 255, size=(64, 64))
    m = rng.integers(0, 128, size=(64, 64))
    s = rng.integers(0, 2, size=(64, 64))
    rows.append((s << 15) | (e << 7) | m)
    # narrow dynamic range blocks around a random binade
    base = rng.integers(60, 190, size=(64, 1))
    e2 = np.clip(base + rng.integers(-12, 1, size=(64, 64)), 0, 254)
    rows.append((rng.integers(0, 2, size=(64, 64)) << 15) | (e2 << 7) | rng.integers(0, 128, (64, 64)))
    # subnormal bf16 only
    rows.append((rng.integers(0, 2, size=(8, 64)) << 15) | rng.integers(0, 128, size=(8, 64)))
    # zeros and negative zeros
    rows.append(np.zeros((2, 64), np.int64))
    rows.append(np.full((2, 64), 0x8000))
    # saturating maxima: 1.75..1.99 * 2^k scaled to (448, 512) with ties below
    sat = np.zeros((16, 64), np.int64)
    for r in range(16):
        k = int(rng.integers(100, 150))
        sat[r] = (k << 7) | rng.integers(0, 128, size=64)
        sat[r, :4] = (k << 7) | np.array([0x70, 0x78, 0x7f, 0x71])  # 1.875, 1.9375, 1.99, 1.88
    rows.append(sat)
    # ties: values whose scaled significand sits half-way between E4M3 steps
    tie = np.zeros((16, 64), np.int64)
    for r in range(16):
        k = int(rng.integers(110, 140))
        tie[r] = ((k - rng.integers(0, 12, size=64)) << 7) | (rng.integers(0, 8, size=64) * 16 + 8)
        tie[r, 0] = (k << 7)
    rows.append(tie)
    return np.concatenate(rows).astype(np.uint16)


def test_quantize_matches_oracle(oracle_lib):
    print("[case] mxfp8 quantize vs oracle", flush=True)
    rng = np.random.default_rng(31)
    bits = edge_blocks(rng)
    w32 = (rng.standard_normal((301, 160)) * 0.02).astype(np.float32)
    bits2 = (w32.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern
    for b in (bits, bits2):
        got_c, got_s = quantize_gpu(b)
        want_c, want_s = oracle_lib.mxfp8_quantize(bf16_bits_to_f32(b))
        assert np.array_equal(got_s, want_s), "scales differ"
        bad = np.argwhere(got_c != want_c)
        assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def test_quantize_empty_and_layout():
    w = torch.zeros((0, 64), dtype=torch.bfloat16, device=gh.DEV)
    c, s = moe.quantize_mxfp8(w)
    assert c.shape == (0, 64) and s.shape == (0, 2)
    with pytest.raises(moe.MoeError):
        moe.quantize_mxfp8(torch.zeros((4, 48), dtype=torch.bfloat16, device=gh.DEV))


def test_pack_layout():
    """Lane L of code chunk (e, g, c) holds the codes of K 64c + 8(L//16)..+7
    then 64c + 32 + 8(L//16)..+7 of its row (gate|up: 8g + L%8 or I + 8g +
    L%8; down: 16g + L%16), zero past K; its scales are 32 bytes, row r's
    two K steps at 2r, 2r+1 (127 past K)."""
    print("[case] mxfp8 pack layout", flush=True)
    cfg = custom("pkmx", T=8, H=192, E=3, k=1, I=96)
    lay = layer_on_gpu(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    s = moe.make_shape(cfg.T, H, E, cfg.k, I, w_mxfp8=1)
    cgu, sgu = moe.quantize_mxfp8(lay.w_gu)
    cdn, sdn = moe.quantize_mxfp8(lay.w_dn)
    pk = moe.pack_weights_mxfp8(s, cgu, sgu, cdn, sdn)
    torch.cuda.synchronize()
    pk = pk.cpu().numpy()
    cgu, sgu, cdn, sdn = (t.cpu().numpy() for t in (cgu, sgu, cdn, sdn))
    ncg, ncd = H // 64, (I + 63) // 64
    gg, gd = I // 8, H // 16
    off_cdn = E * gg * ncg * 1024
    off_sgu = off_cdn + E * gd * ncd * 1024
    off_sdn = off_sgu + E * gg * ncg * 32
    off_hgu = off_sdn + E * gd * ncd * 32
    nbg, nbd = -(-2 * I // 256), -(-H // 256)
    REC = 256 * 64 + 512
    off_hdn = off_hgu + E * nbg * ncg * REC
    assert pk.size == off_hdn + E * nbd * ncd * REC
    rng = np.random.default_rng(4)
    # heavy-tile records (e, nb, c): row rr's 16-byte unit q = K 64c + 8q..+7
    # then 64c + 32 + 8q..+7; scales after the 16 KB of codes, row rr's two K
    # steps at 2 * (4 * (16 * (rr // 64) + rr % 16) + (rr // 16) % 4)
    for _ in range(400):
        gate_up = bool(rng.integers(0, 2))
        e = int(rng.integers(0, E))
        nb = int(rng.integers(0, nbg if gate_up else nbd))
        c = int(rng.integers(0, ncg if gate_up else ncd))
        rr, q = int(rng.integers(0, 256)), int(rng.integers(0, 4))
        if gate_up:
            hc = nb * 128 + (rr // 32) * 16 + rr % 16
            valid, row = hc < I, (hc if rr % 32 < 16 else I + hc)
            src, ssrc, K, nc, base = cgu[e], sgu[e], H, ncg, off_hgu
        else:
            row = nb * 256 + rr
            valid = row < H
            src, ssrc, K, nc, base = cdn[e], sdn[e], I, ncd, off_hdn
        want = np.zeros(16, np.uint8)
        if valid:
            for half in range(2):
                for i in range(8):
                    kk = 64 * c + 32 * half + 8 * q + i
                    if kk < K:
                        want[8 * half + i] = src[row, kk]
        rec = base + ((e * (nbg if gate_up else nbd) + nb) * nc + c) * REC
        assert np.array_equal(pk[rec + rr * 64 + 16 * q: rec + rr * 64 + 16 * q + 16], want)
        slot = 4 * (16 * (rr // 64) + rr % 16) + (rr // 16) % 4
        for st in range(2):
            ks = 2 * c + st
            w = ssrc[row, ks] if valid and ks < K // 32 else 127
            assert pk[rec + 256 * 64 + 2 * slot + st] == w, (gate_up, e, nb, c, rr, st)
    for _ in range(400):
        gate_up = bool(rng.integers(0, 2))
        e = int(rng.integers(0, E))
        g = int(rng.integers(0, gg if gate_up else gd))
        c = int(rng.integers(0, ncg if gate_up else ncd))
        L = int(rng.integers(0, 64))
        if gate_up:
            row = 8 * g + L % 8 if L % 16 < 8 else I + 8 * g + L % 8
            src, ssrc, K, nc = cgu[e], sgu[e], H, ncg
            chunk = (e * gg + g) * nc + c
            base, sbase = 0, off_sgu
        else:
            row = 16 * g + L % 16
            src, ssrc, K, nc = cdn[e], sdn[e], I, ncd
            chunk = (e * gd + g) * nc + c
            base, sbase = off_cdn, off_sdn
        want = np.zeros(16, np.uint8)
        for half in range(2):
            for i in range(8):
                kk = 64 * c + 32 * half + 8 * (L // 16) + i
                if kk < K:
                    want[8 * half + i] = src[row, kk]
        got = pk[base + chunk * 1024 + 16 * L: base + chunk * 1024 + 16 * L + 16]
        assert np.array_equal(got, want), (gate_up, e, g, c, L)
        r16 = L % 16
        for st in range(2):
            ks = 2 * c + st
            w = ssrc[row, ks] if ks < K // 32 else 127
            assert pk[sbase + chunk * 32 + 2 * r16 + st] == w


def dequant_layer(o, lay):
    """A copy of `lay` whose routed weights are the oracle's MXFP8
    quantisation of them, dequantised (exact in bf16)."""
    def dq(w):
        c, s = o.mxfp8_quantize(w.float().cpu().numpy())
        return torch.as_tensor(o.mxfp8_dequantize(c, s), device=w.device).to(torch.bfloat16)
    import dataclasses
    return dataclasses.replace(lay, w_gu=dq(lay.w_gu), w_dn=dq(lay.w_dn))


MX_CASES = {
    "light": custom("light", T=40, H=256, E=64, k=4, I=192),
    # 75 rows per expert: heavy tiles, ragged
    "heavy_ragged": custom("heavy_ragged", T=300, H=320, E=16, k=4, I=96),
    "mixed": custom("mixed", T=203, H=256, E=48, k=10, I=128, zipf_s=1.2, zipf_alpha=0.6),
    "one_token": custom("one_token", T=1, H=512, E=128, k=10, I=256),
    "shared": custom("shared", T=150, H=256, E=32, k=8, I=128, I_shared=160),
    # I % 64 == 32: the last K chunk of W_down is half padding
    "i_tail": custom("i_tail", T=90, H=192, E=12, k=3, I=160),
    "max_e_k": custom("max_e_k", T=33, H=128, E=1024, k=32, I=64),
    # 170 rows on one expert (heavy tiles of 192 or 128 rows)
    "hot": custom("hot", T=170, H=128, E=4, k=1, I=64, zipf_s=3.0, zipf_alpha=1.0),
}


@pytest.mark.parametrize("name", list(MX_CASES))
@pytest.mark.parametrize("y_bf16", [False, True])
def test_layer_bitwise_vs_dequantised_bf16(oracle_lib, name, y_bf16):
    """Default light/heavy rule: light loop, heavy tiles (128/192 rows) or
    both, depending on the shape."""
    print(f"[case] mxfp8 bitwise {name} y_bf16={y_bf16}", flush=True)
    lay = layer_on_gpu(MX_CASES[name])
    ref = dequant_layer(oracle_lib, lay)
    out_mx = moe.MoELayer(lay, y_bf16=y_bf16, weights="mxfp8")()
    out_16 = moe.MoELayer(ref, y_bf16=y_bf16)()
    torch.cuda.synchronize()
    assert torch.equal(out_mx[1], out_16[1])
    assert torch.equal(out_mx[0].view(torch.int32), out_16[0].view(torch.int32)), \
        "MXFP8 layer differs from the bf16 layer on dequantised weights"


@pytest.mark.parametrize("name", ["heavy_ragged", "mixed", "i_tail", "hot", "shared"])
@pytest.mark.parametrize("lm,tm", [(0, 0), (0, 128), (0, 160), (0, 192), (64, 0), (16, 128)])
def test_layer_bitwise_paths(oracle_lib, name, lm, tm):
    """Every MXFP8 path -- heavy tiles of each height, the light loop, and
    splits between the two -- against the bf16 layer on the dequantised
    weights (y bf16)."""
    print(f"[case] mxfp8 paths {name} light_max={lm} tm={tm}", flush=True)
    lay = layer_on_gpu(MX_CASES[name])
    ref = dequant_layer(oracle_lib, lay)
    out_mx = moe.MoELayer(lay, light_max_rows=lm, heavy_tile_rows=tm, y_bf16=True,
                          weights="mxfp8")()
    out_16 = moe.MoELayer(ref, y_bf16=True)()
    torch.cuda.synchronize()
    assert torch.equal(out_mx[0].view(torch.int32), out_16[0].view(torch.int32))


class _LazyMx:
    """Expert weights as the oracle's MXFP8 dequantisation, made one expert
    at a time when the oracle asks for it."""

    def __init__(self, o, w):
        self.o, self.w = o, w

    def __getitem__(self, e):
        c, s = self.o.mxfp8_quantize(self.w[e].float().cpu().numpy())
        return self.o.mxfp8_dequantize(c, s)


def check_mx_layer(o, lay, tokens=None, y_bf16=False):
    c = lay.cfg
    m = moe.MoELayer(lay, y_bf16=y_bf16, weights="mxfp8")
    out, ids, w, counts = m()
    torch.cuda.synchronize()
    out, ids = out.cpu().numpy(), ids.cpu().numpy()
    tok = np.arange(c.T) if tokens is None else np.asarray(tokens)
    tok_t = torch.as_tensor(tok, device=lay.x.device)
    ref = o.forward(lay.x, lay.wg, lay.bias, _LazyMx(o, lay.w_gu), _LazyMx(o, lay.w_dn), c.k,
                    c.renorm, lay.ws_gu, lay.ws_dn, tokens=tok_t, permute=False)
    set_doubt, order_doubt = gh.routing_flags(ref)
    clean = ~(set_doubt | order_doubt)
    assert np.array_equal(ids[tok][clean], ref["ids"][clean])
    return gh.assert_close(out[tok][clean], ref["out"][clean], "mxfp8 layer output")


@pytest.mark.parametrize("name", ["light", "heavy_ragged", "i_tail", "shared", "hot"])
def test_layer_vs_oracle_small(oracle_lib, name):
    print(f"[case] mxfp8 oracle {name}", flush=True)
    ma, rel = check_mx_layer(oracle_lib, layer_on_gpu(MX_CASES[name]))
    print(f"[parity] mxfp8 {name}: max_abs={ma:.3e} relL2={rel:.3e}", flush=True)


@pytest.mark.parametrize("name,sample,y_bf16", [("decode", 16, True), ("prefill", 12, True),
                                                ("skew", 12, True), ("decode", 8, False)])
def test_layer_vs_oracle_full_size(oracle_lib, name, sample, y_bf16):
    """Full-size layers on MXFP8 weights against the oracle on a token
    sample (the oracle quantises only the experts those tokens reach)."""
    print(f"[case] mxfp8 full-size {name} y_bf16={y_bf16}", flush=True)
    cfg = synth.CONFIGS[name]
    lay = layer_on_gpu(cfg)
    tokens = np.sort(np.random.default_rng(2).choice(cfg.T, sample, replace=False))
    ma, rel = check_mx_layer(oracle_lib, lay, tokens=tokens, y_bf16=y_bf16)
    print(f"[parity] mxfp8 {name}: max_abs={ma:.3e} relL2={rel:.3e}", flush=True)
    del lay
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode", "prefill", "skew"])
def test_full_size_bitwise_and_quantisation_error(name):
    """Full-size layers: MXFP8 output equals the bf16 layer on weights
    dequantised by torch's float8_e4m3fn (a library decoding) bit for bit;
    the quantisation's own effect on the output is reported."""
    print(f"[case] mxfp8 {name} bitwise", flush=True)
    lay = layer_on_gpu(synth.CONFIGS[name])

    def dq(w):
        c, s = moe.quantize_mxfp8(w)
        v = c.view(torch.float8_e4m3fn).float()
        sc = torch.exp2(s.float() - 127.0).repeat_interleave(32, dim=-1)
        return (v * sc).to(torch.bfloat16)

    import dataclasses
    ref = dataclasses.replace(lay, w_gu=dq(lay.w_gu), w_dn=dq(lay.w_dn))
    out_mx = moe.MoELayer(lay, y_bf16=True, weights="mxfp8")()[0]
    out_16 = moe.MoELayer(ref, y_bf16=True, packed=True)()[0]
    out_orig = moe.MoELayer(lay, y_bf16=True, packed=True)()[0]
    torch.cuda.synchronize()
    assert torch.equal(out_mx.view(torch.int32), out_16.view(torch.int32))
    ma, rel = gh.err_stats(out_mx.cpu().numpy(), out_orig.cpu().numpy())
    print(f"[quant] mxfp8 vs bf16 weights ({name}): max_abs={ma:.3e} relL2={rel:.3e}", flush=True)
    assert rel < 0.1  # E4M3 keeps 4 significant bits: a few percent of the output
    del lay, ref
    torch.cuda.empty_cache()
