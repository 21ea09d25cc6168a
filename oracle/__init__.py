"""CPU oracle of the sparse MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The GPU library neither imports nor links it, and it imports
nothing from the GPU side; the two meet only in the seeded input generator,
which holds no layer arithmetic.

The arithmetic lives in ``moe_oracle.c`` (plain fp32 loops).  This wrapper
only marshals arrays and composes the stages in the order of the layer's
definition:

    logits -> softmax/top-k/renormalise -> per-(token, slot) expert FFN
    -> weighted combine (+ shared expert)

The per-(token, slot) FFN rows are independent, so the wrapper evaluates them
expert by expert (one expert's weights upcast to fp32 at a time) without
changing any result.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
LIB = os.path.join(_HERE, "libmoe_oracle.so")
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", "-fvisibility=hidden", "-Wall"]

_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(out: str = LIB, src: str = SRC) -> str:
    """Compile the oracle with gcc (plain C99 + OpenMP)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build_from_source_text(text: str, workdir: Optional[str] = None) -> str:
    """Compile a modified copy of the oracle source (used by the tests that
    plant mistakes in the oracle to show the pins catch them)."""
    d = workdir or tempfile.mkdtemp(prefix="oref_")
    src = os.path.join(d, "moe_oracle_variant.c")
    with open(src, "w") as f:
        f.write(text)
    return build(os.path.join(d, "libmoe_oracle_variant.so"), src)


def _np32(a) -> np.ndarray:
    """Exact fp32 host copy of a torch tensor (any float dtype) or array."""
    if type(a).__module__.startswith("torch"):
        import torch
        a = a.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a: np.ndarray, t=_f32p):
    return a.ctypes.data_as(t)


class Oracle:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with oracle.build() "
                "(or __graft_entry__.build())")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oref_set_threads.argtypes = [ctypes.c_int]
        lib.oref_max_threads.restype = ctypes.c_int
        lib.oref_logits.argtypes = [ctypes.c_int] * 3 + [_f32p] * 4
        lib.oref_route.argtypes = [ctypes.c_int] * 4 + [_f32p, _i32p] + [_f32p] * 4
        lib.oref_route.restype = ctypes.c_int
        lib.oref_weights_for_ids.argtypes = [ctypes.c_int] * 4 + [_f32p, _i32p, _f32p]
        lib.oref_weights_for_ids.restype = ctypes.c_int
        lib.oref_permute.argtypes = [ctypes.c_int] * 3 + [_i32p] * 5
        lib.oref_permute.restype = ctypes.c_int
        lib.oref_expert_ffn.argtypes = [ctypes.c_int] * 3 + [_f32p] * 4
        lib.oref_combine.argtypes = [ctypes.c_int] * 3 + [_f32p] * 4
        lib.oref_mxfp8_quantize.argtypes = [ctypes.c_long, ctypes.c_int, _f32p, _u8p, _u8p]
        lib.oref_mxfp8_quantize.restype = ctypes.c_int
        lib.oref_mxfp8_dequantize.argtypes = [ctypes.c_long, ctypes.c_int, _u8p, _u8p, _f32p]
        self.lib = lib

    # -- threads ----------------------------------------------------------
    def set_threads(self, n: int) -> None:
        self.lib.oref_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.oref_max_threads())

    # -- stages -----------------------------------------------------------
    def logits(self, x, wg, bias=None) -> np.ndarray:
        x = _np32(x)
        wg = _np32(wg)
        T, H = x.shape
        H2, E = wg.shape
        assert H == H2
        b = None if bias is None else _np32(bias)
        out = np.empty((T, E), np.float32)
        self.lib.oref_logits(T, H, E, _p(x), _p(wg), None if b is None else _p(b), _p(out))
        return out

    def route(self, logits, k: int, renorm: int = 1):
        lg = _np32(logits)
        T, E = lg.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float32)
        probs = np.empty((T, E), np.float32)
        gk = np.empty((T,), np.float32)
        gi = np.empty((T,), np.float32)
        rc = self.lib.oref_route(T, E, k, int(renorm), _p(lg), _p(ids, _i32p), _p(w),
                                 _p(probs), _p(gk), _p(gi))
        if rc != 0:
            raise ValueError(f"oref_route failed ({rc})")
        return dict(ids=ids, w=w, probs=probs, gap_k=gk, gap_in=gi)

    def weights_for_ids(self, logits, ids, renorm: int = 1) -> np.ndarray:
        lg = _np32(logits)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, E = lg.shape
        k = ids.shape[1]
        w = np.empty((T, k), np.float32)
        rc = self.lib.oref_weights_for_ids(T, E, k, int(renorm), _p(lg), _p(ids, _i32p), _p(w))
        if rc != 0:
            raise ValueError(f"oref_weights_for_ids failed ({rc})")
        return w

    def permute(self, ids, E: int):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, k = ids.shape
        counts = np.empty((E,), np.int32)
        offsets = np.empty((E + 1,), np.int32)
        sorted_ids = np.empty((T * k,), np.int32)
        inv_pos = np.empty((T * k,), np.int32)
        rc = self.lib.oref_permute(T, k, E, _p(ids, _i32p), _p(counts, _i32p),
                                   _p(offsets, _i32p), _p(sorted_ids, _i32p),
                                   _p(inv_pos, _i32p))
        if rc != 0:
            raise ValueError(f"oref_permute failed ({rc})")
        return dict(counts=counts, offsets=offsets, sorted_token_ids=sorted_ids,
                    inv_pos=inv_pos)

    def expert_ffn(self, xr, w_gu, w_dn) -> np.ndarray:
        xr = _np32(xr)
        w_gu = _np32(w_gu)
        w_dn = _np32(w_dn)
        n, H = xr.shape
        I2, H2 = w_gu.shape
        assert H2 == H and w_dn.shape == (H, I2 // 2)
        y = np.empty((n, H), np.float32)
        if n:
            self.lib.oref_expert_ffn(n, H, I2 // 2, _p(xr), _p(w_gu), _p(w_dn), _p(y))
        return y

    def combine(self, w, y, shared=None) -> np.ndarray:
        w = _np32(w)
        y = _np32(y)
        T, k = w.shape
        H = y.shape[1]
        assert y.shape[0] == T * k
        s = None if shared is None else _np32(shared)
        out = np.empty((T, H), np.float32)
        self.lib.oref_combine(T, H, k, _p(w), _p(y), None if s is None else _p(s), _p(out))
        return out

    # -- MXFP8 expert weights (OCP MX v1.0, E4M3 elements, 32-value blocks) --
    def mxfp8_quantize(self, w):
        """w [..., K] (K % 32 == 0) -> (codes uint8 [..., K], scales uint8
        [..., K/32]); see oref_mxfp8_quantize for the rule."""
        w = _np32(w)
        K = w.shape[-1]
        rows = w.size // K if K else 0
        codes = np.empty(w.shape, np.uint8)
        scales = np.empty(w.shape[:-1] + (K // 32,), np.uint8)
        rc = self.lib.oref_mxfp8_quantize(rows, K, _p(w), _p(codes, _u8p), _p(scales, _u8p))
        if rc != 0:
            raise ValueError(f"oref_mxfp8_quantize failed ({rc})")
        return codes, scales

    def mxfp8_dequantize(self, codes, scales) -> np.ndarray:
        """codes uint8 [..., K], scales uint8 [..., K/32] -> fp32 [..., K]."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        K = codes.shape[-1]
        assert K % 32 == 0 and scales.shape == codes.shape[:-1] + (K // 32,)
        out = np.empty(codes.shape, np.float32)
        rows = codes.size // K if K else 0
        self.lib.oref_mxfp8_dequantize(rows, K, _p(codes, _u8p), _p(scales, _u8p), _p(out))
        return out

    # -- composition ------------------------------------------------------
    def routed_rows(self, x32: np.ndarray, ids: np.ndarray, w_gu, w_dn) -> np.ndarray:
        """y[t*k+j] = FFN_{ids[t,j]}(x[t]) for every (t, j); evaluated one
        expert at a time so only that expert's weights are upcast."""
        T, k = ids.shape
        H = x32.shape[1]
        y = np.empty((T * k, H), np.float32)
        flat = ids.reshape(-1)
        for e in np.unique(flat):
            rows = np.nonzero(flat == e)[0]
            y[rows] = self.expert_ffn(x32[rows // k], w_gu[int(e)], w_dn[int(e)])
        return y

    def forward(self, x, wg, bias, w_gu, w_dn, k: int, renorm: int = 1,
                ws_gu=None, ws_dn=None, tokens=None, ids=None, permute=True):
        """The whole layer.  ``tokens`` restricts evaluation to a subset of
        token rows (each token's output depends only on its own row).
        ``ids`` overrides the routing choice (weights are still taken from
        this oracle's probabilities of those ids when given)."""
        x32 = _np32(x if tokens is None else x[tokens])
        lg = self.logits(x32, wg, bias)
        r = self.route(lg, k, renorm)
        if ids is not None:
            ids = np.ascontiguousarray(ids, dtype=np.int32)
            r["w"] = self.weights_for_ids(lg, ids, renorm)
            r["ids"] = ids
        y = self.routed_rows(x32, r["ids"], w_gu, w_dn)
        shared = None
        if ws_gu is not None:
            shared = self.expert_ffn(x32, ws_gu, ws_dn)
        out = self.combine(r["w"], y, shared)
        res = dict(logits=lg, out=out, y=y, shared=shared, **r)
        if permute and tokens is None:
            res.update(self.permute(r["ids"], wg.shape[1]))
        return res


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
