"""ctypes binding of libmoe.so (declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the current HIP device; bf16 tensors
are passed as their raw 16-bit patterns.  The binding checks dtypes, devices,
contiguity and sizes against the shape (the C ABI cannot see buffer sizes),
then calls the entry point of the same name on the current torch stream.
Importing this module does not load the library; the first call does, and
raises if ``libmoe.so`` has not been built.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

# MOE_LIB_PATH names another build of the same C ABI (e.g. a sanitizer build
# of the host code for the host-side tests).
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL = 1
MOE_ERR_SHAPE = 2
MOE_ERR_UNSUPPORTED = 3
MOE_ERR_ALIGN = 4
MOE_ERR_WORKSPACE = 5
MOE_ERR_HIP = 6

EXPORTED = ("moe_workspace_bytes", "moe_packed_weight_bytes", "moe_status_string",
            "moe_last_error", "moe_router", "moe_permute", "moe_pack_weights", "moe_grouped_ffn",
            "moe_shared_ffn", "moe_combine", "moe_forward", "moe_profile_kernel",
            "moe_profile_kernel_launch", "moe_profile_launches", "moe_quantize_mxfp8",
            "moe_pack_weights_mxfp8", "moe_forward_noalloc")
# Fixed scratch of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES in moe.h).
NOALLOC_SCRATCH_BYTES = 64 << 20

# enum moe_kernel
KERNELS = ("router_gemm", "router_select", "perm_count", "perm_scan", "perm_scatter", "ffn_plan",
           "gateup_light", "gateup_heavy", "down_light", "down_heavy", "combine", "perm_small")
KERNEL_ID = {n: i for i, n in enumerate(KERNELS)}
# Experts with 1..LIGHT_MAX_ROWS rows take the light loop when
# light_max_rows is left at -1 (the C ABI's default).
LIGHT_MAX_ROWS = 64
LIGHT_MEAN_ROWS = 8  # the default's device-side rule (moe_shape.light_max_rows = -1)
LIGHT_TAIL_ROWS = 8  # light threshold of that rule when the mean is above LIGHT_MEAN_ROWS


def light_experts(counts, shape):
    """Boolean mask of the experts that take the light loop for these routing
    counts (numpy int array [E]), the rule the library's plan applies."""
    import numpy as np
    counts = np.asarray(counts)
    lm = shape.light_max_rows
    if lm < 0:
        if shape.T <= LIGHT_MAX_ROWS:
            lm = LIGHT_MAX_ROWS
        elif shape.T * shape.k > LIGHT_MEAN_ROWS * shape.E:
            lm = LIGHT_TAIL_ROWS  # the mean is above LIGHT_MEAN_ROWS whatever the routing
        else:
            touched = int((counts > 0).sum())
            lm = LIGHT_MAX_ROWS if int(counts.sum()) <= LIGHT_MEAN_ROWS * touched else LIGHT_TAIL_ROWS
    return (counts >= 1) & (counts <= lm)


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("light_max_rows", ctypes.c_int32),
                ("heavy_tile_rows", ctypes.c_int32), ("y_bf16", ctypes.c_int32),
                ("w_mxfp8", ctypes.c_int32), ("y_fp16", ctypes.c_int32)]

    def __repr__(self):
        return ("MoeShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


class MoeError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


_libs = {}
_active_path = LIB_PATH
_vp = ctypes.c_void_p
_sp = ctypes.POINTER(MoeShape)


@contextlib.contextmanager
def using_library(path: str):
    """Route every call in the block to another build of the same C ABI
    (e.g. a build with other compile-time tunables), then back."""
    global _active_path
    prev = _active_path
    _active_path = path
    try:
        yield lib()
    finally:
        _active_path = prev


def lib() -> ctypes.CDLL:
    path = _active_path
    L = _libs.get(path)
    if L is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m expert_ffn_layer_amd.build`")
        L = ctypes.CDLL(path)
        L.moe_workspace_bytes.argtypes = [_sp]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_packed_weight_bytes.argtypes = [_sp]
        L.moe_packed_weight_bytes.restype = ctypes.c_size_t
        L.moe_pack_weights.argtypes = [_sp] + [_vp] * 4
        L.moe_quantize_mxfp8.argtypes = [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp]
        L.moe_pack_weights_mxfp8.argtypes = [_sp] + [_vp] * 6
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_router.argtypes = [_sp] + [_vp] * 7 + [ctypes.c_size_t, _vp]
        L.moe_permute.argtypes = [_sp] + [_vp] * 6 + [ctypes.c_size_t, _vp]
        L.moe_grouped_ffn.argtypes = [_sp] + [_vp] * 9 + [ctypes.c_size_t, _vp]
        L.moe_shared_ffn.argtypes = [_sp] + [_vp] * 5 + [ctypes.c_size_t, _vp]
        L.moe_combine.argtypes = [_sp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp]
        L.moe_forward.argtypes = [_sp] + [_vp] * 13 + [ctypes.c_size_t, _vp]
        L.moe_forward_noalloc.argtypes = [_sp] + [_vp] * 12 + [_vp]
        L.moe_profile_kernel.argtypes = [ctypes.c_int, _vp, _vp]
        L.moe_profile_kernel_launch.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp]
        L.moe_profile_launches.argtypes = []
        L.moe_profile_launches.restype = ctypes.c_longlong
        for name in ("moe_router", "moe_permute", "moe_pack_weights", "moe_grouped_ffn",
                     "moe_shared_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc",
                     "moe_profile_kernel", "moe_profile_kernel_launch"):
            getattr(L, name).restype = ctypes.c_int
        _libs[path] = L
    return L


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, f"{status_string(rc)}: {last_error()}")


def make_shape(T, H, E, k, I, I_shared=0, renorm=1, light_max_rows=-1,
               heavy_tile_rows=0, y_bf16=0, w_mxfp8=0, y_fp16=0) -> MoeShape:
    return MoeShape(T, H, E, k, I, I_shared, renorm, light_max_rows, heavy_tile_rows,
                    int(bool(y_bf16)), int(bool(w_mxfp8)), int(bool(y_fp16)))


def workspace_bytes(shape: MoeShape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def alloc_workspace(shape: MoeShape, device=None) -> torch.Tensor:
    n = workspace_bytes(shape)
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, f"invalid shape {shape}")
    return torch.empty(n, dtype=torch.uint8, device=device or torch.device("cuda"))


def packed_weight_bytes(shape: MoeShape) -> int:
    return int(lib().moe_packed_weight_bytes(ctypes.byref(shape)))


def pack_weights(shape: MoeShape, w_gate_up, w_down, stream=None) -> torch.Tensor:
    """One-time re-layout of the routed expert weights into the records both
    FFN loops stream (moe_pack_weights); returns the packed uint8 device
    buffer, one copy of the weights."""
    n = packed_weight_bytes(shape)
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, f"invalid shape {shape}")
    E, H, I = shape.E, shape.H, shape.I
    out = torch.empty(n, dtype=torch.uint8, device=w_gate_up.device)
    _check(lib().moe_pack_weights(ctypes.byref(shape),
                                  _ptr(w_gate_up, "w_gate_up", BF16, E * 2 * I * H),
                                  _ptr(w_down, "w_down", BF16, E * H * I), out.data_ptr(),
                                  _stream(stream)))
    return out


def quantize_mxfp8(w, stream=None):
    """MXFP8 (OCP MX, E4M3 codes, one E8M0 scale per 32 values along the last
    dimension) of a bf16 device tensor [..., K]: returns (codes uint8
    [..., K], scales uint8 [..., K/32]) (moe_quantize_mxfp8)."""
    if w.dtype != BF16 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous bf16 device tensor")
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (K // 32,), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quantize_mxfp8(w.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(),
                                    _stream(stream)))
    return codes, scales


def pack_weights_mxfp8(shape: MoeShape, codes_gate_up, scales_gate_up, codes_down, scales_down,
                       stream=None) -> torch.Tensor:
    """Packed MXFP8 expert weights for a shape with w_mxfp8 = 1
    (moe_pack_weights_mxfp8); returns the uint8 device buffer."""
    if not shape.w_mxfp8:
        raise ValueError("shape.w_mxfp8 must be 1")
    n = packed_weight_bytes(shape)
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, f"invalid shape {shape}")
    E, H, I = shape.E, shape.H, shape.I
    U8 = torch.uint8
    out = torch.empty(n, dtype=U8, device=codes_gate_up.device)
    _check(lib().moe_pack_weights_mxfp8(
        ctypes.byref(shape), _ptr(codes_gate_up, "codes_gate_up", U8, E * 2 * I * H),
        _ptr(scales_gate_up, "scales_gate_up", U8, E * 2 * I * H // 32),
        _ptr(codes_down, "codes_down", U8, E * H * I),
        _ptr(scales_down, "scales_down", U8, E * H * I // 32), out.data_ptr(), _stream(stream)))
    return out


def _packed(p: Optional[torch.Tensor], shape: MoeShape):
    if p is None:
        return None
    n = packed_weight_bytes(shape)
    if not p.is_cuda or p.dtype != torch.uint8 or p.numel() < n:
        raise ValueError(f"packed_weights must be a uint8 device tensor of >= {n} bytes")
    return p.data_ptr()


def _ptr(t: Optional[torch.Tensor], name: str, dtype, numel: Optional[int] = None,
         optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _ws(ws: torch.Tensor, shape: MoeShape):
    need = workspace_bytes(shape)
    if ws is None or not ws.is_cuda or ws.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 device tensor")
    if ws.numel() < need:
        raise MoeError(MOE_ERR_WORKSPACE, f"workspace has {ws.numel()} bytes, needs {need}")
    return ws.data_ptr(), ws.numel()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


BF16, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def router(shape, x, w_router, bias, topk_ids, topk_w, probs, workspace, stream=None):
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    args = [_ptr(x, "x", BF16, T * H), _ptr(w_router, "w_router", F32, H * E),
            _ptr(bias, "bias", F32, E, optional=True), _ptr(topk_ids, "topk_ids", I32, T * k),
            _ptr(topk_w, "topk_w", F32, T * k), _ptr(probs, "probs", F32, T * E, optional=True)]
    wp, wn = _ws(workspace, shape)
    _check(lib().moe_router(ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def permute(shape, topk_ids, counts, offsets, sorted_token_ids, inv_pos, workspace, stream=None):
    A, E = shape.T * shape.k, shape.E
    args = [_ptr(topk_ids, "topk_ids", I32, A), _ptr(counts, "counts", I32, E),
            _ptr(offsets, "offsets", I32, E + 1),
            _ptr(sorted_token_ids, "sorted_token_ids", I32, A), _ptr(inv_pos, "inv_pos", I32, A)]
    wp, wn = _ws(workspace, shape)
    _check(lib().moe_permute(ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def grouped_ffn(shape, x, sorted_token_ids, offsets, w_gate_up, w_down, h, y, workspace,
                stream=None, packed_weights=None):
    T, H, E, I, A = shape.T, shape.H, shape.E, shape.I, shape.T * shape.k
    args = [_ptr(x, "x", BF16, T * H), _ptr(sorted_token_ids, "sorted_token_ids", I32, A),
            _ptr(offsets, "offsets", I32, E + 1),
            _ptr(w_gate_up, "w_gate_up", BF16, E * 2 * I * H, optional=packed_weights is not None),
            _ptr(w_down, "w_down", BF16, E * H * I, optional=packed_weights is not None),
            _packed(packed_weights, shape),
            _ptr(h, "h", BF16, A * I, optional=True),
            _ptr(y, "y", y_dtype(shape), A * H)]
    wp, wn = _ws(workspace, shape)
    _check(lib().moe_grouped_ffn(ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def shared_ffn(shape, x, ws_gate_up, ws_down, out, workspace, stream=None):
    T, H, Is = shape.T, shape.H, shape.I_shared
    args = [_ptr(x, "x", BF16, T * H), _ptr(ws_gate_up, "ws_gate_up", BF16, 2 * Is * H),
            _ptr(ws_down, "ws_down", BF16, H * Is), _ptr(out, "out", F32, T * H)]
    wp, wn = _ws(workspace, shape)
    _check(lib().moe_shared_ffn(ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def y_dtype(shape) -> torch.dtype:
    """Element type of the routed expert outputs y for ``shape``."""
    return torch.float16 if shape.y_fp16 else (BF16 if shape.y_bf16 else F32)


def combine(shape, y, inv_pos, topk_w, accumulate, out, stream=None):
    T, H, A = shape.T, shape.H, shape.T * shape.k
    args = [_ptr(y, "y", y_dtype(shape), A * H), _ptr(inv_pos, "inv_pos", I32, A),
            _ptr(topk_w, "topk_w", F32, A)]
    _check(lib().moe_combine(ctypes.byref(shape), *args, int(bool(accumulate)),
                             _ptr(out, "out", F32, T * H), _stream(stream)))


def forward(shape, x, w_router, bias, w_gate_up, w_down, ws_gate_up, ws_down, out, workspace,
            topk_ids_out=None, topk_w_out=None, counts_out=None, stream=None, packed_weights=None):
    args = _forward_args(shape, x, w_router, bias, w_gate_up, w_down, ws_gate_up, ws_down, out,
                         topk_ids_out, topk_w_out, counts_out, packed_weights)
    wp, wn = _ws(workspace, shape)
    _check(lib().moe_forward(ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def forward_noalloc(shape, x, w_router, bias, w_gate_up, w_down, ws_gate_up, ws_down, out,
                    topk_ids_out=None, topk_w_out=None, counts_out=None, stream=None,
                    packed_weights=None):
    """moe_forward_noalloc: the layer on the library's fixed per-GPU scratch
    array (no workspace argument; shapes needing more than
    NOALLOC_SCRATCH_BYTES of scratch are rejected)."""
    args = _forward_args(shape, x, w_router, bias, w_gate_up, w_down, ws_gate_up, ws_down, out,
                         topk_ids_out, topk_w_out, counts_out, packed_weights)
    _check(lib().moe_forward_noalloc(ctypes.byref(shape), *args, _stream(stream)))


def _forward_args(shape, x, w_router, bias, w_gate_up, w_down, ws_gate_up, ws_down, out,
                  topk_ids_out, topk_w_out, counts_out, packed_weights):
    T, H, E, k, I, Is = shape.T, shape.H, shape.E, shape.k, shape.I, shape.I_shared
    return [_ptr(x, "x", BF16, T * H), _ptr(w_router, "w_router", F32, H * E),
            _ptr(bias, "bias", F32, E, optional=True),
            _ptr(w_gate_up, "w_gate_up", BF16, E * 2 * I * H, optional=packed_weights is not None),
            _ptr(w_down, "w_down", BF16, E * H * I, optional=packed_weights is not None),
            _packed(packed_weights, shape),
            _ptr(ws_gate_up, "ws_gate_up", BF16, 2 * Is * H, optional=True),
            _ptr(ws_down, "ws_down", BF16, H * Is, optional=True),
            _ptr(out, "out", F32, T * H),
            _ptr(topk_ids_out, "topk_ids_out", I32, T * k, optional=True),
            _ptr(topk_w_out, "topk_w_out", F32, T * k, optional=True),
            _ptr(counts_out, "counts_out", I32, E, optional=True)]


def profile_kernel(name: Optional[str], start=None, stop=None, launch: int = -1) -> None:
    """Bracket every launch of kernel ``name`` (or only its ``launch``-th one
    from now on) with the two torch.cuda.Event, or None to turn the hook off."""
    if name is None:
        _check(lib().moe_profile_kernel(-1, None, None))
        return
    for ev in (start, stop):
        if not ev.cuda_event:  # torch creates the HIP event on first record
            ev.record()
    _check(lib().moe_profile_kernel_launch(KERNEL_ID[name], int(launch), start.cuda_event,
                                           stop.cuda_event))


def profile_launches() -> int:
    """Launches of the hooked kernel since profile_kernel() set the hook."""
    return int(lib().moe_profile_launches())


class MoELayer:
    """Convenience holder: weights + one workspace; ``__call__`` runs
    moe_forward and returns (out, topk_ids, topk_w, counts)."""

    def __init__(self, layer, light_max_rows: int = -1, heavy_tile_rows: int = 0,
                 packed: bool = False, y_bf16: bool = False, weights: str = "bf16",
                 y_fp16: bool = False):
        """weights="mxfp8" quantises the routed expert weights to MXFP8 on the
        device and runs the layer on them (packed implied)."""
        if weights not in ("bf16", "mxfp8"):
            raise ValueError("weights must be 'bf16' or 'mxfp8'")
        c = layer.cfg
        self.layer = layer
        mx = weights == "mxfp8"
        self.shape = make_shape(c.T, c.H, c.E, c.k, c.I, c.I_shared, c.renorm, light_max_rows,
                                heavy_tile_rows, y_bf16, mx, y_fp16)
        self.workspace = alloc_workspace(self.shape, layer.x.device)
        if mx:
            q_gu, s_gu = quantize_mxfp8(layer.w_gu)
            q_dn, s_dn = quantize_mxfp8(layer.w_dn)
            self.packed = pack_weights_mxfp8(self.shape, q_gu, s_gu, q_dn, s_dn)
            del q_gu, s_gu, q_dn, s_dn
        else:
            self.packed = pack_weights(self.shape, layer.w_gu, layer.w_dn) if packed else None

    def __call__(self, x=None, out=None, want_routing=True):
        L, s = self.layer, self.shape
        x = L.x if x is None else x
        dev = x.device
        out = torch.empty((s.T, s.H), dtype=F32, device=dev) if out is None else out
        ids = torch.empty((s.T, s.k), dtype=I32, device=dev) if want_routing else None
        w = torch.empty((s.T, s.k), dtype=F32, device=dev) if want_routing else None
        counts = torch.empty((s.E,), dtype=I32, device=dev) if want_routing else None
        plain = self.packed is None
        forward(s, x, L.wg, L.bias, L.w_gu if plain else None, L.w_dn if plain else None,
                L.ws_gu, L.ws_dn, out, self.workspace, ids, w, counts, packed_weights=self.packed)
        return out, ids, w, counts
