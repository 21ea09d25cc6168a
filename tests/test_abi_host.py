"""Host-side checks of the C ABI: the library loads, exports every symbol
include/moe.h declares, sizes its workspace without padding, and rejects bad
arguments with the documented codes before any HIP call.  No GPU needed:
every call here fails validation (or is a T == 0 no-op) before touching the
device."""
import ctypes
import os
import re

import pytest

from expert_ffn_layer_amd import moe, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from expert_ffn_layer_amd import build
        build.build()
    return moe.lib()


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(moe_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported(L):
    syms = header_symbols()
    assert set(syms) == set(moe.EXPORTED), syms
    for s in syms:
        assert hasattr(L, s), s


def test_library_has_gfx950_code():
    data = open(moe.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def shp(**kw):
    base = dict(T=64, H=4096, E=512, k=10, I=1024, I_shared=0, renorm=1, light_max_rows=-1,
                heavy_tile_rows=0, y_bf16=0, w_mxfp8=0, y_fp16=0)
    base.update(kw)
    return moe.MoeShape(*[base[n] for n, _ in moe.MoeShape._fields_])


def test_workspace_no_padding(L):
    """Workspace grows with the routed rows A*(H+I), never with E x capacity:
    at the prefill shape it stays within 10% of the h (bf16) and y (fp32)
    buffers."""
    c = synth.CONFIGS["prefill"]
    s = shp(T=c.T)
    need = moe.workspace_bytes(s)
    A = c.T * c.k
    hy = A * (c.I * 2 + c.H * 4)
    assert hy <= need <= 1.1 * hy
    small = moe.workspace_bytes(shp(T=64))
    assert small < need / 50


def test_workspace_bf16_y(L):
    """bf16 y takes exactly 2*A*H bytes less workspace (rounded to the
    256-byte alignment of each buffer)."""
    c = synth.CONFIGS["prefill"]
    A = c.T * c.k
    full = moe.workspace_bytes(shp(T=c.T))
    half = moe.workspace_bytes(shp(T=c.T, y_bf16=1))
    assert full - half == A * c.H * 2
    assert moe.make_shape(4, 64, 8, 2, 32, y_bf16=True).y_bf16 == 1
    # fp16 y: the same bytes as bf16
    assert moe.workspace_bytes(shp(T=c.T, y_fp16=1)) == half
    assert moe.make_shape(4, 64, 8, 2, 32, y_fp16=True).y_fp16 == 1


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), moe.MOE_ERR_SHAPE), (dict(T=-1), moe.MOE_ERR_SHAPE), (dict(k=600), moe.MOE_ERR_SHAPE),
    (dict(H=100), moe.MOE_ERR_UNSUPPORTED), (dict(I=48), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, k=4), moe.MOE_ERR_UNSUPPORTED), (dict(k=33), moe.MOE_ERR_UNSUPPORTED),
    (dict(renorm=2), moe.MOE_ERR_UNSUPPORTED), (dict(light_max_rows=65), moe.MOE_ERR_UNSUPPORTED),
    (dict(heavy_tile_rows=100), moe.MOE_ERR_UNSUPPORTED), (dict(heavy_tile_rows=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=40), moe.MOE_ERR_UNSUPPORTED), (dict(T=300000000, k=10), moe.MOE_ERR_SHAPE),
    (dict(T=1 << 19, k=1), moe.MOE_ERR_UNSUPPORTED), (dict(I=1 << 18), moe.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=1 << 18), moe.MOE_ERR_UNSUPPORTED),
    (dict(y_bf16=2), moe.MOE_ERR_UNSUPPORTED), (dict(y_bf16=-1), moe.MOE_ERR_UNSUPPORTED),
    (dict(w_mxfp8=2), moe.MOE_ERR_UNSUPPORTED), (dict(w_mxfp8=-1), moe.MOE_ERR_UNSUPPORTED),
    (dict(y_fp16=2), moe.MOE_ERR_UNSUPPORTED), (dict(y_fp16=1, y_bf16=1), moe.MOE_ERR_UNSUPPORTED),
])
def test_bad_shapes(L, kw, code):
    s = shp(**kw)
    assert moe.workspace_bytes(s) == 0
    P = ctypes.c_void_p(0x10000)
    rc = L.moe_router(ctypes.byref(s), P, P, None, P, P, None, P, 1 << 40, None)
    assert rc == code, moe.last_error()
    assert moe.last_error()


def test_argument_errors(L):
    s = shp()
    need = moe.workspace_bytes(s)
    P = ctypes.c_void_p(0x10000)
    bad = ctypes.c_void_p(0x10008)
    assert L.moe_router(ctypes.byref(s), None, P, None, P, P, None, P, need, None) == moe.MOE_ERR_NULL
    assert "x" in moe.last_error()
    assert L.moe_router(ctypes.byref(s), bad, P, None, P, P, None, P, need, None) == moe.MOE_ERR_ALIGN
    assert L.moe_router(ctypes.byref(s), P, P, None, P, P, None, P, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_router(ctypes.byref(s), P, P, None, P, P, None, ctypes.c_void_p(0x10010), need,
                        None) == moe.MOE_ERR_ALIGN
    assert L.moe_router(None, P, P, None, P, P, None, P, need, None) == moe.MOE_ERR_NULL
    assert L.moe_grouped_ffn(ctypes.byref(s), P, P, P, P, P, None, None, None, P, need,
                             None) == moe.MOE_ERR_NULL
    assert L.moe_combine(ctypes.byref(s), P, P, None, 0, P, None) == moe.MOE_ERR_NULL
    assert L.moe_shared_ffn(ctypes.byref(s), P, P, P, P, P, need, None) == moe.MOE_ERR_SHAPE
    s2 = shp(I_shared=1024)
    need2 = moe.workspace_bytes(s2)
    # shared expert requested but its down weights missing
    assert L.moe_forward(ctypes.byref(s2), P, P, None, P, P, None, P, None, P, None, None, None, P, need2,
                         None) == moe.MOE_ERR_NULL
    assert "ws_down" in moe.last_error()


def test_profile_hook_arguments(L):
    """The measurement hook validates its arguments without touching the GPU
    (it only stores the event handles)."""
    P = ctypes.c_void_p(0x10000)
    assert L.moe_profile_kernel(99, P, P) == moe.MOE_ERR_SHAPE
    assert L.moe_profile_kernel_launch(moe.KERNEL_ID["combine"], -2, P, P) == moe.MOE_ERR_SHAPE
    assert L.moe_profile_kernel_launch(moe.KERNEL_ID["combine"], 0, None, P) == moe.MOE_ERR_NULL
    assert L.moe_profile_kernel_launch(moe.KERNEL_ID["combine"], 1, P, P) == moe.MOE_OK
    assert moe.profile_launches() == 0
    assert L.moe_profile_kernel(-1, None, None) == moe.MOE_OK


def test_empty_batch_is_noop(L):
    """T == 0 validates and returns OK without launching anything."""
    s = shp(T=0)
    need = moe.workspace_bytes(s)
    P = ctypes.c_void_p(0x10000)
    assert L.moe_router(ctypes.byref(s), P, P, None, P, P, None, P, need, None) == moe.MOE_OK
    assert L.moe_grouped_ffn(ctypes.byref(s), P, P, P, P, P, None, None, P, P, need, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(s), P, P, P, 0, P, None) == moe.MOE_OK


def test_status_strings(L):
    for code in range(7):
        assert moe.status_string(code)


def test_packed_weight_bytes(L):
    """bf16: one copy, the records of 256-row weight tiles by 64-wide K
    stages (weight rows padded to 256, K to 64): the weights' own size when
    2I and H are multiples of 256 and I of 64."""
    s = shp()
    assert moe.packed_weight_bytes(s) == 512 * 3 * 1024 * 4096 * 2
    s = shp(E=3, k=2, H=320, I=96)
    assert moe.packed_weight_bytes(s) == 3 * (256 * 320 + 512 * 128) * 2
    assert moe.packed_weight_bytes(shp(H=100)) == 0


def test_pack_weights_argument_errors(L):
    s = shp()
    P = ctypes.c_void_p(0x10000)
    assert L.moe_pack_weights(ctypes.byref(s), P, P, None, None) == moe.MOE_ERR_NULL
    assert L.moe_pack_weights(ctypes.byref(s), None, P, P, None) == moe.MOE_ERR_NULL
    assert L.moe_pack_weights(ctypes.byref(s), P, P, ctypes.c_void_p(0x10010), None) == moe.MOE_ERR_ALIGN
    need = moe.workspace_bytes(s)
    # a misaligned packed buffer is refused before anything is enqueued
    assert L.moe_grouped_ffn(ctypes.byref(s), P, P, P, P, P, ctypes.c_void_p(0x10010), None, P, P,
                             need, None) == moe.MOE_ERR_ALIGN


def test_mxfp8_packed_bytes(L):
    """bf16 packed weights are one copy (records: rows padded to 256, K to
    64, 2 bytes per weight); MXFP8 holds two (light loop, heavy tiles), one
    byte per weight plus a scale byte per 32."""
    for (H, I) in ((4096, 1024), (64, 96), (128, 32)):
        E = 8
        b16 = moe.packed_weight_bytes(shp(E=E, H=H, I=I, k=2))
        mx = moe.packed_weight_bytes(shp(E=E, H=H, I=I, k=2, w_mxfp8=1))
        r256 = lambda n: (n + 255) // 256 * 256
        Ip = (I + 63) // 64 * 64
        assert b16 == E * (r256(2 * I) * H + r256(H) * Ip) * 2
        light = E * (2 * I * H + H * Ip) * (1 + 1 / 32)
        heavy = E * (r256(2 * I) * H + r256(H) * Ip) * (1 + 1 / 32)
        assert mx == light + heavy


def test_mxfp8_argument_errors(L):
    """Quantiser and MXFP8 packer validate before any HIP call; with
    w_mxfp8 = 1 the layer needs the packed weights and not the bf16 ones."""
    P = ctypes.c_void_p(0x10000)
    bad = ctypes.c_void_p(0x10008)
    assert L.moe_quantize_mxfp8(P, 4, 48, P, P, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_mxfp8(P, -1, 64, P, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quantize_mxfp8(P, 0, 64, None, None, None) == moe.MOE_OK
    assert L.moe_quantize_mxfp8(None, 4, 64, P, P, None) == moe.MOE_ERR_NULL
    assert L.moe_quantize_mxfp8(bad, 4, 64, P, P, None) == moe.MOE_ERR_ALIGN
    assert L.moe_quantize_mxfp8(P, 4, 64, P, None, None) == moe.MOE_ERR_NULL
    s16, smx = shp(), shp(w_mxfp8=1)
    assert L.moe_pack_weights_mxfp8(ctypes.byref(s16), P, P, P, P, P, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_weights_mxfp8(ctypes.byref(smx), P, None, P, P, P, None) == moe.MOE_ERR_NULL
    assert L.moe_pack_weights_mxfp8(ctypes.byref(smx), P, P, P, P,
                                    ctypes.c_void_p(0x10010), None) == moe.MOE_ERR_ALIGN
    need = moe.workspace_bytes(smx)
    # no packed weights with w_mxfp8 = 1
    assert L.moe_grouped_ffn(ctypes.byref(smx), P, P, P, None, None, None, None, P, P, need,
                             None) == moe.MOE_ERR_NULL
    assert "packed" in moe.last_error()
    assert L.moe_forward(ctypes.byref(smx), P, P, None, None, None, None, None, None, P, None, None,
                         None, P, need, None) == moe.MOE_ERR_NULL
    assert "packed" in moe.last_error()


def test_mxfp8_tile_limit(L):
    """MXFP8 heavy tiles stop at 192 rows: a forced 256 is rejected."""
    assert moe.workspace_bytes(shp(w_mxfp8=1, heavy_tile_rows=256)) == 0
    assert moe.workspace_bytes(shp(w_mxfp8=1, heavy_tile_rows=192)) > 0
    assert moe.workspace_bytes(shp(w_mxfp8=1, heavy_tile_rows=0)) > 0


def test_plain_weights_optional_with_packed(L):
    """With packed weights the plain layout is not read: NULL w_gate_up /
    w_down pass validation (the call then stops at the misaligned y)."""
    s = shp()
    need = moe.workspace_bytes(s)
    P = ctypes.c_void_p(0x10000)
    bad = ctypes.c_void_p(0x10008)
    rc = L.moe_grouped_ffn(ctypes.byref(s), P, P, P, None, None, P, None, bad, P, need, None)
    assert rc == moe.MOE_ERR_ALIGN and "y" in moe.last_error()
    # without packed weights they are required
    rc = L.moe_grouped_ffn(ctypes.byref(s), P, P, P, None, None, None, None, P, P, need, None)
    assert rc == moe.MOE_ERR_NULL and "w_gate_up" in moe.last_error()
    rc = L.moe_forward(ctypes.byref(s), P, P, None, None, None, P, None, None, bad, None, None,
                       None, P, need, None)
    assert rc == moe.MOE_ERR_ALIGN and "out" in moe.last_error()


def test_workspace_holds_plan_of_repeated_ids(L):
    """moe_permute accepts ids repeated within a token, so the plan region is
    sized for the tiles of an expert holding every routed row: at T <= 64 the
    workspace still grows with the rows, by two ints per possible tile."""
    a = moe.workspace_bytes(shp(T=64))
    b = moe.workspace_bytes(shp(T=64, light_max_rows=0))
    assert a > 0 and b > 0
    # the all-heavy layout can hold at least A/128 + 1 tiles as well
    assert abs(a - b) < 64 * 1024


def test_noalloc_limits(L):
    """moe_forward_noalloc checks the shape and its scratch size on the host:
    an invalid shape gives moe_forward's code, an oversized one
    MOE_ERR_WORKSPACE naming the limit, both before any HIP call."""
    P = ctypes.c_void_p(0x10000)
    big = shp(T=4096)
    assert moe.workspace_bytes(big) > moe.NOALLOC_SCRATCH_BYTES
    rc = L.moe_forward_noalloc(ctypes.byref(big), P, P, None, P, P, None, None, None, P, None,
                               None, None, None)
    assert rc == moe.MOE_ERR_WORKSPACE and "MOE_NOALLOC_SCRATCH_BYTES" in moe.last_error()
    rc = L.moe_forward_noalloc(ctypes.byref(shp(k=0)), P, P, None, P, P, None, None, None, P,
                               None, None, None, None)
    assert rc == moe.MOE_ERR_SHAPE
    assert moe.workspace_bytes(shp(T=64)) <= moe.NOALLOC_SCRATCH_BYTES
    # the header's limit is the binding's
    text = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20
