"""Host-only checks of the C ABI (no GPU needed).

* the library loads and exports every function include/moe_nvfp4.h declares;
* every validation failure returns its documented status before any HIP call
  (fake, aligned, non-null addresses are never dereferenced on this path);
* workspace size queries are consistent.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x10000)  # aligned fake device address; validation fails before any use
P2 = ctypes.c_void_p(0x20000)


@pytest.fixture(scope="module")
def L():
    from nvfp4_w4a4_mixture_amd import _lib

    return _lib.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"sizeof"})


def test_header_symbols_exported(L):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_binding_signatures_cover_header():
    from nvfp4_w4a4_mixture_amd import _lib

    assert sorted(_lib.SIGNATURES) == header_functions()


def test_version(L):
    assert L.moe_abi_version() == 3


def _route(L, x=P, T=4, H=64, ldx=64, wr=P, bias=P, E=8, k=2, rsf=2.5, ws=P2, wsb=1 << 20):
    return L.moe_route(x, T, H, ldx, wr, bias, E, k, rsf, P, P, P, P, P, ws, wsb, None)


def test_route_validation(L):
    assert _route(L, x=None) == NULL
    assert _route(L, bias=None) == NULL
    assert _route(L, T=-1) == SHAPE
    assert _route(L, ldx=32) == SHAPE
    assert _route(L, k=0) == SHAPE
    assert _route(L, k=9, E=8) == SHAPE
    assert _route(L, E=257, k=8) == SHAPE
    assert _route(L, rsf=0.0) == SHAPE
    assert _route(L, ws=None) == WORKSPACE
    assert _route(L, wsb=4) == WORKSPACE
    assert _route(L, ws=ctypes.c_void_p(0x10008)) == ALIGN
    assert b"moe_route" in L.moe_last_error()


def test_route_quantize_validation(L):
    rq = L.moe_route_quantize

    def call(x=P, T=4, H=64, ldx=64, codes=P, scales=P, gs=P):
        return rq(x, T, H, ldx, P, P, 8, 2, 2.5, gs, codes, scales, P, P, P, P, P, P2, 1 << 20, None)

    assert call(codes=None) == NULL
    assert call(gs=None) == NULL
    assert call(scales=None) == NULL
    assert call(H=40, ldx=40) == SHAPE  # H % 16
    assert call(ldx=68) == ALIGN  # ldx % 8
    assert call(x=ctypes.c_void_p(0x10008)) == ALIGN
    assert call(codes=ctypes.c_void_p(0x10004)) == ALIGN
    assert b"moe_route_quantize" in L.moe_last_error()


def test_quantize_act_validation(L):
    q = L.nvfp4_quantize_act
    assert q(None, 4, 64, 64, P, P, P, None) == NULL
    assert q(P, 4, 60, 64, P, P, P, None) == SHAPE  # cols % 16
    assert q(P, 4, 64, 32, P, P, P, None) == SHAPE  # ld < cols
    assert q(P, -1, 64, 64, P, P, P, None) == SHAPE
    assert q(P, 4, 64, 68, P, P, P, None) == ALIGN  # ld % 8
    assert q(ctypes.c_void_p(0x10002), 4, 64, 64, P, P, P, None) == ALIGN
    assert q(P, 4, 64, 64, P, ctypes.c_void_p(0x10004), P, None) == ALIGN
    assert q(P, 0, 64, 64, P, P, P, None) == OK  # no rows: no-op, no device call


def test_quantize_weights_validation(L):
    q = L.nvfp4_quantize_weights
    assert q(P, 2, 16, 128, P, P, None, None) == NULL
    assert q(P, 2, 16, 40, P, P, P, None) == SHAPE
    assert q(P, 2, 16, 64, P, P, P, None) == SHAPE  # cols % 128 (tiled scales)
    assert q(P, 2, 24, 128, P, P, P, None) == SHAPE  # rows % 16
    assert q(P, 2, 0, 128, P, P, P, None) == SHAPE
    assert q(ctypes.c_void_p(0x10008), 2, 16, 128, P, P, P, None) == ALIGN
    assert q(P, 0, 16, 128, P, P, P, None) == OK


def _ffn(L, T=16, H=256, E=8, I=128, k=2, ws=P2, wsb=1 << 30, xc=P, sq=None, po=P, ps=P):
    return L.moe_nvfp4_grouped_ffn(xc, P, P, T, H, P, P, P, P, P, P, P, E, I, k, P, P, P, po, ps, sq, ws, wsb, None)


def test_ffn_validation(L):
    assert _ffn(L, xc=None) == NULL
    assert _ffn(L, po=None) == NULL
    assert _ffn(L, ps=None) == NULL
    assert _ffn(L, H=200) == SHAPE  # H % 256
    assert _ffn(L, I=96) == SHAPE  # I % 128
    assert _ffn(L, k=9, E=8) == SHAPE
    assert _ffn(L, E=300, k=8) == SHAPE
    assert _ffn(L, T=-2) == SHAPE
    assert _ffn(L, ws=None) == WORKSPACE
    assert _ffn(L, wsb=16) == WORKSPACE
    assert _ffn(L, xc=ctypes.c_void_p(0x10008)) == ALIGN
    assert _ffn(L, po=ctypes.c_void_p(0x10004)) == ALIGN
    assert _ffn(L, ps=ctypes.c_void_p(0x10002)) == ALIGN
    assert _ffn(L, ps=ctypes.c_void_p(0x10004)) == _ffn(L)  # 4-byte alignment is enough for pair_scale
    assert L.moe_nvfp4_grouped_ffn(P, ctypes.c_void_p(0x10004), P, 16, 256, P, P, P, P, P, P, P, 8, 128, 2, P, P, P,
                                   P, P, None, P2, 1 << 30, None) == ALIGN  # x_scales 16-byte aligned
    assert _ffn(L, ws=ctypes.c_void_p(0x10010)) == ALIGN
    assert _ffn(L, T=0) == OK  # no pairs: no-op


def test_ffn_rejects_shapes_past_32bit_offsets(L):
    """The expert kernels address x codes (T*H/2 bytes), h codes (T*k*I/2 bytes) and one
    expert's w13 codes (I*H bytes) with 32-bit offsets, and launch one grid row per m-tile:
    shapes past those limits are rejected before anything is enqueued."""
    big = 1 << 62
    # largest legal x: T*H/2 just under 4 GiB at H = 6144 (k = 1 keeps h small)
    t_max = ((1 << 32) - 1) // 3072
    # (a legal shape stops at the missing workspace, checked after the shape: nothing is launched)
    assert _ffn(L, T=t_max, H=6144, I=128, k=1, E=8, ws=None) == WORKSPACE
    assert _ffn(L, T=t_max + 1, H=6144, I=128, k=1, E=8, wsb=big) == SHAPE
    assert b"x codes" in L.moe_last_error()
    # h codes: T*k*I/2 at I = 2048, k = 8 reaches 4 GiB at T*k = 4,194,304
    assert _ffn(L, T=524287, H=256, I=2048, k=8, E=80, ws=None) == WORKSPACE
    assert _ffn(L, T=524288, H=256, I=2048, k=8, E=80, wsb=big) == SHAPE
    assert b"h codes" in L.moe_last_error()
    # one expert's w13 codes: I*H bytes
    assert _ffn(L, T=16, H=65536, I=65536, k=2, E=8, wsb=big) == SHAPE
    g = L.moe_nvfp4_gate_up_swiglu
    assert g(P, P, P, t_max + 1, 6144, P, P, P, P, 8, 128, 1, P, P, P, P, P2, big, None) == SHAPE
    d = L.moe_nvfp4_down_scatter
    assert d(P, P, P, 524288, 256, P, P, P, 80, 2048, 8, P, P, P, P, P, None, P2, big, None) == SHAPE


def test_noalloc_ffn_validation(L):
    """The static-scratch FFN: same checks as the workspace call, and shapes whose workspace
    exceeds the static scratch are rejected before anything is enqueued."""
    f = L.moe_nvfp4_grouped_ffn_noalloc

    def call(T=16, H=256, E=8, I=128, k=2, xc=P, po=P):
        return f(xc, P, P, T, H, P, P, P, P, P, P, P, E, I, k, P, P, P, po, P, None, None)

    assert call(xc=None) == NULL
    assert call(H=200) == SHAPE
    assert call(xc=ctypes.c_void_p(0x10008)) == ALIGN
    assert call(T=0) == OK
    scratch = 32 << 20
    assert L.moe_ffn_workspace_bytes(8192, 8, 80, 6144, 2048) > scratch
    assert call(T=8192, H=6144, E=80, I=2048, k=8) == SHAPE
    assert b"static scratch" in L.moe_last_error()


def test_ffn_workspace_queries(L):
    full = L.moe_ffn_workspace_bytes(8192, 8, 80, 6144, 2048)
    stage = L.moe_ffn_stage_workspace_bytes(8192, 8, 80, 6144, 2048)
    h_bytes = 8192 * 8 * (2048 // 2 + 2048 // 16)
    assert full >= stage + h_bytes
    assert full % 256 == 0 and stage % 256 == 0
    assert L.moe_ffn_workspace_bytes(-1, 8, 80, 6144, 2048) == 0
    assert L.moe_route_workspace_bytes(16, 6144, 80, 8) > 0


def test_stage_validation(L):
    g = L.moe_nvfp4_gate_up_swiglu
    assert g(P, P, P, 16, 256, P, P, P, P, 8, 128, 2, P, P, None, P, P2, 1 << 30, None) == NULL
    assert g(P, P, P, 16, 100, P, P, P, P, 8, 128, 2, P, P, P, P, P2, 1 << 30, None) == SHAPE
    d = L.moe_nvfp4_down_scatter
    assert d(P, P, P, 16, 256, P, P, P, 8, 128, 2, P, P, None, P, P, None, P2, 1 << 30, None) == NULL
    assert d(P, P, P, 16, 256, P, P, P, 8, 128, 2, P, P, P, P, None, None, P2, 1 << 30, None) == NULL  # pair_scale
    assert d(P, P, P, 16, 256, P, P, P, 8, 128, 2, P, P, P, P, P, None, None, 0, None) == WORKSPACE


def test_combine_and_reap_validation(L):
    c = L.moe_combine
    assert c(None, P, 4, 2, 64, 0, P, None) == NULL
    assert c(P, None, 4, 2, 64, 0, P, None) == NULL
    assert c(P, P, 4, 2, 66, 0, P, None) == SHAPE
    assert c(P, P, 4, 2, 68, 0, P, None) == SHAPE  # H % 8: eight FP16 columns per 16-byte load
    assert c(P, P, 4, 2, 64, 2, P, None) == SHAPE
    assert c(P, P, 4, 0, 64, 0, P, None) == SHAPE
    assert c(P, P, 4, 2, 64, 0, ctypes.c_void_p(0x10004), None) == ALIGN
    assert c(ctypes.c_void_p(0x10008), P, 4, 2, 64, 0, P, None) == ALIGN
    assert c(P, ctypes.c_void_p(0x10002), 4, 2, 64, 0, P, None) == ALIGN
    assert c(P, 0, 0, 2, 64, 0, P, None) == OK
    r = L.reap_saliency
    assert r(P, P, P, None, 4, 2, 8, P, None) == NULL
    assert r(P, P, P, P, 4, 2, 0, P, None) == SHAPE
    assert r(P, P, P, P, 4, 2, 300, P, None) == SHAPE


def test_prune_validation(L):
    s = L.reap_prune_select
    assert s(P, 128, 80, None, None) == NULL
    assert s(None, 128, 80, P, None) == NULL
    assert s(P, 128, 0, P, None) == SHAPE
    assert s(P, 128, 129, P, None) == SHAPE
    assert s(P, 300, 80, P, None) == SHAPE
    assert s(P, 128, 80, ctypes.c_void_p(0x10002), None) == ALIGN
    g = L.moe_gather_experts
    assert g(None, 128, 64, P, 80, P2, None) == NULL
    assert g(P, 128, 64, None, 80, P2, None) == NULL
    assert g(P, 0, 64, P, 80, P2, None) == SHAPE
    assert g(P, 128, 0, P, 80, P2, None) == SHAPE
    assert g(P, 128, 64, P, 0, P2, None) == SHAPE
    assert g(P, 128, 64, P, 70000, P2, None) == SHAPE
    assert g(P, 1 << 40, 1 << 40, P, 80, P2, None) == SHAPE  # size overflows
    assert g(P, 128, 64, ctypes.c_void_p(0x30002), 80, P2, None) == ALIGN
    # src [0x10000, 0x12000) overlaps dst [0x11000, ...)
    assert g(P, 128, 64, ctypes.c_void_p(0x40000), 80, ctypes.c_void_p(0x11000), None) == SHAPE
    assert "overlap" in L.moe_last_error().decode()


def test_shared_and_rotation_validation(L):
    g = L.moe_shared_gate_up
    assert g(P, 4, 250, 256, P, 128, P, P, 1 << 20, None) == SHAPE  # H % 256
    assert g(P, 4, 256, 256, P, 100, P, P, 1 << 20, None) == SHAPE  # I % 128
    assert g(P, 4, 256, 250, P, 128, P, P, 1 << 20, None) == SHAPE  # ldx < H
    assert g(None, 4, 256, 256, P, 128, P, P, 1 << 20, None) == NULL
    assert g(ctypes.c_void_p(0x10008), 4, 256, 256, P, 128, P, P, 1 << 20, None) == ALIGN
    assert g(P, 4, 256, 256, P, 128, P, None, 0, None) == WORKSPACE  # T <= 16 needs the partial sums
    assert g(P, 0, 256, 256, P, 128, P, None, 0, None) == OK
    assert L.moe_shared_workspace_bytes(4, 256, 128) >= 4 * 128 * 2 and L.moe_shared_workspace_bytes(-1, 256, 128) == 0
    d = L.moe_shared_down
    assert d(P, 4, 128, P, 256, None, P, 1 << 20, None) == NULL
    assert d(P, 4, 128, P, 256, ctypes.c_void_p(0x10004), P, 1 << 20, None) == ALIGN
    e = L.moe_shared_expert
    assert e(P, 4, 256, 256, P, P, 128, P, P, 16, None) == WORKSPACE
    c = L.moe_combine_block
    assert c(P, P, None, 4, 2, 64, 0, P, None) == NULL
    assert c(P, None, P, 4, 2, 64, 0, P, None) == NULL
    assert c(P, P, P, 4, 2, 66, 0, P, None) == SHAPE
    assert c(P, ctypes.c_void_p(0x10002), P, 4, 2, 64, 0, P, None) == ALIGN
    r = L.hadamard_rotate_bf16
    assert r(P, 4, 256, 256, None, 48, P2, 256, None) == SHAPE  # block not a power of two
    assert r(P, 4, 256, 256, None, 512, P2, 256, None) == SHAPE  # block > cols
    assert r(P, 4, 260, 264, None, 4, P2, 264, None) == SHAPE  # cols % 8
    assert r(P, 4, 32768, 32768, None, 2, P2, 32768, None) == SHAPE  # cols above the LDS row limit
    assert r(P, 4, 256, 256, None, 16, None, 256, None) == NULL
    assert r(P, 4, 256, 256, None, 16, ctypes.c_void_p(0x20008), 256, None) == ALIGN
    assert r(P, 4, 256, 256, None, 16, ctypes.c_void_p(0x10100), 256, None) == SHAPE  # partial overlap
    assert r(P, 0, 256, 256, None, 16, P2, 256, None) == OK


def test_combine_reap_validation(L):
    f = L.moe_combine_reap
    assert f(P, P, 4, 2, 66, 0, P, P, P, P, P, 8, P, None) == SHAPE
    assert f(P, P, 4, 2, 64, 0, P, P, P, P, P, 0, P, None) == SHAPE
    assert f(P, P, 4, 2, 64, 0, P, None, P, P, P, 8, P, None) == NULL
    assert f(P, None, 4, 2, 64, 0, P, P, P, P, P, 8, P, None) == NULL
    assert f(P, P, 4, 2, 64, 0, ctypes.c_void_p(0x10004), P, P, P, P, 8, P, None) == ALIGN
    assert f(P, ctypes.c_void_p(0x10002), 4, 2, 64, 0, P, P, P, P, P, 8, P, None) == ALIGN


def test_prepack_validation(L):
    for fn in (L.moe_nvfp4_prepack_weights, L.moe_nvfp4_unpack_weights):
        assert fn(P, P, 2, 24, 256, 1, P2, ctypes.c_void_p(0x30000), None) == SHAPE  # N % 16
        assert fn(P, P, 2, 32, 200, 1, P2, ctypes.c_void_p(0x30000), None) == SHAPE  # K % 128
        assert fn(P, P, 2, 32, 256, 2, P2, ctypes.c_void_p(0x30000), None) == SHAPE  # kind
        assert fn(P, None, 2, 32, 256, 1, P2, ctypes.c_void_p(0x30000), None) == NULL
        assert fn(P, ctypes.c_void_p(0x10004), 2, 32, 256, 1, P2, ctypes.c_void_p(0x30000), None) == ALIGN
        assert fn(P, P, 2, 32, 256, 1, P2, ctypes.c_void_p(0x10008), None) == SHAPE  # scale arrays overlap
        assert fn(P, P, 0, 32, 256, 1, P2, ctypes.c_void_p(0x30000), None) == OK


def test_missing_library_fails_loudly(tmp_path):
    from nvfp4_w4a4_mixture_amd import _lib

    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "nope.so"))


def test_tiled_weight_scale_layout():
    """The tests' untiling helper follows the header's byte formula for tiled weight scales."""
    import sys
    import numpy as np

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_cases import untile_weight_scales

    R, K = 48, 384
    nb = K // 16
    flat = np.arange(R * nb, dtype=np.int64)  # flat[i] = storage byte index i
    tiled = flat.reshape(R // 16, K // 128, 16, 8)
    rm = untile_weight_scales(tiled)  # rm[r, b] = storage index of scale (r, b)
    for r in range(R):
        for b in range(nb):
            assert rm[r, b] == (r // 16) * K + (b // 8) * 128 + (r % 16) * 8 + b % 8
