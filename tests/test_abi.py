"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and host-side validation returns the documented status
codes (with a message) before any HIP call."""

import ctypes
import os
import re

import pytest

import block_scaled_fp4_topk_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moefp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)) - {"if", "while"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libmoefp4.so is not built (python -m block_scaled_fp4_topk_amd.build)")
    return m.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"moe_fp4_forward", "moe_fp4_forward_fused", "moe_fp4_route", "fp4_requant_gran_k", "moe_fp4_workspace_bytes",
            "moe_fp4_quantize_act", "moe_fp4_quantize_act_fp4", "moe_fp4_prepare_gemm_weights",
            "moefp4_last_error", "moefp4_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.moefp4_version()


def test_binding_exports():
    """Every name the binding lists exists, and each C entry point for users
    has its Python wrapper (no GPU needed)."""
    for n in m.__all__:
        assert hasattr(m, n), n
    for n in ("forward", "route", "requant_gran_k", "prepare_gemm_weights", "quantize_act",
              "quantize_act_fp4", "workspace_bytes", "dropped_assignments"):
        assert callable(getattr(m, n)), n


def P(**kw):
    d = dict(T=64, E=256, top_k=8, H=6144, I=2048, gran_k=16, act_fmt=0, w13_order=0, out_fmt=0, w_layout=0)
    d.update(kw)
    return m.Problem(**d)


def ws_status(p):
    n = ctypes.c_size_t(0)
    return m.lib().moe_fp4_workspace_bytes(ctypes.byref(p), ctypes.byref(n)), n.value


def test_workspace_sizes(L):
    st, n = ws_status(P())
    assert st == 0 and n > 512 * 6144 * 4  # holds the f32 FC2 rows
    st8, n8 = ws_status(P(T=8192, gran_k=32, act_fmt=1))
    assert st8 == 0 and n8 > 65536 * 6144 * 4
    # A4 with the library quantising x: x codes T*H/2 and h codes A*I/2 fit
    st4, n4 = ws_status(P(T=8192, gran_k=32, act_fmt=4))
    assert st4 == 0 and n4 > 65536 * 6144 * 4 + 8192 * 6144 // 2 + 65536 * 2048 // 2


@pytest.mark.parametrize("kw,status", [
    (dict(gran_k=8), m.EINVAL),
    (dict(top_k=0), m.EINVAL),
    (dict(top_k=300), m.EINVAL),
    (dict(E=0), m.EINVAL),
    (dict(E=4096, top_k=8), m.EUNSUPPORTED),
    (dict(H=6000), m.EINVAL),
    (dict(I=2000), m.EINVAL),
    (dict(I=2080), m.EUNSUPPORTED),
    (dict(act_fmt=1, gran_k=16), m.EUNSUPPORTED),
    (dict(act_fmt=2, gran_k=16), m.EUNSUPPORTED),
    (dict(act_fmt=3, gran_k=16), m.EUNSUPPORTED),
    (dict(act_fmt=4, gran_k=16), m.EUNSUPPORTED),
    (dict(act_fmt=3, gran_k=32, H=6400), m.EUNSUPPORTED),   # FP4 x: H % 512
    (dict(act_fmt=4, gran_k=32, I=2304), m.EUNSUPPORTED),   # FP4 x: I % 512
    (dict(act_fmt=7), m.EINVAL),
    (dict(w13_order=3), m.EINVAL),
    (dict(out_fmt=2), m.EINVAL),
    (dict(T=-1), m.EINVAL),
    (dict(w_layout=2), m.EINVAL),
    # GEMM-layout weights: only where the prefill GEMM runs
    (dict(w_layout=1), m.EUNSUPPORTED),                                   # bf16 decode
    (dict(w_layout=1, gran_k=32, act_fmt=1), m.EUNSUPPORTED),             # FP8 decode (16-row tiles)
    (dict(w_layout=1, gran_k=32, act_fmt=1, T=8192, I=2304), m.EUNSUPPORTED),  # 64-row tiles
    # the 16-row decode tiles address an expert's weights and the fp16 rows
    # of x with 32-bit offsets
    (dict(H=65536, I=32768), m.EUNSUPPORTED),                             # I*H = 2^31
    (dict(T=8192, top_k=1, E=512, H=262144, I=256), m.EUNSUPPORTED),      # T*H = 2^31 (group16, bf16 x)
])
def test_problem_validation(L, kw, status):
    st, _ = ws_status(P(**kw))
    assert st == status
    assert len(L.moefp4_last_error()) > 0


def test_forward_rejects_before_launch(L):
    p = P()
    z = ctypes.c_void_p(0)
    # NULL tensors
    st = L.moe_fp4_forward(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z, z, 0, z)
    assert st == m.EINVAL and b"non-NULL" in L.moefp4_last_error()
    # fake (never dereferenced) aligned pointers, missing workspace
    f = ctypes.c_void_p(1 << 20)
    st = L.moe_fp4_forward(ctypes.byref(p), f, z, f, f, f, f, z, f, f, z, f, z, 0, z)
    assert st == m.EWORKSPACE
    # x_sf given for bf16 activations
    st = L.moe_fp4_forward(ctypes.byref(p), f, f, f, f, f, f, z, f, f, z, f, f, 1 << 40, z)
    assert st == m.EINVAL and b"x_sf" in L.moefp4_last_error()
    # T = 0 is a valid empty call
    p0 = P(T=0)
    assert L.moe_fp4_forward(ctypes.byref(p0), z, z, z, z, z, z, z, z, z, z, z, z, 0, z) == 0


def test_forward_fused_rejects_before_launch(L):
    """The single-launch forward validates like moe_fp4_forward and refuses
    problems that do not run on the 16-row decode tiles, before any launch."""
    z = ctypes.c_void_p(0)
    f = ctypes.c_void_p(1 << 20)
    p = P()
    st = L.moe_fp4_forward_fused(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z, z, 0, z)
    assert st == m.EINVAL and b"non-NULL" in L.moefp4_last_error()
    st = L.moe_fp4_forward_fused(ctypes.byref(p), f, z, f, f, f, f, z, f, f, z, f, z, 0, z)
    assert st == m.EWORKSPACE
    # prefill-shaped (64 assignments per expert on 128-row GEMM tiles): refused
    pp = P(T=8192, top_k=8, E=256, gran_k=32, act_fmt=m.ACT_FP8_UE8M0_K32)
    st = L.moe_fp4_forward_fused(ctypes.byref(pp), f, f, f, f, f, f, z, f, f, z, f, f, 1 << 40, z)
    assert st == m.EUNSUPPORTED and b"decode tiles" in L.moefp4_last_error()
    p0 = P(T=0)
    assert L.moe_fp4_forward_fused(ctypes.byref(p0), z, z, z, z, z, z, z, z, z, z, z, z, 0, z) == 0


def test_requant_rejects_before_launch(L):
    z = ctypes.c_void_p(0)
    f = ctypes.c_void_p(1 << 20)
    g = ctypes.c_void_p(1 << 30)
    rq = L.fp4_requant_gran_k
    assert rq(2, 4, 64, f, g, 32, z, f, g, 16, z) == m.EUNSUPPORTED
    assert rq(2, 4, 64, f, g, 16, z, f, g, 64, z) == m.EINVAL
    assert rq(2, 4, 48, f, g, 16, z, f, g, 32, z) == m.EINVAL            # K % 32
    assert rq(2, 4, 64, z, g, 16, z, f, g, 32, z) == m.EINVAL            # NULL src
    assert rq(2, 4, 64, f, f, 16, z, ctypes.c_void_p(1 << 24), g, 32, z) == m.EINVAL  # src_sf overlaps src
    assert rq(0, 4, 64, z, z, 16, z, z, z, 32, z) == 0                   # empty
    assert rq(2, 4, 64, ctypes.c_void_p((1 << 20) + 8), g, 16, z, f, ctypes.c_void_p(1 << 31), 32, z) == m.EINVAL


def test_quantize_act_rejects_before_launch(L):
    z = ctypes.c_void_p(0)
    f = ctypes.c_void_p(1 << 20)
    g = ctypes.c_void_p(1 << 30)
    q = L.moe_fp4_quantize_act
    assert q(4, 48, f, g, f, z) == m.EINVAL                       # H % 32
    assert q(4, 0, f, g, f, z) == m.EINVAL
    assert q(-1, 64, f, g, f, z) == m.EINVAL
    assert q(4, 64, z, g, f, z) == m.EINVAL                       # NULL x
    assert q(4, 64, ctypes.c_void_p((1 << 20) + 8), g, f, z) == m.EINVAL  # misaligned x
    assert q(0, 64, z, z, z, z) == 0                              # empty


def test_quantize_act_fp4_rejects_before_launch(L):
    z = ctypes.c_void_p(0)
    f = ctypes.c_void_p(1 << 20)
    g = ctypes.c_void_p(1 << 30)
    q = L.moe_fp4_quantize_act_fp4
    assert q(4, 48, f, g, f, z) == m.EINVAL                       # H % 32
    assert q(4, 64, f, z, f, z) == m.EINVAL                       # NULL x_fp4
    assert q(4, 64, f, ctypes.c_void_p((1 << 30) + 4), f, z) == m.EINVAL  # misaligned x_fp4
    assert q(0, 64, z, z, z, z) == 0                              # empty


def test_forward_a4_needs_x_sf(L):
    p = P(gran_k=32, act_fmt=3)
    f = ctypes.c_void_p(1 << 20)
    z = ctypes.c_void_p(0)
    st = L.moe_fp4_forward(ctypes.byref(p), f, z, f, f, f, f, z, f, f, z, f, f, 1 << 40, z)
    assert st == m.EINVAL and b"x_sf" in L.moefp4_last_error()


def test_forward_quant_x_rejects_x_sf(L):
    p = P(gran_k=32, act_fmt=2)
    f = ctypes.c_void_p(1 << 20)
    z = ctypes.c_void_p(0)
    st = L.moe_fp4_forward(ctypes.byref(p), f, f, f, f, f, f, z, f, f, z, f, f, 1 << 40, z)
    assert st == m.EINVAL and b"x_sf" in L.moefp4_last_error()


def test_gemm_layout_problem_accepted(L):
    st, n = ws_status(P(T=8192, gran_k=32, act_fmt=1, w_layout=1))
    assert st == 0 and n > 0
    st, n = ws_status(P(T=8192, gran_k=32, act_fmt=4, w_layout=1))
    assert st == 0 and n > 0


def test_prepare_gemm_rejects_before_launch(L):
    z = ctypes.c_void_p(0)
    f = ctypes.c_void_p(1 << 20)
    g = ctypes.c_void_p(1 << 32)
    h = ctypes.c_void_p(1 << 34)
    k = ctypes.c_void_p(1 << 36)
    pg = L.moe_fp4_prepare_gemm_weights
    assert pg(2, 1024, 512, 0, 0, z, z, z, z, z) == m.EINVAL             # NULL
    assert pg(2, 1000, 512, 0, 0, f, g, h, k, z) == m.EINVAL             # N % 512
    assert pg(2, 1024, 640, 1, 0, f, g, h, k, z) == m.EINVAL             # K % 512
    assert pg(2, 1024, 512, 2, 0, f, g, h, k, z) == m.EINVAL             # which
    assert pg(2, 1024, 512, 0, 5, f, g, h, k, z) == m.EINVAL             # order
    assert pg(2, 1024, 512, 0, 0, f, g, f, k, z) == m.EINVAL             # dst overlaps src
    assert pg(2, 1024, 512, 0, 0, ctypes.c_void_p((1 << 20) + 4), g, h, k, z) == m.EINVAL  # alignment
    assert pg(0, 1024, 512, 0, 0, z, z, z, z, z) == 0                    # empty
    assert len(L.moefp4_last_error()) == 0


def test_measurement_helpers_validate_before_launch(L):
    """The profiling hooks refuse bad arguments with a message and launch
    nothing: the MFMA rate probe needs a sink and at least one iteration and
    workgroup; the stage-event hook needs six events (NULL switches it off)."""
    z = ctypes.c_void_p(0)
    flops = ctypes.c_double(0.0)
    probe = L.moefp4_mfma_peak_probe
    assert probe(0, 0, 1, ctypes.c_void_p(1 << 20), ctypes.byref(flops), z) == m.EINVAL
    assert probe(0, 1, 0, ctypes.c_void_p(1 << 20), ctypes.byref(flops), z) == m.EINVAL
    assert probe(0, 1, 1, z, ctypes.byref(flops), z) == m.EINVAL
    assert b"sink" in L.moefp4_last_error()
    assert probe(1, 1, 1, ctypes.c_void_p(1 << 20), None, z) == m.EINVAL
    events = (ctypes.c_void_p * 6)()
    assert L.moefp4_set_stage_events(events, 5) == m.EINVAL
    assert b"6" in L.moefp4_last_error()
    assert L.moefp4_set_stage_events(None, 0) == 0
