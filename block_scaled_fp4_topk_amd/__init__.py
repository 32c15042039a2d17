"""block_scaled_fp4_topk_amd -- Python binding of libmoefp4 (MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in ``include/moefp4.h``:
every step of the MoE forward and of the requantisation runs in the HIP
kernels of the library.  PyTorch only provides device memory and the current
stream.  There is no CPU fallback: if ``libmoefp4.so`` is missing or no GPU is
present the calls raise.

Functions mirror the C entry points:
  workspace_bytes(problem)            -> moe_fp4_workspace_bytes
  workspace_offsets(problem)          -> moe_fp4_workspace_offsets
  route(problem, topk_ids, ...)       -> moe_fp4_route
  forward(x, topk_ids, topk_w, ...)   -> moe_fp4_forward (fused=True: moe_fp4_forward_fused)
  forward_static(x, topk_ids, ...)    -> moe_fp4_forward_static (no workspace)
  requant_gran_k(src, src_sf, ...)    -> fp4_requant_gran_k
  prepare_gemm_weights(src, src_sf, ...) -> moe_fp4_prepare_gemm_weights
  prepare_gemm_weights_g16(src, src_sf, src_gs, ...) -> moe_fp4_prepare_gemm_weights_g16
  quantize_act(x, ...)                -> moe_fp4_quantize_act
  quantize_act_fp4(x, ...)            -> moe_fp4_quantize_act_fp4
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["Problem", "MoeFp4Error", "lib", "workspace_bytes", "workspace_offsets", "route", "forward",
           "forward_problem", "forward_static",
           "requant_gran_k", "prepare_gemm_weights", "prepare_gemm_weights_g16", "quantize_act", "quantize_act_fp4",
           "dropped_assignments", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoefp4.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)
ACT_BF16, ACT_FP8_UE8M0_K32, ACT_BF16_QUANT_FP8_K32, ACT_FP4_UE8M0_K32, ACT_BF16_QUANT_FP4_K32 = range(5)
GATE_UP, UP_GATE = 0, 1


OUT_BF16, OUT_F32 = 0, 1
W_RAW, W_GEMM = 0, 1


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "E", "top_k", "H", "I", "gran_k", "act_fmt", "w13_order", "out_fmt", "w_layout")]


class MoeFp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moefp4 status {status}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p


def lib():
    """Load libmoefp4.so (built in-tree by ``python -m block_scaled_fp4_topk_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m block_scaled_fp4_topk_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        L.moe_fp4_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_fp4_workspace_bytes.restype = st
        L.moe_fp4_workspace_offsets.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_fp4_workspace_offsets.restype = st
        L.moe_fp4_route.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_fp4_route.restype = st
        L.moe_fp4_forward.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, ctypes.c_size_t, _P]
        L.moe_fp4_forward.restype = st
        L.moe_fp4_forward_fused.argtypes = L.moe_fp4_forward.argtypes
        L.moe_fp4_forward_fused.restype = st
        L.moe_fp4_forward_static.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P]
        L.moe_fp4_forward_static.restype = st
        L.fp4_requant_gran_k.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                         ctypes.c_int32, _P, _P, _P, ctypes.c_int32, _P]
        L.fp4_requant_gran_k.restype = st
        L.moe_fp4_prepare_gemm_weights.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P]
        L.moe_fp4_prepare_gemm_weights.restype = st
        L.moe_fp4_prepare_gemm_weights_g16.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P]
        L.moe_fp4_prepare_gemm_weights_g16.restype = st
        L.moe_fp4_quantize_act.argtypes = [ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P]
        L.moe_fp4_quantize_act.restype = st
        L.moe_fp4_quantize_act_fp4.argtypes = [ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P]
        L.moe_fp4_quantize_act_fp4.restype = st
        L.moefp4_last_error.argtypes = []
        L.moefp4_last_error.restype = ctypes.c_char_p
        L.moefp4_mfma_peak_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                             ctypes.POINTER(ctypes.c_double), _P]
        L.moefp4_mfma_peak_probe.restype = st
        L.moefp4_set_stage_events.argtypes = [_P, ctypes.c_int32]
        L.moefp4_set_stage_events.restype = st
        L.moefp4_version.argtypes = []
        L.moefp4_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise MoeFp4Error(status, lib().moefp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtypes):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _order(w13_order):
    if isinstance(w13_order, str):
        return {"gate_up": GATE_UP, "w31": GATE_UP, "up_gate": UP_GATE, "w13": UP_GATE}[w13_order]
    return w13_order


def make_problem(T, E, top_k, H, I, gran_k, act_fmt=ACT_BF16, w13_order=GATE_UP,
                 out_fmt=OUT_BF16, w_layout=W_RAW) -> Problem:
    if isinstance(w_layout, str):
        w_layout = {"raw": W_RAW, "gemm": W_GEMM}[w_layout]
    return Problem(T, E, top_k, H, I, gran_k, act_fmt, _order(w13_order), out_fmt, w_layout)


def workspace_bytes(problem: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_fp4_workspace_bytes(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def workspace_offsets(problem: Problem):
    """(h, h_sf, slot_of) byte offsets of the forward's intermediate h, its
    UE8M0 scales (0 if none) and the assignment -> slot map in the workspace
    (moe_fp4_workspace_offsets)."""
    h, hs, so = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().moe_fp4_workspace_offsets(ctypes.byref(problem), ctypes.byref(h), ctypes.byref(hs),
                                           ctypes.byref(so)))
    return h.value, hs.value, so.value


def _workspace(problem, workspace, device):
    import torch
    need = workspace_bytes(problem)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def route(problem: Problem, topk_ids, workspace=None, stream=None):
    """Returns (counts [E], offsets [E+1], sorted_assign [T*k], slot_of [T*k]) int32 tensors."""
    import torch
    _dev(topk_ids, "topk_ids", (torch.int32,))
    dev = topk_ids.device
    A = problem.T * problem.top_k
    counts = torch.empty(problem.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(problem.E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    so = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    ws = _workspace(problem, workspace, dev)
    _check(lib().moe_fp4_route(ctypes.byref(problem), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                               _ptr(sa), _ptr(so), _ptr(ws), ws.numel(), _stream(stream)))
    return counts, offsets, sa[:A], so[:A]


def forward_problem(x, topk_ids, w13, w2, gran_k, x_sf=None, w13_order="gate_up", out_dtype=None,
                    quantize_x=False, w_layout="raw") -> Problem:
    """The problem descriptor forward() passes to moe_fp4_forward for these
    arguments (shapes from the tensors, the activation format from x / x_sf
    / quantize_x)."""
    import torch
    quant = {False: None, None: None, True: "fp8", "fp8": "fp8", "fp4": "fp4"}.get(quantize_x, "?")
    if quant == "?":
        raise ValueError(f"quantize_x must be False, True, 'fp8' or 'fp4', got {quantize_x!r}")
    a8 = x_sf is not None
    E, two_i, _ = w13.shape
    H = w2.shape[1]
    T, xcols = x.shape
    a4 = a8 and xcols * 2 == H
    if xcols != H and not a4:
        raise ValueError(f"x has {xcols} columns; expected H={H} (or H/2 packed FP4 codes with x_sf)")
    k = topk_ids.shape[1]
    if out_dtype is None:
        out_dtype = torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if quant and a8:
        raise ValueError("quantize_x takes bfloat16 x without x_sf")
    act = (ACT_FP4_UE8M0_K32 if a4 else ACT_FP8_UE8M0_K32 if a8 else
           ACT_BF16_QUANT_FP8_K32 if quant == "fp8" else ACT_BF16_QUANT_FP4_K32 if quant == "fp4" else ACT_BF16)
    return make_problem(T, E, k, H, two_i // 2, gran_k, act, w13_order,
                        OUT_F32 if out_dtype == torch.float32 else OUT_BF16, w_layout)


def forward(x, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs, gran_k, x_sf=None,
            w13_order="gate_up", out=None, workspace=None, stream=None, out_dtype=None,
            quantize_x=False, w_layout="raw", fused=False):
    """MoE forward on the GPU.  x: [T, H] bfloat16 (A16); uint8/float8_e4m3fn
    [T, H] with x_sf [T, H/32] uint8 (A8); or uint8 [T, H/2] (two E2M1 codes
    per byte) with x_sf (A4).  quantize_x with bfloat16 x asks the library to
    quantise x first: True or "fp8" -> the A8 format (act_fmt
    BF16_QUANT_FP8_K32), "fp4" -> the A4 format (BF16_QUANT_FP4_K32).
    Weights uint8 as in include/moefp4.h; w_layout="gemm" for weights from
    prepare_gemm_weights.  fused=True runs FC1 and FC2 in one persistent
    launch (moe_fp4_forward_fused; 16-row decode tiles only, same result).
    Returns out [T, H] bfloat16 (default) or float32 (out_dtype=torch.float32)."""
    import torch
    u8 = (torch.uint8,)
    fp8 = (torch.uint8, torch.float8_e4m3fn)
    a8 = x_sf is not None
    _dev(x, "x", fp8 if a8 else (torch.bfloat16, torch.int16, torch.uint16))
    _dev(x_sf, "x_sf", u8)
    _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,))
    for n, t in (("w13", w13), ("w13_sf", w13_sf), ("w2", w2), ("w2_sf", w2_sf)):
        _dev(t, n, u8)
    _dev(w13_gs, "w13_gs", (torch.float32,))
    _dev(w2_gs, "w2_gs", (torch.float32,))
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    p = forward_problem(x, topk_ids, w13, w2, gran_k, x_sf, w13_order, out_dtype, quantize_x, w_layout)
    if out is None:
        out = torch.empty((p.T, p.H), dtype=out_dtype, device=x.device)
    _dev(out, "out", (out_dtype,))
    ws = _workspace(p, workspace, x.device)
    fn = lib().moe_fp4_forward_fused if fused else lib().moe_fp4_forward
    _check(fn(ctypes.byref(p), _ptr(x), _ptr(x_sf), _ptr(topk_ids), _ptr(topk_w), _ptr(w13), _ptr(w13_sf),
              _ptr(w13_gs), _ptr(w2), _ptr(w2_sf), _ptr(w2_gs), _ptr(out), _ptr(ws), ws.numel(),
              _stream(stream)))
    return out


def forward_static(x, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs, gran_k, x_sf=None,
                   w13_order="gate_up", out=None, stream=None, out_dtype=None, quantize_x=False, w_layout="raw"):
    """forward() without a workspace: moe_fp4_forward_static, whose
    workspace is the library's static device scratch (64 MiB per GPU; larger
    problems raise with status EWORKSPACE).  Calls that overlap on one GPU
    race; calls on one stream are ordered."""
    import torch
    u8 = (torch.uint8,)
    a8 = x_sf is not None
    _dev(x, "x", (torch.uint8, torch.float8_e4m3fn) if a8 else (torch.bfloat16, torch.int16, torch.uint16))
    _dev(x_sf, "x_sf", u8)
    _dev(topk_ids, "topk_ids", (torch.int32,))
    _dev(topk_w, "topk_w", (torch.float32,))
    for n, t in (("w13", w13), ("w13_sf", w13_sf), ("w2", w2), ("w2_sf", w2_sf)):
        _dev(t, n, u8)
    _dev(w13_gs, "w13_gs", (torch.float32,))
    _dev(w2_gs, "w2_gs", (torch.float32,))
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    p = forward_problem(x, topk_ids, w13, w2, gran_k, x_sf, w13_order, out_dtype, quantize_x, w_layout)
    if out is None:
        out = torch.empty((p.T, p.H), dtype=out_dtype, device=x.device)
    _dev(out, "out", (out_dtype,))
    _check(lib().moe_fp4_forward_static(ctypes.byref(p), _ptr(x), _ptr(x_sf), _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(w13), _ptr(w13_sf), _ptr(w13_gs), _ptr(w2), _ptr(w2_sf),
                                        _ptr(w2_gs), _ptr(out), _stream(stream)))
    return out


def requant_gran_k(src, src_sf, src_gs=None, src_gran=16, dst_gran=32, dst=None, dst_sf=None,
                   stream=None):
    """Group16 -> group32 requantisation.  src [E, N, K/2] uint8, src_sf
    [E, N, K/16] uint8 (E4M3), src_gs [E] float32 or None.  Returns
    (dst [E, N, K/2], dst_sf [E, N, K/32]); dst may be src (in place)."""
    import torch
    _dev(src, "src", (torch.uint8,))
    _dev(src_sf, "src_sf", (torch.uint8,))
    _dev(src_gs, "src_gs", (torch.float32,))
    E, N, kh = src.shape
    K = 2 * kh
    if dst is None:
        dst = torch.empty_like(src)
    if dst_sf is None:
        dst_sf = torch.empty((E, N, K // dst_gran), dtype=torch.uint8, device=src.device)
    _dev(dst, "dst", (torch.uint8,))
    _dev(dst_sf, "dst_sf", (torch.uint8,))
    _check(lib().fp4_requant_gran_k(E, N, K, _ptr(src), _ptr(src_sf), src_gran, _ptr(src_gs),
                                    _ptr(dst), _ptr(dst_sf), dst_gran, _stream(stream)))
    return dst, dst_sf




def prepare_gemm_weights(src, src_sf, which, w13_order="gate_up", dst=None, dst_sf=None, stream=None):
    """RAW group32 weights (src [E, N, K/2] uint8, src_sf [E, N, K/32] uint8)
    -> (dst, dst_sf) of the same shapes in the prefill GEMM layout
    (moe_fp4_prepare_gemm_weights).  which: "w13" (or 0) / "w2" (or 1)."""
    import torch
    _dev(src, "src", (torch.uint8,))
    _dev(src_sf, "src_sf", (torch.uint8,))
    w = {"w13": 0, "w2": 1}.get(which, which)
    E, N, kh = src.shape
    if dst is None:
        dst = torch.empty_like(src)
    if dst_sf is None:
        dst_sf = torch.empty_like(src_sf)
    _dev(dst, "dst", (torch.uint8,))
    _dev(dst_sf, "dst_sf", (torch.uint8,))
    _check(lib().moe_fp4_prepare_gemm_weights(E, N, 2 * kh, w, _order(w13_order), _ptr(src), _ptr(src_sf),
                                              _ptr(dst), _ptr(dst_sf), _stream(stream)))
    return dst, dst_sf


def prepare_gemm_weights_g16(src, src_sf, src_gs, which, w13_order="gate_up", dst=None, dst_sf=None,
                             stream=None):
    """RAW group16 weights (src [E, N, K/2] uint8, src_sf [E, N, K/16] E4M3
    bytes, src_gs [E] float32 or None) -> (dst [E, N, K/2], dst_sf [E, N,
    K/32]) in the prefill GEMM layout with group32 UE8M0 scales, the global
    scale folded in (moe_fp4_prepare_gemm_weights_g16)."""
    import torch
    _dev(src, "src", (torch.uint8,))
    _dev(src_sf, "src_sf", (torch.uint8,))
    _dev(src_gs, "src_gs", (torch.float32,))
    w = {"w13": 0, "w2": 1}.get(which, which)
    E, N, kh = src.shape
    if dst is None:
        dst = torch.empty_like(src)
    if dst_sf is None:
        dst_sf = torch.empty((E, N, 2 * kh // 32), dtype=torch.uint8, device=src.device)
    _dev(dst, "dst", (torch.uint8,))
    _dev(dst_sf, "dst_sf", (torch.uint8,))
    _check(lib().moe_fp4_prepare_gemm_weights_g16(E, N, 2 * kh, w, _order(w13_order), _ptr(src), _ptr(src_sf),
                                                  _ptr(src_gs), _ptr(dst), _ptr(dst_sf), _stream(stream)))
    return dst, dst_sf


def quantize_act_fp4(x, x_fp4=None, x_sf=None, stream=None):
    """bfloat16 [T, H] -> (E2M1 codes [T, H/2] uint8, two per byte, UE8M0
    scales [T, H/32] uint8), per 32 elements (moe_fp4_quantize_act_fp4)."""
    import torch
    _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    T, H = x.shape
    if x_fp4 is None:
        x_fp4 = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    if x_sf is None:
        x_sf = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _dev(x_fp4, "x_fp4", (torch.uint8,))
    _dev(x_sf, "x_sf", (torch.uint8,))
    _check(lib().moe_fp4_quantize_act_fp4(T, H, _ptr(x), _ptr(x_fp4), _ptr(x_sf), _stream(stream)))
    return x_fp4, x_sf


def quantize_act(x, x_fp8=None, x_sf=None, stream=None):
    """bfloat16 [T, H] -> (E4M3 codes [T, H] uint8, UE8M0 scales [T, H/32]
    uint8), per 32 elements (moe_fp4_quantize_act)."""
    import torch
    _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    T, H = x.shape
    if x_fp8 is None:
        x_fp8 = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    if x_sf is None:
        x_sf = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _dev(x_fp8, "x_fp8", (torch.uint8,))
    _dev(x_sf, "x_sf", (torch.uint8,))
    _check(lib().moe_fp4_quantize_act(T, H, _ptr(x), _ptr(x_fp8), _ptr(x_sf), _stream(stream)))
    return x_fp8, x_sf


def mfma_peak_probe(a4: bool, iters: int, blocks: int, sink, stream=None) -> float:
    """Enqueue the register-only block-scaled MFMA loop (moefp4_mfma_peak_probe);
    returns the flops it performs.  sink: float32 CUDA tensor of blocks*256."""
    import torch
    _dev(sink, "sink", (torch.float32,))
    f = ctypes.c_double(0)
    _check(lib().moefp4_mfma_peak_probe(1 if a4 else 0, iters, blocks, _ptr(sink), ctypes.byref(f), _stream(stream)))
    return f.value


def set_stage_events(events_array, n: int):
    """Profiling hook (moefp4_set_stage_events): events_array is a ctypes
    array of 6 hipEvent_t handles, or None to stop recording."""
    _check(lib().moefp4_set_stage_events(events_array, n))


def dropped_assignments(workspace) -> int:
    """Number of assignments with an expert id outside [0, E) in the last
    route / forward call that used ``workspace`` (synchronises)."""
    return int(workspace[:4].view(dtype=__import__("torch").int32).item())
