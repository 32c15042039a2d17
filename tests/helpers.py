"""Shared helpers of the GPU tests: move synthetic inputs to the device, run
the library through its C ABI, and apply the stated accuracy bound."""

import numpy as np
import torch

import block_scaled_fp4_topk_amd as moe


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (torch.cuda.is_available() is False)"


def to_dev(inp):
    d = {}
    if inp.x_sf is None:
        d["x"] = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
        d["x_sf"] = None
    else:
        d["x"] = torch.from_numpy(inp.x).cuda()
        d["x_sf"] = torch.from_numpy(inp.x_sf).cuda()
    d["topk_ids"] = torch.from_numpy(inp.topk_ids).cuda()
    d["topk_w"] = torch.from_numpy(inp.topk_w).cuda()
    for n in ("w13", "w13_sf", "w2", "w2_sf"):
        d[n] = torch.from_numpy(getattr(inp, n)).cuda()
    for n in ("w13_gs", "w2_gs"):
        v = getattr(inp, n)
        d[n] = None if v is None else torch.from_numpy(v).cuda()
    return d


def gpu_forward(inp, d, order="gate_up", **kw):
    return moe.forward(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["w13_sf"], d["w13_gs"],
                       d["w2"], d["w2_sf"], d["w2_gs"], inp.cfg.gran, x_sf=d["x_sf"],
                       w13_order=order, **kw)


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_forward(inp, d, ref, what, order="gate_up", band=None):
    """The FP32 result meets the bound; the bf16 output is exactly its RNE
    rounding (so it differs from the exact result by the bound plus half a
    bf16 ulp of the value)."""
    f32 = gpu_forward(inp, d, order, out_dtype=torch.float32)
    b16 = gpu_forward(inp, d, order)
    torch.cuda.synchronize()
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16)), \
        what + ": bf16 output is not the RNE rounding of the FP32 result"
    return check_bound(f32.cpu().numpy().astype(np.float64), ref, what, band)


def check_bound(got, ref, what="", band=None):
    """|err| <= 2e-2 * rms(ref) (+ the oracle's decision band: results that
    other equally valid near-tie roundings of h give) element-wise, and
    sum|err| / sum|ref| <= 5e-3."""
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    band = np.zeros_like(ref) if band is None else band
    excess = err - (2e-2 * rms + band)
    maxerr = float(np.max(err))
    mre = float(np.sum(err) / np.sum(np.abs(ref)))
    i = np.unravel_index(np.argmax(excess), err.shape)
    msg = (f"{what}: max|err| {maxerr:.3e} = {maxerr / rms:.4f} rms (bound 2e-2 rms = {2e-2 * rms:.3e}), "
           f"worst vs bound at {i}: err {err[i]:.3e} band {band[i]:.3e}, "
           f"elements with a nonzero band {int(np.count_nonzero(band))}/{band.size}, "
           f"mean rel {mre:.3e} (bound 5e-3)")
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert np.all(excess <= 0) and mre <= 5e-3, msg
    return maxerr / rms, mre
