"""Shared helpers of the GPU tests: move synthetic inputs to the device, run
the library through its C ABI, and apply the stated accuracy bound."""

import numpy as np
import torch

import block_scaled_fp4_topk_amd as moe
import oracle


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


def forward_ws(inp, d, order="gate_up", **kw):
    """FP32 forward with an explicit workspace: (out, workspace, problem), so
    that the quantised h it leaves there can be checked (check_h)."""
    p = moe.forward_problem(d["x"], d["topk_ids"], d["w13"], d["w2"], inp.cfg.gran, d["x_sf"], order,
                            torch.float32, kw.get("quantize_x", False), kw.get("w_layout", "raw"))
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = gpu_forward(inp, d, order, out_dtype=torch.float32, workspace=ws, **kw)
    return out, ws, p


def check_forward(inp, d, ref, what, order="gate_up", band=None, hrows=None, **kw):
    """The FP32 result meets the bound; the bf16 output is exactly its RNE
    rounding (so it differs from the exact result by the bound plus half a
    bf16 ulp of the value); with the oracle's h rows given, every quantised h
    value the forward left in its workspace equals the oracle's wherever the
    exact h is farther than the decision radius from a decision boundary."""
    f32, ws, p = forward_ws(inp, d, order, **kw)
    torch.cuda.synchronize()
    if hrows is not None:
        check_h(ws, p, hrows, what)
    b16 = gpu_forward(inp, d, order, **kw)
    torch.cuda.synchronize()
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16)), \
        what + ": bf16 output is not the RNE rounding of the FP32 result"
    return check_bound(f32.cpu().numpy().astype(np.float64), ref, what, band)


def workspace_h(ws, p, slots):
    """The quantised h rows of the given slots that a forward on problem p
    left in workspace ws, decoded to FP64."""
    h_off, hs_off, _ = moe.workspace_offsets(p)
    A, I = p.T * p.top_k, p.I
    rows = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=ws.device)
    a4 = p.act_fmt in (moe.ACT_FP4_UE8M0_K32, moe.ACT_BF16_QUANT_FP4_K32)
    a8 = p.act_fmt != moe.ACT_BF16
    if a4:
        codes = ws[h_off:h_off + A * I // 2].view(A, I // 2)[rows].cpu().numpy()
        vals = oracle.e2m1_decode(oracle.unpack_fp4(codes))
    elif a8:
        vals = oracle.e4m3_decode(ws[h_off:h_off + A * I].view(A, I)[rows].cpu().numpy())
    else:
        bits = ws[h_off:h_off + 2 * A * I].view(torch.int16).view(A, I)[rows].cpu().numpy()
        return oracle.bf16_bits_decode(bits.view(np.uint16))
    sf = ws[hs_off:hs_off + A * (I // 32)].view(A, I // 32)[rows].cpu().numpy()
    return vals * np.repeat(oracle.ue8m0_decode(sf), 32, axis=1)


def check_h(ws, p, hrows, what=""):
    """Compare the forward's quantised h (FC2's input) with the oracle's, slot
    by slot: a value may differ only where the exact h lies within the
    decision radius (times its block maximum) of a boundary of the
    quantisation rule.  Prints one "[hcheck]" line: the number of differing
    values and the largest decision margin among them (log2, in block
    maxima), and the smallest margin over all values."""
    a4 = p.act_fmt in (moe.ACT_FP4_UE8M0_K32, moe.ACT_BF16_QUANT_FP4_K32)
    a8 = p.act_fmt != moe.ACT_BF16 and not a4
    slots = sorted(hrows)
    exact = np.stack([hrows[s][0] for s in slots])
    want = np.stack([hrows[s][1] for s in slots])
    got = workspace_h(ws, p, slots)
    margin = oracle.h_decision_margin(exact, a8, a4)
    radius = oracle.decision_radius(a8, a4)
    diff = got != want
    worst = float(np.max(margin[diff])) if diff.any() else 0.0
    lg = lambda v: f"2**{np.log2(v):.2f}" if v > 0 else "0"
    msg = (f"[hcheck] {what}: quantised h differs from the oracle's at {int(diff.sum())}/{diff.size} values, "
           f"largest margin among them {lg(worst)} (radius {lg(radius)}), "
           f"smallest margin overall {lg(float(np.min(margin)))}")
    print(msg, flush=True)
    assert np.all(margin[diff] <= radius), msg


def check_bound(got, ref, what="", band=None):
    """|err| <= 2e-2 * rms(ref) (+ the oracle's decision band: results that
    other equally valid near-tie roundings of h give) element-wise, and
    sum|err| / sum|ref| <= 5e-3.  Prints one "[bound]" line: the largest
    error without the band, the number of elements whose error exceeds the
    plain 2e-2 * rms bound (where the band was needed), the largest band."""
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    band = np.zeros_like(ref) if band is None else band
    plain = 2e-2 * rms
    excess = err - (plain + band)
    maxerr = float(np.max(err))
    needed = int(np.count_nonzero(err > plain))
    mre = float(np.sum(err) / np.sum(np.abs(ref)))
    i = np.unravel_index(np.argmax(excess), err.shape)
    msg = (f"[bound] {what}: max|err| without band {maxerr / rms:.4f} rms (plain bound 0.02), "
           f"elements above the plain bound {needed}/{err.size}, "
           f"max band {float(np.max(band)) / rms:.4f} rms, nonzero band {int(np.count_nonzero(band))}/{band.size}, "
           f"worst vs bound at {i}: err {err[i]:.3e} band {band[i]:.3e}, "
           f"mean rel {mre:.3e} (bound 5e-3)")
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert np.all(excess <= 0) and mre <= 5e-3, msg
    return maxerr / rms, mre
