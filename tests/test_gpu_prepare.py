"""GEMM weight layout (moe_fp4_prepare_gemm_weights): the GPU reorder equals
the layout's definition (written out here in numpy from the header's
formulas), and a forward on prepared weights equals the forward on the RAW
weights bit for bit (same kernel arithmetic, only the weight addressing
differs) and meets the accuracy bound against the oracle, at prefill shapes
with FP8 and FP4 activations, both w13 orders, and at the full prefill
workload."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import oracle
from oracle.moe import decode_activations
import synth
from helpers import check_bound, check_h, forward_ws, gpu_forward, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def gemm_layout_ref(src, src_sf, w13, order):
    """The definition: 512-row blocks (w13: 256 gate rows then the matching
    up rows), per 128-wide K stage 2048 16-byte slots, slot j holding piece
    (j & 3) ^ ((j >> 4) & 3) of the stage's 64 bytes of block row j >> 2;
    scales per 512-wide group: the block's 512 rows' 16 bytes in order."""
    E, N, kh = src.shape
    K = 2 * kh
    dst = np.empty_like(src)
    dsf = np.empty_like(src_sf)

    def row(nb, i):
        if not w13:
            return nb * 512 + i
        i0 = nb * 256 + (i % 256)
        return N // 2 + i0 if (i >= 256) != (order == 1) else i0

    for e in range(E):
        d = dst[e].reshape(-1, 16)
        ds = dsf[e].reshape(-1, 16)
        for nb in range(N // 512):
            for s in range(K // 128):
                for j in range(2048):
                    p = (j & 3) ^ ((j >> 4) & 3)
                    c = (nb * (K // 128) + s) * 2048 + j
                    d[c] = src[e, row(nb, j >> 2), 64 * s + 16 * p: 64 * s + 16 * p + 16]
            for g in range(K // 512):
                for i in range(512):
                    ds[(nb * (K // 512) + g) * 512 + i] = src_sf[e, row(nb, i), 16 * g: 16 * g + 16]
    return dst, dsf


@pytest.mark.parametrize("which,N,K,order", [("w13", 1024, 1024, 0), ("w13", 1024, 512, 1), ("w2", 1536, 1024, 0)])
def test_prepare_matches_definition(which, N, K, order):
    require_gpu()
    print(f"prepare {which} N={N} K={K} order={order}", flush=True)
    rng = np.random.default_rng(3)
    src = rng.integers(0, 256, size=(2, N, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 256, size=(2, N, K // 32), dtype=np.uint8)
    d, dsf = moe.prepare_gemm_weights(torch.from_numpy(src).cuda(), torch.from_numpy(sf).cuda(), which, order)
    torch.cuda.synchronize()
    rd, rdsf = gemm_layout_ref(src, sf, which == "w13", order)
    assert np.array_equal(d.cpu().numpy(), rd)
    assert np.array_equal(dsf.cpu().numpy(), rdsf)


def prepared(d, order="gate_up"):
    p = dict(d)
    p["w13"], p["w13_sf"] = moe.prepare_gemm_weights(d["w13"], d["w13_sf"], "w13", order)
    p["w2"], p["w2_sf"] = moe.prepare_gemm_weights(d["w2"], d["w2_sf"], "w2")
    return p


CASES = [
    synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=81, gran=32, act="fp8",
                  global_scale="none", routing="zipf"),
    synth.variant(synth.CONFIGS["tiny"], T=300, E=8, k=2, H=512, I=512, seed=82, gran=32, act="fp8",
                  global_scale="uniform"),
    synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=83, gran=32, act="bf16q4",
                  global_scale="none", routing="zipf"),
]


@pytest.mark.parametrize("cfg", CASES, ids=["fp8_zipf", "fp8_k512_gs", "a4_zipf"])
@pytest.mark.parametrize("order", ["gate_up", "up_gate"])
def test_forward_prepared_equals_raw(cfg, order):
    require_gpu()
    print(f"prepared forward T={cfg.T} E={cfg.E} H={cfg.H} I={cfg.I} act={cfg.act} order={order}", flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    q = {"bf16q4": "fp4"}.get(cfg.act, False)
    raw = gpu_forward(inp, d, order, out_dtype=torch.float32, quantize_x=q)
    pd = prepared(d, order)
    prep, ws, p = forward_ws(inp, pd, order, quantize_x=q, w_layout="gemm")
    torch.cuda.synchronize()
    assert torch.equal(raw.view(torch.int32), prep.view(torch.int32))
    # and the forward on prepared weights against the oracle directly
    if cfg.act == "bf16q4":
        _, xr, xr_sf = oracle.quantize_a4(decode_activations(inp.x))
    else:
        xr, xr_sf = inp.x, inp.x_sf
    ref, band, hrows = oracle.moe_forward(xr, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs, inp.w2,
                                          inp.w2_sf, inp.w2_gs, cfg.gran, x_sf=xr_sf, w13_order=order,
                                          a4=cfg.act == "bf16q4", return_band=True, return_h=True)
    check_h(ws, p, hrows, f"GEMM-layout forward {cfg.act} {order}")
    check_bound(prep.cpu().numpy().astype(np.float64), ref, f"GEMM-layout forward {cfg.act} {order}", band)


def test_full_prefill_prepared_equals_raw():
    """The prefill workload in the benchmark's launch configuration."""
    require_gpu()
    print("generating full prefill32 inputs", flush=True)
    inp = synth.make_moe_inputs(synth.CONFIGS["prefill32"])
    d = to_dev(inp)
    print("prefill32 prepared: running on GPU", flush=True)
    raw = gpu_forward(inp, d, out_dtype=torch.float32)
    prep = gpu_forward(inp, prepared(d), out_dtype=torch.float32, w_layout="gemm")
    torch.cuda.synchronize()
    assert torch.equal(raw.view(torch.int32), prep.view(torch.int32))


@pytest.mark.parametrize("which,N,K,order", [("w13", 1024, 1024, 0), ("w13", 1024, 1536, 1), ("w2", 1536, 1024, 0)])
def test_prepare_g16_matches_requant_then_prepare(which, N, K, order):
    """The one-pass group16 -> GEMM-layout group32 preparation equals the
    requantisation followed by the reorder, bit for bit, and the oracle's
    requantisation laid out by the layout's definition."""
    require_gpu()
    print(f"prepare g16 {which} N={N} K={K} order={order}", flush=True)
    E = 3
    src = np.empty((E, N, K // 2), np.uint8)
    sf = np.empty((E, N, K // 16), np.uint8)
    for e in range(E):
        src[e], sf[e] = synth.make_fp4_tensor(91, 10, e, N, K, 16, (-10.0, -3.0))
    gs = np.array([0.75, -1.5, 1.25], np.float32)  # a negative global scale flips signs
    ts, tsf, tgs = (torch.from_numpy(a).cuda() for a in (src, sf, gs))
    d, dsf = moe.prepare_gemm_weights_g16(ts, tsf, tgs, which, order)
    r, rsf = moe.requant_gran_k(ts, tsf, tgs)
    p, psf = moe.prepare_gemm_weights(r, rsf, which, order)
    torch.cuda.synchronize()
    assert torch.equal(d, p) and torch.equal(dsf, psf)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, gs)
    ld, ldsf = gemm_layout_ref(rd, rdsf, which == "w13", order)
    assert np.array_equal(d.cpu().numpy(), ld)
    assert np.array_equal(dsf.cpu().numpy(), ldsf)


@pytest.mark.parametrize("order", ["gate_up", "up_gate"])
def test_forward_on_g16_prepared_weights(order):
    """A group16 NVFP4 layer prepared in one pass (requantised to group32
    with the global scales folded in, GEMM layout) runs the FP8 x FP4
    prefill GEMM; the oracle runs the same layer requantised by its own
    arithmetic."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=92, gran=16, act="fp8",
                        global_scale="uniform", routing="zipf")
    print(f"forward on g16-prepared weights order={order}", flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    pd = dict(d, w13_gs=None, w2_gs=None)
    pd["w13"], pd["w13_sf"] = moe.prepare_gemm_weights_g16(d["w13"], d["w13_sf"], d["w13_gs"], "w13", order)
    pd["w2"], pd["w2_sf"] = moe.prepare_gemm_weights_g16(d["w2"], d["w2_sf"], d["w2_gs"], "w2")
    g32 = synth.variant(cfg, gran=32, global_scale="none")
    out, ws, p = forward_ws(synth.MoEInputs(g32, inp.x, inp.x_sf, inp.topk_ids, inp.topk_w, None, None, None,
                                            None, None, None), pd, order, w_layout="gemm")
    torch.cuda.synchronize()
    w13, w13_sf = oracle.requant_g16_to_g32(inp.w13, inp.w13_sf, inp.w13_gs)
    w2, w2_sf = oracle.requant_g16_to_g32(inp.w2, inp.w2_sf, inp.w2_gs)
    ref, band, hrows = oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, w13, w13_sf, None, w2, w2_sf, None, 32,
                                          x_sf=inp.x_sf, w13_order=order, return_band=True, return_h=True)
    check_h(ws, p, hrows, f"g16-prepared forward {order}")
    check_bound(out.cpu().numpy().astype(np.float64), ref, f"g16-prepared forward {order}", band)
