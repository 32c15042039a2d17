"""The forward entry point that allocates nothing (moe_fp4_forward_static,
its workspace a static device array in the library) against the one with a
caller workspace (moe_fp4_forward): bit-identical FP32 and bf16 outputs on
two calls in a row, the second smaller (the static scratch keeps the first
call's contents), across the decode and 64-row paths; and a problem beyond
the scratch's size is refused before any launch."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import synth
from helpers import gpu_forward, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (larger call, smaller call)
    (synth.variant(synth.CONFIGS["tiny"], T=64, E=32, k=8, H=1024, I=512, seed=101),
     synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=8, H=1024, I=512, seed=102)),
    (synth.variant(synth.CONFIGS["tiny"], T=300, E=4, k=2, H=768, I=512, seed=103, gran=32, act="fp8",
                   global_scale="none", routing="zipf"),
     synth.variant(synth.CONFIGS["tiny"], T=40, E=4, k=2, H=768, I=512, seed=104, gran=32, act="fp8",
                   global_scale="none")),
]


def _static(inp, d, **kw):
    return moe.forward_static(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["w13_sf"], d["w13_gs"], d["w2"],
                              d["w2_sf"], d["w2_gs"], inp.cfg.gran, x_sf=d["x_sf"], **kw)


@pytest.mark.parametrize("pair", CASES, ids=["decode_g16", "fp8_64row"])
def test_static_equals_workspace_forward(pair):
    require_gpu()
    for cfg in pair:
        print(f"forward_static T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} {cfg.act} g{cfg.gran}", flush=True)
        inp = synth.make_moe_inputs(cfg)
        d = to_dev(inp)
        for dt in (torch.float32, torch.bfloat16):
            a = _static(inp, d, out_dtype=dt)
            b = gpu_forward(inp, d, out_dtype=dt)
            torch.cuda.synchronize()
            ia = a.view(torch.int32) if dt == torch.float32 else a.view(torch.int16)
            ib = b.view(torch.int32) if dt == torch.float32 else b.view(torch.int16)
            assert torch.equal(ia, ib)


def test_static_refuses_oversize():
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["decode32"], T=1024, E=8)
    p = moe.make_problem(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.gran, moe.ACT_FP8_UE8M0_K32)
    assert moe.workspace_bytes(p) > 64 << 20
    x = torch.zeros((cfg.T, cfg.H), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((cfg.T, cfg.H // 32), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    w13 = torch.zeros((cfg.E, 2 * cfg.I, cfg.H // 2), dtype=torch.uint8, device="cuda")
    w13s = torch.zeros((cfg.E, 2 * cfg.I, cfg.H // 32), dtype=torch.uint8, device="cuda")
    w2 = torch.zeros((cfg.E, cfg.H, cfg.I // 2), dtype=torch.uint8, device="cuda")
    w2s = torch.zeros((cfg.E, cfg.H, cfg.I // 32), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.forward_static(x, ids, w, w13, w13s, None, w2, w2s, None, 32, x_sf=xs)
    assert ei.value.status == moe.EWORKSPACE and "static scratch" in str(ei.value)
