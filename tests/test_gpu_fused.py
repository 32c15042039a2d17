"""The single-launch forward (moe_fp4_forward_fused: FC1 and FC2 of the
16-row decode tiles in one persistent kernel, h passed through each XCD's L2
under per-tile counters).  Its arithmetic is the two-launch forward's, item
for item, so its output must equal moe_fp4_forward's bit for bit on every
decode-shaped case (every activation / scale format, both w13 orders,
ragged tiles, the largest decode batch and the full decode16 / decode32
workloads), no wait may have hit its time limit, and it is checked against
the oracle directly on a few cases."""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_bound, check_h, forward_ws, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def combos(base):
    return [
        synth.variant(base, gran=16, act="bf16", global_scale="uniform"),
        synth.variant(base, gran=32, act="bf16", global_scale="none"),
        synth.variant(base, gran=32, act="fp8", global_scale="none"),
    ]


def _id(c):
    return f"{c.act}-g{c.gran}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-I{c.I}"


DECODE = (combos(synth.CONFIGS["tiny"])
          + combos(synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=21))
          + combos(synth.variant(synth.CONFIGS["tiny"], T=13, E=6, k=3, H=768, I=256, seed=22))
          + combos(synth.variant(synth.CONFIGS["tiny"], T=16, E=8, k=4, H=4352, I=2304, seed=25))
          + combos(synth.variant(synth.CONFIGS["tiny"], T=1024, E=512, k=8, H=512, I=256, seed=43))
          # last scale groups of 5 (FC1) and 7 (FC2) group16 chunks
          + [synth.variant(synth.CONFIGS["tiny"], T=16, E=8, k=4, H=3328, I=1792, seed=26, gran=16, act="bf16",
                           global_scale="uniform")])


def both(inp, d, order="gate_up", **kw):
    """(two-launch output, fused output, fused workspace, problem), FP32."""
    ref, _, _ = forward_ws(inp, d, order, **kw)
    out, ws, p = forward_ws(inp, d, order, fused=True, **kw)
    torch.cuda.synchronize()
    timeouts = int(ws[4:8].view(torch.int32).item())
    assert timeouts == 0, f"{timeouts} waits of the fused kernel hit their time limit"
    return ref, out, ws, p


def assert_same(ref, out, what):
    a, b = ref.view(torch.int32), out.view(torch.int32)
    n = int((a != b).sum().item())
    print(f"[fused] {what}: {n} of {a.numel()} FP32 outputs differ from the two-launch forward's", flush=True)
    assert n == 0


@pytest.mark.parametrize("cfg", DECODE, ids=[_id(c) for c in DECODE])
def test_fused_equals_two_launch(cfg):
    require_gpu()
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    for order in ("gate_up", "up_gate"):
        ref, out, _, _ = both(inp, d, order)
        assert_same(ref, out, f"{_id(cfg)} {order}")


@pytest.mark.parametrize("quant", ["fp8", "fp4"])
def test_fused_quantised_x(quant):
    """bf16 x quantised by the library (FP8, or MXFP4: the A4 decode path,
    decode kernel MODE 3)."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=51, gran=32, act="bf16",
                        global_scale="none")
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    ref, out, _, _ = both(inp, d, quantize_x=quant)
    assert_same(ref, out, f"quantised x {quant}")


def test_fused_against_oracle():
    """Directly against the oracle (group16 bf16 and FP8), with the quantised
    h the fused kernel left in its workspace checked value by value."""
    require_gpu()
    for cfg in (synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=52, gran=16,
                              act="bf16", global_scale="uniform"),
                synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=53, gran=32,
                              act="fp8", global_scale="none")):
        inp = synth.make_moe_inputs(cfg)
        d = to_dev(inp)
        out, ws, p = forward_ws(inp, d, fused=True)
        torch.cuda.synchronize()
        assert int(ws[4:8].view(torch.int32).item()) == 0
        ref, band, hrows = oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                                              inp.w2, inp.w2_sf, inp.w2_gs, cfg.gran, x_sf=inp.x_sf,
                                              return_band=True, return_h=True)
        check_h(ws, p, hrows, f"fused {_id(cfg)}")
        check_bound(out.cpu().numpy().astype(np.float64), ref, f"fused {_id(cfg)}", band)


def test_fused_deterministic():
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], T=64, E=32, k=8, H=1024, I=512, seed=54)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    first, _, _ = forward_ws(inp, d, fused=True)
    for _ in range(3):
        again, _, _ = forward_ws(inp, d, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int32), again.view(torch.int32))


@pytest.mark.parametrize("name", ["decode16", "decode32"])
def test_fused_full_size(name):
    """The full decode workloads: bit-identical to the two-launch forward."""
    require_gpu()
    inp = synth.make_moe_inputs(synth.CONFIGS[name])
    d = to_dev(inp)
    print(f"fused {name}: running on GPU", flush=True)
    ref, out, _, _ = both(inp, d)
    assert_same(ref, out, name)
