"""The A4 path on the GPU (MXFP4 activations: E2M1 codes + UE8M0 per 32,
FP4 x FP4 block-scaled MFMA) against the oracle: the bfloat16 -> MXFP4
quantiser bit-exact over the whole finite bfloat16 range (zeros, signed
zeros, subnormals, blocks of zeros, rounding ties), and the forward with
caller-quantised and library-quantised x at prefill and decode shapes (the
128-row GEMM tiles and the 16-row decode tiles) and at the full decode and
prefill sizes on sampled tokens, within the stated bound around the
oracle's A4 result."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import oracle
from oracle.moe import decode_activations
import synth
from helpers import check_bound, check_h, forward_ws, gpu_forward, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bits_any_finite(rng, T, H):
    b = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint32).astype(np.uint16)
    bad = (b & 0x7F80) == 0x7F80
    b[bad] &= 0xBFFF
    return b


def _bits_scaled_normal(rng, T, H):
    v = rng.standard_normal((T, H)) * np.exp2(rng.integers(-40, 41, size=(T, 1)))
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_special(rng, T, H):
    b = _bits_scaled_normal(rng, T, H)
    b[0, :32] = 0
    b[0, 32:64] = 0x8000
    b[1, :32] = 0x8000
    b[1, 5] = 0x3F80
    # block max 6 * 2**-3 = 0.75 with the E2M1 ties 5, 3.5, 2.5, 1.75, 1.25,
    # 0.75, 0.25 (times 2**-3) and a negative one
    ties = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -2.5, -0.25], np.float32) * 2.0 ** -3
    row = np.zeros(32, np.float32)
    row[:ties.size] = ties
    b[2, :32] = torch.from_numpy(row).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # bfloat16 subnormals only (the scale clamps at 2**-127)
    b[3, :32] = (np.arange(32, dtype=np.uint16) * 3 + 1) | np.where(np.arange(32) % 2, 0x8000, 0).astype(np.uint16)
    # the largest finite magnitudes
    b[3, 32:64] = 0x7F7F
    b[3, 40] = 0xFF7F
    return b


CASES = [
    ("any_finite", _bits_any_finite, 37, 96),
    ("scaled_normal", _bits_scaled_normal, 64, 6144),
    ("special", _bits_special, 8, 256),
    ("prefill_rows", _bits_scaled_normal, 2000, 1024),
]


@pytest.mark.parametrize("name,gen,T,H", CASES, ids=[c[0] for c in CASES])
def test_quantize_act_fp4_bit_exact(name, gen, T, H):
    require_gpu()
    print(f"quantize_act_fp4 case {name} T={T} H={H}", flush=True)
    rng = np.random.default_rng(18)
    bits = gen(rng, T, H)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = moe.quantize_act_fp4(x)
    torch.cuda.synchronize()
    _, rq, rs = oracle.quantize_a4(decode_activations(bits))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def _a4_ref(inp, x4, x4sf, tokens=None, out_cols=None):
    return oracle.moe_forward(x4, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                              inp.w2, inp.w2_sf, inp.w2_gs, inp.cfg.gran, x_sf=x4sf, a4=True,
                              tokens=tokens, out_cols=out_cols, return_band=True, return_h=True)


FWD = [
    # prefill-shaped: several 128-row tiles per expert, ragged tails
    synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=71, gran=32,
                  act="bf16", global_scale="uniform", routing="zipf"),
    # decode-shaped batch (16-row tiles of the decode kernel)
    synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=72, gran=32,
                  act="bf16", global_scale="none"),
    # decode-shaped with K spanning two weight-scale groups (16 chunks of
    # group32 scales per 128-byte line), the second one ragged
    synth.variant(synth.CONFIGS["tiny"], T=16, E=8, k=4, H=4608, I=2560, seed=73, gran=32,
                  act="bf16", global_scale="none"),
]


@pytest.mark.parametrize("cfg", FWD, ids=["prefill", "decode", "decode_long_k"])
def test_forward_a4(cfg):
    require_gpu()
    print(f"A4 forward: T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I}", flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    # the library quantises bf16 x ...
    f32, ws, p = forward_ws(inp, d, quantize_x="fp4")
    b16 = gpu_forward(inp, d, quantize_x="fp4")
    # ... or takes caller-quantised MXFP4 x: the same bits
    _, x4, x4sf = oracle.quantize_a4(decode_activations(inp.x))
    d4 = dict(d, x=torch.from_numpy(x4).cuda(), x_sf=torch.from_numpy(x4sf).cuda())
    f32b = gpu_forward(inp, d4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))
    assert torch.equal(f32.view(torch.int32), f32b.view(torch.int32))
    ref, band, hrows = _a4_ref(inp, x4, x4sf)
    check_h(ws, p, hrows, "A4 forward")
    check_bound(f32.cpu().numpy().astype(np.float64), ref, "A4 forward", band)


def test_full_decode_a4_sampled():
    """The decode32 shape (256 tokens over 256 experts, top-8, H = 6144,
    I = 2048) with the library quantising x to MXFP4: 16-row expert tiles;
    the oracle computes a sample of tokens over sampled columns."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["decode32"], act="bf16")
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    print("decode32 A4: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d, quantize_x="fp4")
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    tokens = sorted({0, cfg.T - 1, int(rng.integers(cfg.T)), int(rng.integers(cfg.T))})
    cols = np.sort(rng.choice(cfg.H, size=768, replace=False))
    _, x4, x4sf = oracle.quantize_a4(decode_activations(inp.x))
    print(f"decode32 A4: oracle on tokens {tokens}", flush=True)
    ref, band, hrows = _a4_ref(inp, x4, x4sf, tokens=tokens, out_cols=cols)
    check_h(ws, p, hrows, "decode32 A4 sampled")
    got = out[tokens][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_bound(got, ref, "decode32 A4 sampled", band)


def test_full_prefill_a4_sampled():
    """The prefill32 workload with the library quantising x to MXFP4, in the
    benchmark's launch configuration; the oracle computes a sample of tokens
    (including one routed to the most loaded expert) over sampled columns."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["prefill32"], act="bf16")
    print("generating prefill32 (bf16 x) inputs", flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    print("prefill32 A4: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d, quantize_x="fp4")
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    counts = np.bincount(inp.topk_ids.ravel(), minlength=cfg.E)
    heavy = int(np.flatnonzero((inp.topk_ids == counts.argmax()).any(axis=1))[0])
    tokens = sorted({0, cfg.T - 1, heavy, int(rng.integers(cfg.T))})
    cols = np.sort(rng.choice(cfg.H, size=768, replace=False))
    _, x4, x4sf = oracle.quantize_a4(decode_activations(inp.x))
    print(f"prefill32 A4: oracle on tokens {tokens}", flush=True)
    ref, band, hrows = _a4_ref(inp, x4, x4sf, tokens=tokens, out_cols=cols)
    check_h(ws, p, hrows, "prefill32 A4 sampled")
    got = out[tokens][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_bound(got, ref, "prefill32 A4 sampled", band)
