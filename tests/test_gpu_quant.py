"""The bfloat16 -> FP8 (E4M3 + UE8M0 per 32) activation quantiser on the GPU
vs the oracle's quantisation rule: bit-exact codes and scale bytes over the
whole finite bfloat16 range (zeros, signed zeros, subnormals, blocks of
zeros, exact rounding ties), and the MoE forward with the library
quantising bfloat16 x itself (act_fmt BF16_QUANT_FP8_K32) against the oracle
run on the oracle-quantised x."""

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
    """Random bfloat16 bit patterns, every finite value possible."""
    b = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint32).astype(np.uint16)
    bad = (b & 0x7F80) == 0x7F80  # inf / NaN exponent
    b[bad] &= 0xBFFF               # clear the top exponent bit
    return b


def _bits_scaled_normal(rng, T, H):
    """N(0, 1) rows scaled by 2**U[-40, 40] per row, bfloat16 (RNE cast)."""
    v = rng.standard_normal((T, H)) * np.exp2(rng.integers(-40, 41, size=(T, 1)))
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_special(rng, T, H):
    """Blocks of zeros, signed zeros, and values that land exactly on E4M3
    rounding midpoints after the per-block scaling."""
    b = _bits_scaled_normal(rng, T, H)
    b[0, :32] = 0                     # a block of +0
    b[0, 32:64] = 0x8000              # a block of -0
    b[1, :32] = 0x8000
    b[1, 5] = 0x3F80                  # 1.0 among -0s
    # block with max 448 * 2**-3 = 56 and ties: 56 * (k + 0.5) / 16 style
    # values: 1.0625 (between 1 and 1.125 on the E4M3 grid at scale 2**-3
    # -> 8.5 units) etc.
    ties = np.array([56.0, 8.5 / 8, 9.5 / 8, -10.5 / 8, 0.5 * 2**-9 * 8, -1.5 * 2**-9 * 8], np.float32)
    row = np.zeros(32, np.float32)
    row[:ties.size] = ties
    b[2, :32] = torch.from_numpy(row).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # a block of bfloat16 subnormals only (its scale clamps at 2**-127)
    b[3, :32] = (np.arange(32, dtype=np.uint16) * 3 + 1) | np.where(np.arange(32) % 2, 0x8000, 0).astype(np.uint16)
    return b


CASES = [
    ("any_finite", _bits_any_finite, 37, 96),
    ("scaled_normal", _bits_scaled_normal, 64, 6144),
    ("special", _bits_special, 8, 256),
    ("prefill_rows", _bits_scaled_normal, 2000, 1024),
]


@pytest.mark.parametrize("name,gen,T,H", CASES, ids=[c[0] for c in CASES])
def test_quantize_act_bit_exact(name, gen, T, H):
    require_gpu()
    print(f"quantize_act case {name} T={T} H={H}", flush=True)
    rng = np.random.default_rng(17)
    bits = gen(rng, T, H)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = moe.quantize_act(x)
    torch.cuda.synchronize()
    _, rq, rs = oracle.quantize_h_a8(decode_activations(bits))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def _quant_inputs(inp):
    """The same problem with x replaced by the oracle's FP8 quantisation of it."""
    _, codes, sf = oracle.quantize_h_a8(decode_activations(inp.x))
    return codes, sf


FWD = [
    # decode-shaped (16-row tiles), several experts per token
    synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=51, gran=32,
                  act="bf16", global_scale="uniform"),
    # prefill-shaped (128-row tiles of the FP8 x FP4 GEMM)
    synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=52, gran=32,
                  act="bf16", global_scale="none", routing="zipf"),
]


@pytest.mark.parametrize("cfg", FWD, ids=["decode", "prefill"])
def test_forward_quantize_x(cfg):
    require_gpu()
    print(f"forward with quantised x: T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I}", flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    f32, ws, p = forward_ws(inp, d, quantize_x=True)
    b16 = gpu_forward(inp, d, quantize_x=True)
    torch.cuda.synchronize()
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))
    codes, sf = _quant_inputs(inp)
    ref, band, hrows = oracle.moe_forward(codes, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                                          inp.w2, inp.w2_sf, inp.w2_gs, cfg.gran, x_sf=sf, return_band=True,
                                          return_h=True)
    check_h(ws, p, hrows, "quantised-x forward")
    check_bound(f32.cpu().numpy().astype(np.float64), ref, "quantised-x forward", band)
