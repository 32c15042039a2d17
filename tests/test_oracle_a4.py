"""Pins of the oracle's A4 path (MXFP4 activations: E2M1 codes + UE8M0 per
32): the row quantiser against brute force over the E2M1 grid (minimal
exponent, nearest code, ties to the even code, signed zeros, zero blocks,
nibble order), its decode, the decision band on hand-built blocks, and the
whole forward against a scalar-loop version whose every decode goes through
torch (bias identity for E2M1, float8_e8m0fnu views for the scales)."""

import math

import numpy as np
import torch

import oracle
import synth
from oracle.moe import decode_activations

GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _brute_code(y):
    """E2M1 code of y (|y| <= 6) by nearest grid value, ties to the even code."""
    d = np.abs(GRID - abs(y))
    cand = np.flatnonzero(d == d.min())
    mag = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
    return int(mag) | (8 if math.copysign(1.0, y) < 0 else 0)


def test_quantize_a4_brute_force():
    rng = np.random.default_rng(40)
    v = rng.standard_normal((5, 128)) * np.exp2(rng.integers(-30, 30, size=(5, 1)))
    v[1, :32] = 0.0
    v[1, 32:64] = -0.0
    v[2, 64:96] = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25] * 4) * 2.0 ** -3  # ties at e = -3
    v[2, 65] = -v[2, 65]
    v[3, 0] = -2.0 ** -140  # a value far below the block maximum
    vh, packed, sb = oracle.quantize_a4(v)
    codes = oracle.unpack_fp4(packed)
    for r in range(v.shape[0]):
        for b in range(4):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            e = int(sb[r, b]) - 127
            if amax == 0:
                assert e == -127
            else:
                assert 6 * 2.0 ** e >= amax > 6 * 2.0 ** (e - 1)
            for i, y in enumerate(blk):
                c = _brute_code(y / 2.0 ** e)
                assert codes[r, 32 * b + i] == c, (r, b, i, y, e)
                assert vh[r, 32 * b + i] == math.copysign(GRID[c & 7], -1.0 if c & 8 else 1.0) * 2.0 ** e
    # the tie block: 5 -> 4, 3.5 -> 4, 2.5 -> 2, 1.75 -> 2, 1.25 -> 1, 0.75 -> 1, 0.25 -> 0
    assert list(codes[2, 64:72]) == [7, 8 | 6, 6, 4, 4, 2, 2, 0]
    # byte j holds element 2j in its low nibble
    assert packed[2, 32] == codes[2, 64] | (codes[2, 65] << 4)
    # decode of the packed form gives the quantised values
    assert np.array_equal(decode_activations(packed, sb, a4=True), vh)


def test_decision_band_a4():
    """Block max 1.4 (e = -2, scaled grid step 0.5 below 2): scaled 1.25 is a
    midpoint, within the radius 1.4 * 2**-17 of it the band is one step, away
    from it zero; a block maximum on 6 * 2**e spans both exponents."""
    h = np.zeros((1, 32))
    h[0, 0] = 1.4
    h[0, 1] = 1.25 * 0.25                    # scaled 1.25: midpoint of 1 and 1.5
    h[0, 2] = 1.25 * 0.25 + 2.0 ** -19       # within 1.4 * 2**-17 of it
    h[0, 3] = 1.25 * 0.25 + 2.0 ** -15       # outside
    band = oracle.h_decision_band(h, False, a4=True)
    assert band[0, 1] == 0.5 * 0.25 and band[0, 2] == 0.5 * 0.25
    assert band[0, 3] == 0 and band[0, 0] == 0
    # amax just above 6 * 2**-3: e = -2, but e = -3 is within the radius;
    # 0.16 quantises to 0.125 under e = -2 (0.64 -> 0.5) and to 0.1875 under
    # e = -3 (1.28 -> 1.5), while the maximum is 0.75 under both
    h2 = np.zeros((1, 32))
    h2[0, 0] = 6 * 2.0 ** -3 * (1 + 2.0 ** -20)
    h2[0, 1] = 0.16
    hh, _, sb = oracle.quantize_a4(h2)
    assert int(sb[0, 0]) - 127 == -2 and hh[0, 1] == 0.125
    b2 = oracle.h_decision_band(h2, False, a4=True)
    assert b2[0, 0] == 0 and b2[0, 1] == 0.0625


def _e2m1_torch(codes):
    c = np.asarray(codes, np.int64)
    bits = ((c >> 3) << 15) | (((c >> 1) & 3) << 7) | ((c & 1) << 6)
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy() * 2.0 ** 126


def _w_torch(packed, sf):
    p = np.asarray(packed)
    c = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    c[..., 0::2] = p & 15
    c[..., 1::2] = p >> 4
    s = torch.from_numpy(np.ascontiguousarray(sf)).view(torch.float8_e8m0fnu).double().numpy()
    return _e2m1_torch(c) * np.repeat(s, 32, axis=-1)


def test_a4_forward_brute_force():
    """A4 end to end on a tiny problem: x quantised by brute force, FC1 by
    scalar loops, h quantised by brute force per 32, FC2, weighted sum."""
    cfg = synth.variant(synth.CONFIGS["decode32"], T=2, E=3, k=2, H=64, I=64, seed=10, act="bf16")
    inp = synth.make_moe_inputs(cfg)
    xf = decode_activations(inp.x)
    _, x4, x4sf = oracle.quantize_a4(xf)
    got = oracle.moe_forward(x4, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, None, inp.w2,
                             inp.w2_sf, None, 32, x_sf=x4sf, a4=True)

    def quant_block_brute(blk):
        amax = np.max(np.abs(blk))
        if amax == 0:
            return np.zeros_like(blk)
        e = math.ceil(math.log2(amax / 6))
        while 6 * 2.0 ** (e - 1) >= amax:
            e -= 1
        while 6 * 2.0 ** e < amax:
            e += 1
        return np.array([math.copysign(GRID[_brute_code(y / 2.0 ** e) & 7], y) * 2.0 ** e for y in blk])

    x = np.concatenate([quant_block_brute(xf[t, 32 * b:32 * b + 32])[None] for t in range(2)
                        for b in range(2)]).reshape(2, 64)
    ref = np.zeros((2, 64))
    for t in range(2):
        for j in range(2):
            e = int(inp.topk_ids[t, j])
            W13 = _w_torch(inp.w13[e], inp.w13_sf[e])
            W2 = _w_torch(inp.w2[e], inp.w2_sf[e])
            h = np.zeros(64)
            for i in range(64):
                g = sum(x[t, q] * W13[i, q] for q in range(64))
                u = sum(x[t, q] * W13[64 + i, q] for q in range(64))
                h[i] = g / (1 + math.exp(-g)) * u
            hq = np.concatenate([quant_block_brute(h[32 * b:32 * b + 32]) for b in range(2)])
            for n in range(64):
                ref[t, n] += float(inp.topk_w[t, j]) * sum(hq[i] * W2[n, i] for i in range(64))
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
