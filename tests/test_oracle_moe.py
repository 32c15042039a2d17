"""Pins of the oracle's routing and MoE forward: a library stable sort,
invariants, a brute-force scalar-loop MoE on tiny inputs whose weight decode
goes through torch (bias identity + float8 views), a hand-built closed form,
and exact algebraic properties."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.moe import decode_activations


def test_route_matches_stable_argsort():
    rng = np.random.default_rng(0)
    for E, T, k in [(8, 32, 2), (256, 64, 8), (5, 7, 3)]:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        counts, offsets, sa, slot = oracle.route(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(sa, np.argsort(flat, kind="stable"))
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(slot[sa], np.arange(T * k))  # inverse permutation


def test_route_drops_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], dtype=np.int32)
    counts, offsets, sa, slot = oracle.route(ids, 4)
    assert list(counts) == [2, 2, 0, 0]
    assert list(sa) == [0, 5, 3, 4, -1, -1]
    assert slot[1] == -1 and slot[2] == -1


def _decode_w_torch(packed, sf, gran, gs):
    """Independent weight decode: E2M1 by the bias identity through torch
    bfloat16 (x 2**126), scales through torch float8 views."""
    p = np.asarray(packed)
    c = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    c[..., 0::2] = p & 15
    c[..., 1::2] = p >> 4
    bits = ((c >> 3) << 15) | (((c >> 1) & 3) << 7) | ((c & 1) << 6)
    v = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy() * 2.0 ** 126
    dt = torch.float8_e4m3fn if gran == 16 else torch.float8_e8m0fnu
    s = torch.from_numpy(np.ascontiguousarray(sf)).view(dt).double().numpy()
    return v * np.repeat(s, gran, axis=-1) * (1.0 if gs is None else float(gs))


def _assert_not_near_tie(v, sig_bits, min_exp):
    """torch casts FP64 -> FP32 -> narrow format; that equals one RNE rounding
    unless v lies within an FP32 ulp of a tie of the narrow format."""
    if v == 0:
        return
    e = max(math.frexp(abs(v))[1] - 1, min_exp)
    q = abs(v) / 2.0 ** (e - sig_bits + 1)
    assert abs(q - math.floor(q) - 0.5) > 2.0 ** -12, "too close to a tie for a torch reference"


def _bf16_round_torch(v):
    _assert_not_near_tie(v, 8, -126)
    return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double())


def _brute_moe(inp, order="gate_up"):
    """Scalar loops: for every token and every chosen expert, FC1 row by row,
    SwiGLU with math.exp, bfloat16 h through torch, FC2, weighted sum."""
    c = inp.cfg
    x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).double().numpy()
    out = np.zeros((c.T, c.H))
    for t in range(c.T):
        for j in range(c.k):
            e = int(inp.topk_ids[t, j])
            W13 = _decode_w_torch(inp.w13[e], inp.w13_sf[e], c.gran,
                                  None if inp.w13_gs is None else inp.w13_gs[e])
            W2 = _decode_w_torch(inp.w2[e], inp.w2_sf[e], c.gran,
                                 None if inp.w2_gs is None else inp.w2_gs[e])
            h = []
            for i in range(c.I):
                gi, ui = (i, c.I + i) if order == "gate_up" else (c.I + i, i)
                g = sum(float(x[t, q]) * float(W13[gi, q]) for q in range(c.H))
                u = sum(float(x[t, q]) * float(W13[ui, q]) for q in range(c.H))
                h.append(_bf16_round_torch(g / (1.0 + math.exp(-g)) * u))
            for n in range(c.H):
                y = sum(h[i] * float(W2[n, i]) for i in range(c.I))
                out[t, n] += float(inp.topk_w[t, j]) * y
    return out


def _tiny(T=3, E=3, k=2, H=32, I=32, gran=16, seed=5, gs="uniform"):
    cfg = synth.variant(synth.CONFIGS["tiny"], T=T, E=E, k=k, H=H, I=I, gran=gran,
                        seed=seed, global_scale=gs)
    return synth.make_moe_inputs(cfg)


@pytest.mark.parametrize("gran,order", [(16, "gate_up"), (16, "up_gate"), (32, "gate_up")])
def test_forward_brute_force(gran, order):
    inp = _tiny(gran=gran, gs="uniform" if gran == 16 else "none")
    ref = _brute_moe(inp, order)
    got = oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf,
                             inp.w13_gs, inp.w2, inp.w2_sf, inp.w2_gs, gran,
                             w13_order=order)
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_forward_closed_form():
    """One token, two experts, one-hot x: FC1 picks column 0 of each W13 row,
    W2 is a signed permutation, so out[n] = sum_j w_j * bf16(silu(g)u)[pi(n)] * w2v."""
    H = I = 32
    E, k = 2, 2
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80  # 1.0
    ids = np.array([[1, 0]], np.int32)
    tw = np.array([[0.75, 0.25]], np.float32)
    codes13 = np.zeros((E, 2 * I, H), np.uint8)
    codes2 = np.zeros((E, H, I), np.uint8)
    rng = np.random.default_rng(7)
    g_code = rng.integers(0, 16, size=(E, I))
    u_code = rng.integers(0, 16, size=(E, I))
    codes13[:, :I, 0] = g_code
    codes13[:, I:, 0] = u_code
    perm = np.stack([rng.permutation(I) for _ in range(E)])
    w2c = rng.integers(1, 16, size=(E, H))
    for e in range(E):
        codes2[e, np.arange(H), perm[e]] = w2c[e]
    sf13 = np.full((E, 2 * I, H // 16), 0x40, np.uint8)  # E4M3 2.0
    sf2 = np.full((E, H, I // 16), 0x30, np.uint8)       # E4M3 0.5
    gs13 = np.array([1.25, 0.75], np.float32)
    gs2 = np.array([1.5, 2.0], np.float32)
    out = oracle.moe_forward(x, ids, tw, oracle.pack_fp4(codes13), sf13, gs13,
                             oracle.pack_fp4(codes2), sf2, gs2, 16)
    table = [0, .5, 1, 1.5, 2, 3, 4, 6]

    def val(c):
        return (-1.0 if c & 8 else 1.0) * table[c & 7]

    exp = np.zeros(H)
    for j in range(k):
        e = int(ids[0, j])
        hb = []
        for i in range(I):
            g = val(int(g_code[e, i])) * 2.0 * float(gs13[e])
            u = val(int(u_code[e, i])) * 2.0 * float(gs13[e])
            hb.append(_bf16_round_torch(g / (1 + math.exp(-g)) * u))
        for n in range(H):
            exp[n] += float(tw[0, j]) * hb[perm[e, n]] * val(int(w2c[e, n])) * 0.5 * float(gs2[e])
    assert np.allclose(out[0], exp, rtol=1e-13, atol=1e-300)


def _fwd(inp, **kw):
    args = dict(x=inp.x, topk_ids=inp.topk_ids, topk_w=inp.topk_w, w13=inp.w13,
                w13_sf=inp.w13_sf, w13_gs=inp.w13_gs, w2=inp.w2, w2_sf=inp.w2_sf,
                w2_gs=inp.w2_gs, gran=inp.cfg.gran, x_sf=inp.x_sf)
    args.update(kw)
    return oracle.moe_forward(**args)


def test_properties():
    inp = _tiny(T=6, E=4, k=2, H=64, I=32)
    base = _fwd(inp)
    # linear in the router weights (exact: scaling by 2)
    assert np.array_equal(_fwd(inp, topk_w=inp.topk_w * 2), 2 * base)
    # linear in the FC2 global scale (h does not depend on it)
    assert np.array_equal(_fwd(inp, w2_gs=inp.w2_gs * 2), 2 * base)
    # zero up-half -> zero output
    w13z = oracle.unpack_fp4(inp.w13).copy()
    w13z[:, 32:, :] = 0
    assert np.all(_fwd(inp, w13=oracle.pack_fp4(w13z)) == 0)
    # token permutation equivariance
    p = np.random.default_rng(3).permutation(6)
    got = _fwd(inp, x=inp.x[p], topk_ids=inp.topk_ids[p], topk_w=inp.topk_w[p])
    assert np.allclose(got, base[p], rtol=1e-12, atol=1e-12 * np.abs(base).max())
    # up_gate order == gate_up order of the rows rotated by I
    rot = np.roll(inp.w13, 32, axis=1)
    rots = np.roll(inp.w13_sf, 32, axis=1)
    got = _fwd(inp, w13=rot, w13_sf=rots, w13_order="up_gate")
    assert np.array_equal(got, base)
    # a duplicated expert in one token acts like one pick with the summed weight
    ids = inp.topk_ids.copy()
    ids[0, 1] = ids[0, 0]
    w = inp.topk_w.copy()
    w[0, 0], w[0, 1] = 0.25, 0.5  # their FP32 sum is exact
    a = _fwd(inp, topk_ids=ids, topk_w=w)
    w1 = w.copy()
    w1[0, 0] = w[0, 0] + w[0, 1]
    w1[0, 1] = 0
    b = _fwd(inp, topk_ids=ids, topk_w=w1)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-12 * np.abs(b).max())
    # subsets of tokens / columns agree with the full result
    sub = _fwd(inp, tokens=[4, 1], out_cols=[0, 7, 63])
    assert np.array_equal(sub, base[[4, 1]][:, [0, 7, 63]])


def test_quantize_h_a8_brute_force():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((4, 128)) * np.exp2(rng.integers(-20, 20, size=(4, 1)))
    h[1, :32] = 0.0
    hh, q, sb = oracle.quantize_h_a8(h)
    grid = oracle.e4m3_decode(np.arange(0x7F))
    for r in range(4):
        for b in range(4):
            blk = h[r, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            e = int(sb[r, b]) - 127
            if amax == 0:
                assert e == -127
                continue
            assert 448 * 2.0 ** e >= amax > 448 * 2.0 ** (e - 1)
            for i, v in enumerate(blk):
                d = np.abs(grid * 2.0 ** e - abs(v))
                cand = np.flatnonzero(d == d.min())
                want = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
                assert (q[r, 32 * b + i] & 0x7F) == want
                assert hh[r, 32 * b + i] == np.copysign(grid[want] * 2.0 ** e, v)


def test_a8_forward_brute_force():
    """A8: decoded FP8 activations, h quantised per 32 -- checked against a
    scalar-loop version that uses torch float8 views for every decode."""
    cfg = synth.variant(synth.CONFIGS["decode32"], T=2, E=3, k=2, H=64, I=64, seed=9)
    inp = synth.make_moe_inputs(cfg)
    got = _fwd(inp)
    xq = torch.from_numpy(inp.x).view(torch.float8_e4m3fn).double().numpy()
    xs = torch.from_numpy(inp.x_sf).view(torch.float8_e8m0fnu).double().numpy()
    x = xq * np.repeat(xs, 32, axis=1)
    ref = np.zeros((2, 64))
    for t in range(2):
        for j in range(2):
            e = int(inp.topk_ids[t, j])
            W13 = _decode_w_torch(inp.w13[e], inp.w13_sf[e], 32, None)
            W2 = _decode_w_torch(inp.w2[e], inp.w2_sf[e], 32, None)
            h = np.zeros(64)
            for i in range(64):
                g = sum(x[t, q] * W13[i, q] for q in range(64))
                u = sum(x[t, q] * W13[64 + i, q] for q in range(64))
                h[i] = g / (1 + math.exp(-g)) * u
            hq = np.zeros(64)
            for b in range(2):
                blk = h[32 * b:32 * b + 32]
                e8 = math.ceil(math.log2(np.max(np.abs(blk)) / 448))
                while 448 * 2.0 ** (e8 - 1) >= np.max(np.abs(blk)):
                    e8 -= 1
                while 448 * 2.0 ** e8 < np.max(np.abs(blk)):
                    e8 += 1
                for y in blk / 2.0 ** e8:
                    _assert_not_near_tie(y, 4, -6)
                q = torch.from_numpy(blk / 2.0 ** e8).to(torch.float8_e4m3fn).double().numpy()
                hq[32 * b:32 * b + 32] = q * 2.0 ** e8
            for n in range(64):
                ref[t, n] += float(inp.topk_w[t, j]) * sum(hq[i] * W2[n, i] for i in range(64))
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_decision_band():
    """The band is one grid step exactly for values within the radius (times
    the block maximum) of a rounding midpoint, zero elsewhere, and covers the
    neighbouring exponent when a block maximum sits on 448 * 2**e."""
    assert oracle.decision_radius(False) == 2.0 ** -17 and oracle.decision_radius(True, a4=True) == 2.0 ** -17
    assert oracle.decision_radius(True) == 2.0 ** -13
    # bf16, block max 4: radius 4 * 2**-17 = 2**-15.  1 + 2**-8 is a midpoint
    # (step 2**-7); 1 + 2**-8 + 2**-16 is within the radius, + 2**-14 is not
    h = np.zeros((1, 32))
    h[0, :5] = [1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -16, 1.0 + 2.0 ** -8 + 2.0 ** -14,
                1.0 + 2.0 ** -9, 4.0]
    b = oracle.h_decision_band(h, a8=False)
    assert list(b[0, :5]) == [2.0 ** -7, 2.0 ** -7, 0.0, 0.0, 0.0] and not b[0, 5:].any()
    # E4M3, block max 300 (e = 0, FP8 radius 300 * 2**-13 ~ 0.037): the midpoint
    # 1 + 2**-4 is ambiguous by one step (0.125); 2.3 is clear; a value in the
    # subnormal range is ambiguous by its quantum 2**-9 (its half-step is
    # smaller than the radius)
    blk = np.zeros((1, 32))
    blk[0, :4] = [300.0, 1.0 + 2.0 ** -4, 2.3, 3 * 2.0 ** -9]
    b = oracle.h_decision_band(blk, a8=True)
    assert b[0, 0] == 0 and b[0, 1] == 0.125 and b[0, 2] == 0 and b[0, 3] == 2.0 ** -9
    # block max on the exponent boundary 448 * 2**0: the band covers the
    # requantisation of the whole block with e = 1
    blk[0, 0] = 448.0
    b = oracle.h_decision_band(blk, a8=True)
    prim = oracle.quantize_h_a8(blk)[0]
    alt = np.ldexp(oracle.e4m3_decode(oracle.rne_e4m3(blk / 2.0)), 1)
    assert np.all(b >= np.abs(alt - prim)) and np.any(alt != prim)


def _seq_fp32_h_distance(cfg, rows, toks, experts):
    """Largest |h32 - h| / (block max of |h|) over the first `toks` tokens and
    the first `rows` gate rows (with their up rows) of the first `experts`
    experts: h exact (FP64), h32 from an FP32 emulation of the kernels'
    arithmetic -- exact products, each added to an FP32 sum in sequence (the
    most roundings any accumulation order takes), the global scale applied
    to the FP32 sum, SwiGLU in FP32."""
    inp = synth.make_moe_inputs(cfg)
    xv = decode_activations(inp.x, inp.x_sf)
    kind = {16: "e4m3", 32: "ue8m0"}[cfg.gran]
    sel = np.r_[0:rows, cfg.I:cfg.I + rows]
    worst = 0.0
    for e in range(experts):
        W = oracle.dequant_fp4(inp.w13[e][sel], inp.w13_sf[e][sel], cfg.gran, kind, None)
        gs = 1.0 if inp.w13_gs is None else float(inp.w13_gs[e])
        X = xv[:toks]
        P = X[:, None, :] * W[None, :, :]
        P32 = P.astype(np.float32)
        assert np.array_equal(P32.astype(np.float64), P), "FC1 products are exact in FP32"
        G = (X @ W.T) * gs
        G32 = np.add.accumulate(P32, axis=2, dtype=np.float32)[..., -1] * np.float32(gs)
        h = oracle.silu(G[:, :rows]) * G[:, rows:]
        g3, u3 = G32[:, :rows], G32[:, rows:]
        h32 = (g3 / (np.float32(1) + np.exp(-g3)) * u3).astype(np.float64)
        bmax = np.abs(h).reshape(toks, rows // 32, 32).max(axis=-1)
        d = np.abs(h32 - h).reshape(toks, rows // 32, 32) / bmax[..., None]
        worst = max(worst, float(d.max()))
    return worst


@pytest.mark.parametrize("name", ["decode16", "decode32", "prefill_bf16_g32", "tiny"])
def test_decision_radius_covers_fp32(name):
    """The decision radius (2**-17 of the block maximum) is at least four times
    the distance between the exact h and an FP32 computation of it in the
    order with the most roundings, on the workloads' shapes (K = 6144 for
    the GLM-sized layers)."""
    cfg = {"decode16": synth.variant(synth.CONFIGS["decode16"], T=8, E=2),
           "decode32": synth.variant(synth.CONFIGS["decode32"], T=8, E=2),
           "prefill_bf16_g32": synth.variant(synth.CONFIGS["decode32"], T=8, E=2, act="bf16"),
           "tiny": synth.CONFIGS["tiny"]}[name]
    rows = 128 if name == "tiny" else 192
    d = _seq_fp32_h_distance(cfg, rows=rows, toks=8, experts=2)
    print(f"{name}: max |h32 - h| = 2**{np.log2(d):.2f} of the block max", flush=True)
    assert d <= oracle.moe.DECISION_RADIUS / 4


def test_decision_margin():
    """The margin is the distance to the nearest rounding midpoint (or block
    exponent boundary) over the block maximum; it is within the radius exactly
    where the band is nonzero on the grid cases."""
    h = np.zeros((1, 32))
    h[0, :5] = [1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -13, 1.0, 3.0 + 2.0 ** -7, 4.0]
    m = oracle.h_decision_margin(h, a8=False)
    # midpoint; 2**-13 from it; on the grid (half a step 2**-8 from the
    # midpoints); 3 + 2**-7 is the midpoint of 3 and 3 + 2**-6; the maximum 4
    # sits on the grid, half a step 2**-6 from the midpoints
    assert m[0, 0] == 0.0 and m[0, 1] == 2.0 ** -15 and m[0, 2] == 2.0 ** -10
    assert m[0, 3] == 0.0 and m[0, 4] == 2.0 ** -6 / 4
    b = oracle.h_decision_band(h, a8=False)
    assert np.array_equal(b != 0, m <= oracle.moe.DECISION_RADIUS)
    # E4M3, block max 300 (e = 0): 1 + 2**-4 is a midpoint; 2.3 is 0.075 from
    # the midpoint 2.375 of 2.25 and 2.5; 300 lies 4 from the midpoint 304 of
    # 288 and 320 (its
    # exponent boundaries 224 and 448 are farther)
    blk = np.zeros((1, 32))
    blk[0, :3] = [300.0, 1.0 + 2.0 ** -4, 2.3]
    m = oracle.h_decision_margin(blk, a8=True)
    assert m[0, 1] == 0.0
    assert np.isclose(m[0, 2], 0.075 / 300, rtol=1e-12)
    assert m[0, 0] == 4.0 / 300
    # a block maximum on the exponent boundary: every element has margin 0
    blk[0, 0] = 448.0
    assert np.all(oracle.h_decision_margin(blk, a8=True)[0] == 0.0)
    # A4: block max 1.4 (e = -2: scaled 5.6), scaled 1.25 is a midpoint
    h4 = np.zeros((1, 32))
    h4[0, :2] = [1.4, 1.25 * 0.25]
    m4 = oracle.h_decision_margin(h4, False, a4=True)
    assert m4[0, 1] == 0.0 and m4[0, 0] > 0
