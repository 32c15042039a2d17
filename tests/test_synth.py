"""Input generator: deterministic per seed, per-expert streams independent of
how many experts are drawn, shapes and value ranges as documented."""

import numpy as np

import oracle
import synth


def test_deterministic_and_per_expert():
    cfg = synth.variant(synth.CONFIGS["decode16"], T=4, E=6, H=256, I=128)
    a = synth.make_moe_inputs(cfg)
    b = synth.make_moe_inputs(cfg)
    for f in ("x", "topk_ids", "topk_w", "w13", "w13_sf", "w13_gs", "w2", "w2_sf", "w2_gs"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c, s = synth.make_fp4_tensor(cfg.seed, synth._S_W13, 3, 256, 256, 16)
    assert np.array_equal(c, a.w13[3]) and np.array_equal(s, a.w13_sf[3])


def test_ranges():
    cfg = synth.variant(synth.CONFIGS["decode16"], T=8, E=16, H=512, I=256)
    a = synth.make_moe_inputs(cfg)
    s = oracle.e4m3_decode(a.w13_sf)
    assert s.min() >= 2.0 ** -10 and s.max() <= 2.0 ** -3
    assert np.all((a.w13_gs >= 0.5) & (a.w13_gs <= 2.0))
    ids = a.topk_ids
    assert ids.shape == (8, 8) and all(len(set(r)) == 8 for r in ids)
    c32 = synth.variant(synth.CONFIGS["decode32"], T=8, E=16, H=512, I=256)
    b = synth.make_moe_inputs(c32)
    assert b.w13_sf.min() >= 117 and b.w13_sf.max() <= 125 and b.w13_gs is None
    assert b.x_sf.min() >= 119 and b.x_sf.max() <= 121
    assert np.all(np.isfinite(oracle.e4m3_decode(b.x)))


def test_zipf_skew():
    cfg = synth.variant(synth.CONFIGS["prefill32"], T=2048, H=64, I=64, E=256)
    ids, w = synth.make_routing(cfg)
    n = np.bincount(ids.ravel(), minlength=256)
    assert n.sum() == 2048 * 8 and n.max() > 10 * np.median(n)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
