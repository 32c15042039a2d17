"""Edge cases of the MoE forward on the GPU vs the FP64 oracle: an empty
batch, a single token, every token on every expert (k = E), one expert
taking most of the batch in the 16-row-tile regime (several full tiles of
one expert and a ragged one), and tokens of very different magnitudes in one
expert tile (the per-token staging scales of x and the per-assignment
scales of h must be applied row by row)."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import oracle
import synth
from helpers import check_forward, gpu_forward, require_gpu, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [
    dict(gran=16, act="bf16", global_scale="uniform"),
    dict(gran=32, act="bf16", global_scale="none"),
    dict(gran=32, act="fp8", global_scale="none"),
]
FMT_IDS = ["bf16-g16", "bf16-g32", "fp8-g32"]


def _ref(inp):
    return oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                              inp.w2, inp.w2_sf, inp.w2_gs, inp.cfg.gran, x_sf=inp.x_sf,
                              return_band=True, return_h=True)


def _check(inp, what):
    d = to_dev(inp)
    ref, band, hrows = _ref(inp)
    check_forward(inp, d, ref, what, band=band, hrows=hrows)


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_empty_batch(fmt):
    require_gpu()
    print("empty batch", fmt, flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=1, seed=61, **fmt)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    for k in ("x", "topk_ids", "topk_w") + (("x_sf",) if d["x_sf"] is not None else ()):
        d[k] = d[k][:0]
    out = gpu_forward(inp, d)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, cfg.H)


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_single_token(fmt):
    require_gpu()
    print("single token", fmt, flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=1, E=4, k=2, seed=62, **fmt)
    _check(synth.make_moe_inputs(cfg), "single token")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_every_expert(fmt):
    require_gpu()
    print("k = E", fmt, flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=8, E=4, k=4, seed=63, **fmt)
    _check(synth.make_moe_inputs(cfg), "k = E")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_one_heavy_expert(fmt):
    """40 tokens all pick expert 3 first: 40 assignments of one expert on
    16-row tiles (16 + 16 + 8) while the batch stays in that regime."""
    require_gpu()
    print("one heavy expert", fmt, flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=40, E=8, k=2, seed=64, **fmt)
    inp = synth.make_moe_inputs(cfg)
    rng = np.random.default_rng(640)
    ids = np.empty((cfg.T, 2), np.int32)
    ids[:, 0] = 3
    ids[:, 1] = rng.choice([0, 1, 2, 4, 5, 6, 7], size=cfg.T)
    inp.topk_ids = ids
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert counts[3] == 40 and ids.size / np.count_nonzero(counts) <= 16
    _check(inp, "one heavy expert")


def _scale_bf16_rows(bits, exps):
    """bf16 bit rows times 2**exps[row] (exact: the values stay normal)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    f = f * np.exp2(np.asarray(exps, np.float64))[:, None]
    out = (f.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    back = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, f)
    return out


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_row_magnitudes(fmt):
    """Tokens scaled by 2**-40 .. 2**20 share expert tiles: the per-token
    fp16 staging exponent of x (group16), the per-assignment one of h, and
    the per-32 activation scales (FP8) must follow each row."""
    require_gpu()
    print("row magnitudes", fmt, flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=16, E=4, k=2, seed=65, **fmt)
    inp = synth.make_moe_inputs(cfg)
    exps = np.array([-40, -20, 0, 10, 20, -8, 4, 16] * 2)[: cfg.T]
    if inp.x_sf is None:
        inp.x = _scale_bf16_rows(inp.x, exps)
    else:
        sf = inp.x_sf.astype(np.int32) + exps[:, None]
        assert sf.min() >= 1 and sf.max() <= 254
        inp.x_sf = sf.astype(np.uint8)
    _check(inp, "row magnitudes")


def test_dropped_only_token():
    """A token whose every pick is out of range gets a zero output row."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], T=6, E=4, k=2, seed=66)
    inp = synth.make_moe_inputs(cfg)
    ids = inp.topk_ids.copy()
    ids[2] = [-1, 9]
    inp.topk_ids = ids
    d = to_dev(inp)
    out = gpu_forward(inp, d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[2]).item() == 0
    ref, band, hrows = _ref(inp)
    check_forward(inp, d, ref, "dropped-only token", band=band, hrows=hrows)
    ws = torch.empty(moe.workspace_bytes(moe.make_problem(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.gran)),
                     dtype=torch.uint8, device="cuda")
    gpu_forward(inp, d, workspace=ws)
    torch.cuda.synchronize()
    assert moe.dropped_assignments(ws) == 2
