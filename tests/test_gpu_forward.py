"""MoE forward on the GPU vs the FP64 oracle, within the stated bound
(max |err| <= 2e-2 rms(ref), mean relative error <= 5e-3): every supported
(activation, scale) combination, both w13 row orders, ragged tiles, the
multi-tile prefill path, duplicate and out-of-range expert ids, bitwise
determinism, and the full-size workloads on sampled tokens."""

import numpy as np
import pytest
import torch

import oracle
from oracle.moe import decode_activations
import synth
from helpers import check_bound, check_forward, check_h, forward_ws, gpu_forward, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def ref_forward(inp, order="gate_up", tokens=None, out_cols=None, return_h=False):
    """(FP64 output, decision band[, {slot: (h, hhat)}]) of the oracle."""
    return oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                              inp.w2, inp.w2_sf, inp.w2_gs, inp.cfg.gran, x_sf=inp.x_sf,
                              w13_order=order, tokens=tokens, out_cols=out_cols,
                              return_band=True, return_h=return_h)


def combos(base):
    return [
        synth.variant(base, gran=16, act="bf16", global_scale="uniform"),
        synth.variant(base, gran=32, act="bf16", global_scale="none"),
        synth.variant(base, gran=32, act="bf16", global_scale="uniform"),
        synth.variant(base, gran=32, act="fp8", global_scale="none"),
    ]


def _id(c):
    return f"{c.act}-g{c.gran}-{c.global_scale}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-I{c.I}"


SMALL = (combos(synth.CONFIGS["tiny"])
         + combos(synth.variant(synth.CONFIGS["tiny"], T=16, E=32, k=4, H=1024, I=512, seed=21))
         + combos(synth.variant(synth.CONFIGS["tiny"], T=13, E=6, k=3, H=768, I=256, seed=22))
         + combos(synth.variant(synth.CONFIGS["tiny"], T=300, E=8, k=2, H=512, I=512, seed=23,
                                routing="zipf"))
         # prefill regime: several 128-row tiles per expert, ragged tails,
         # several row blocks, K = 1536 (a partial last scale group) and
         # K = 1024 (one whole group)
         + combos(synth.variant(synth.CONFIGS["tiny"], T=400, E=4, k=2, H=1536, I=1024, seed=24,
                                routing="zipf")))


# decode regime (16-row tiles) with long K: several scale groups per row, a
# one-chunk last group (FC1 group16: 17 chunks = 8 + 8 + 1; FC2 group16: 9
# = 8 + 1), and scale rows that are not 16-byte multiples (group32: 136 and
# 72 bytes)
DECODE_LONG_K = combos(synth.variant(synth.CONFIGS["tiny"], T=16, E=8, k=4, H=4352, I=2304, seed=25))
# the other lengths of a last scale group (group16: 8 chunks of 256 per
# group, the group's chunks unrolled; FC1 with its paired buffers): FC1 13 =
# 8 + 5 and 14 = 8 + 6 chunks, FC2 7 and 6
DECODE_GROUP_TAILS = [
    synth.variant(synth.CONFIGS["tiny"], T=16, E=8, k=4, H=3328, I=1792, seed=26, gran=16, act="bf16",
                  global_scale="uniform"),
    synth.variant(synth.CONFIGS["tiny"], T=12, E=8, k=3, H=3584, I=1536, seed=30, gran=16, act="bf16",
                  global_scale="none"),
]
# the smallest shapes the forward takes (H = I = 256: one 256-K chunk in FC1
# and FC2), on the 16-row decode tiles and (T = 300 over 2 experts) on the
# 64-row tiles
SMALLEST = (combos(synth.variant(synth.CONFIGS["tiny"], T=20, E=4, k=2, H=256, I=256, seed=27))
            + combos(synth.variant(synth.CONFIGS["tiny"], T=300, E=2, k=2, H=256, I=256, seed=28)))
SMALL = SMALL + DECODE_LONG_K + DECODE_GROUP_TAILS + SMALLEST


@pytest.mark.parametrize("cfg", SMALL, ids=[_id(c) for c in SMALL])
def test_forward_small(cfg):
    require_gpu()
    print("forward", _id(cfg), flush=True)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    for order in ("gate_up", "up_gate"):
        ref, band, hrows = ref_forward(inp, order, return_h=True)
        check_forward(inp, d, ref, f"{_id(cfg)} {order}", order, band, hrows)


# FP8 activations (caller-quantised, or bf16 x the library quantises) on the
# 64-row tiles: more than 16 assignments per active expert with H or I not a
# multiple of 512 (the prefill GEMM's row blocks), several tiles per expert,
# ragged tails, several weight-row blocks
MID_FP8 = [
    synth.variant(synth.CONFIGS["tiny"], T=300, E=4, k=2, H=768, I=512, seed=27, gran=32, act="fp8",
                  global_scale="none", routing="zipf"),
    synth.variant(synth.CONFIGS["tiny"], T=300, E=4, k=2, H=1024, I=1280, seed=28, gran=32, act="fp8",
                  global_scale="uniform"),
    synth.variant(synth.CONFIGS["tiny"], T=300, E=4, k=2, H=768, I=1280, seed=29, gran=32, act="bf16q",
                  global_scale="none", routing="zipf"),
]


@pytest.mark.parametrize("cfg", MID_FP8, ids=[_id(c) for c in MID_FP8])
def test_forward_fp8_64row_tiles(cfg):
    require_gpu()
    print("forward 64-row FP8 tiles", _id(cfg), flush=True)
    inp = synth.make_moe_inputs(cfg)
    active = np.unique(inp.topk_ids).size
    # the dispatch rule of the forward for this kernel
    assert inp.topk_ids.size / active > 16 and (cfg.H % 512 or cfg.I % 512)
    d = to_dev(inp)
    quant = cfg.act == "bf16q"
    if quant:
        # the oracle runs on its own FP8 quantisation of x (the library's is
        # bit-exact with it, test_gpu_quant)
        _, codes, sf = oracle.quantize_h_a8(decode_activations(inp.x))
        rinp = synth.MoEInputs(cfg, codes, sf, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                               inp.w2, inp.w2_sf, inp.w2_gs)
    else:
        rinp = inp
    for order in ("gate_up", "up_gate"):
        ref, band, hrows = ref_forward(rinp, order, return_h=True)
        check_forward(inp, d, ref, f"{_id(cfg)} {order}", order, band, hrows, quantize_x=quant)


def test_duplicate_and_dropped_ids():
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], T=24, E=8, k=3, seed=31)
    inp = synth.make_moe_inputs(cfg)
    ids = inp.topk_ids.copy()
    ids[0, 1] = ids[0, 0]          # same expert twice in one token
    ids[1, 2] = -1                 # dropped
    ids[2, 0] = 8                  # dropped
    ids[3] = ids[3, 0]             # all three picks the same expert
    inp.topk_ids = ids
    d = to_dev(inp)
    ref, band, hrows = ref_forward(inp, return_h=True)
    check_forward(inp, d, ref, "dup+dropped", band=band, hrows=hrows)


def test_deterministic():
    require_gpu()
    for base in (synth.variant(synth.CONFIGS["tiny"], T=64, E=32, k=8, H=1024, I=512, seed=41),
                 synth.variant(synth.CONFIGS["tiny"], T=512, E=8, k=2, H=512, I=512, seed=42,
                               routing="zipf", gran=32, act="fp8", global_scale="none")):
        inp = synth.make_moe_inputs(base)
        d = to_dev(inp)
        a = gpu_forward(inp, d, out_dtype=torch.float32).clone()
        b = gpu_forward(inp, d, out_dtype=torch.float32).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        print(f"generating full {name} inputs", flush=True)
        inp = synth.make_moe_inputs(synth.CONFIGS[name])
        _FULL.clear()
        _FULL[name] = (inp, to_dev(inp))
    return _FULL[name]


@pytest.mark.parametrize("name", ["decode16", "decode32", "prefill32"])
def test_full_size_sampled(name):
    """The full workload in the launch configuration the benchmark times;
    the oracle computes a sample of tokens (including one routed to the most
    loaded expert) over a sample of output columns."""
    require_gpu()
    inp, d = full_inputs(name)
    print(f"{name}: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d)
    b16 = gpu_forward(inp, d)
    torch.cuda.synchronize()
    assert torch.equal(out.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))
    rng = np.random.default_rng(0)
    counts = np.bincount(inp.topk_ids.ravel(), minlength=inp.cfg.E)
    heavy = int(np.flatnonzero((inp.topk_ids == counts.argmax()).any(axis=1))[0])
    tokens = sorted({0, inp.cfg.T - 1, heavy, int(rng.integers(inp.cfg.T))})
    cols = np.sort(rng.choice(inp.cfg.H, size=768, replace=False))
    print(f"{name}: oracle on tokens {tokens}", flush=True)
    ref, band, hrows = ref_forward(inp, tokens=tokens, out_cols=cols, return_h=True)
    check_h(ws, p, hrows, f"{name} sampled")
    got = out[tokens][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_bound(got, ref, f"{name} sampled", band)


def test_full_prefill_ragged_tiles_sampled():
    """prefill32 in the benchmark's launch configuration, sampled where the
    128-row expert tiles are partly filled: for 16 experts spread over the
    Zipf load range (lightest to heaviest), the token of the expert's last
    assignment (in its last, ragged tile), plus the first and last tokens;
    512 sampled output columns."""
    require_gpu()
    inp, d = full_inputs("prefill32")
    cfg = inp.cfg
    print("prefill32 ragged tiles: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d)
    torch.cuda.synchronize()
    flat = inp.topk_ids.ravel()
    counts = np.bincount(flat, minlength=cfg.E)
    by_load = np.argsort(counts, kind="stable")
    active = by_load[counts[by_load] > 0]
    picked = active[np.linspace(0, active.size - 1, 16).round().astype(int)]
    tokens = {0, cfg.T - 1}
    for e in picked:
        tokens.add(int(np.flatnonzero(flat == e)[-1] // cfg.k))
    tokens = sorted(tokens)
    print(f"prefill32 ragged tiles: experts {picked.tolist()} with {counts[picked].tolist()} assignments "
          f"(last tile rows {(counts[picked] - 1) % 128 + 1}); oracle on tokens {tokens}", flush=True)
    cols = np.sort(np.random.default_rng(5).choice(cfg.H, size=512, replace=False))
    ref, band, hrows = ref_forward(inp, tokens=tokens, out_cols=cols, return_h=True)
    check_h(ws, p, hrows, "prefill32 ragged tiles sampled")
    got = out[tokens][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_bound(got, ref, "prefill32 ragged tiles sampled", band)


def test_many_items_per_workgroup():
    """A prefill batch large enough that each persistent GEMM workgroup walks
    more than one batch of 64 work-item descriptors (FC2: 1536 expert tiles x
    12 row blocks over one workgroup per CU), checked on sampled tokens."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["prefill32"], name="prefill_many_items", T=24576, E=32, I=512,
                        routing="softmax_topk", seed=26, weight_seed=None)
    inp = synth.make_moe_inputs(cfg)
    d = to_dev(inp)
    print(f"many items: T={cfg.T} E={cfg.E} H={cfg.H} I={cfg.I}: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    tokens = sorted({0, cfg.T - 1, int(rng.integers(cfg.T)), int(rng.integers(cfg.T))})
    cols = np.sort(rng.choice(cfg.H, size=768, replace=False))
    print(f"many items: oracle on tokens {tokens}", flush=True)
    ref, band, hrows = ref_forward(inp, tokens=tokens, out_cols=cols, return_h=True)
    check_h(ws, p, hrows, "many items sampled")
    got = out[tokens][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_bound(got, ref, "many items sampled", band)


@pytest.mark.parametrize("gran,act", [(16, "bf16"), (32, "fp8")])
def test_decode_largest_batch(gran, act):
    """The largest decode-shaped batch: 8192 assignments over 512 experts
    (16 per active expert, the most that still takes 16-row tiles, and the
    most the single-workgroup route takes); for bf16 x on group16 weights the
    route launch's 256 extra workgroups write the fp16 rows (4 each) that FC1
    copies to LDS.  The oracle checks a sample of tokens spread over the
    batch on every output column."""
    require_gpu()
    cfg = synth.variant(synth.CONFIGS["tiny"], name="decode_largest", T=1024, E=512, k=8, H=512, I=256,
                        gran=gran, act=act, global_scale="uniform" if gran == 16 else "none", seed=43)
    inp = synth.make_moe_inputs(cfg)
    counts = np.bincount(inp.topk_ids.ravel(), minlength=cfg.E)
    assert cfg.T * cfg.k == 8192 and cfg.T * cfg.k / np.count_nonzero(counts) <= 16
    d = to_dev(inp)
    print(f"decode largest batch {act}-g{gran}: T={cfg.T} E={cfg.E} k={cfg.k}, "
          f"{np.count_nonzero(counts)} active experts, up to {counts.max()} rows: running on GPU", flush=True)
    out, ws, p = forward_ws(inp, d)
    torch.cuda.synchronize()
    tokens = sorted({0, 1, 3, 4, 255, 256, cfg.T // 2, cfg.T - 2, cfg.T - 1}
                    | set(np.random.default_rng(7).choice(cfg.T, size=23, replace=False).tolist()))
    ref, band, hrows = ref_forward(inp, tokens=tokens, return_h=True)
    check_h(ws, p, hrows, f"decode largest batch {act}-g{gran}")
    got = out[tokens].cpu().numpy().astype(np.float64)
    check_bound(got, ref, f"decode largest batch {act}-g{gran}", band)
