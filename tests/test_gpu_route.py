"""Routing on the GPU vs the oracle: bit-exact counts, offsets, the stable
per-expert order of assignments and its inverse, dropped out-of-range ids."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import oracle
import synth
from helpers import require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", 32, 8, 2, "softmax_topk", False),
    ("decode", 64, 256, 8, "softmax_topk", False),
    ("decode32", 256, 256, 8, "softmax_topk", False),
    ("prefill_zipf", 8192, 256, 8, "zipf", False),
    ("odd", 7, 5, 3, "softmax_topk", False),
    ("e512", 100, 512, 4, "softmax_topk", False),
    ("single", 1, 1, 1, "softmax_topk", False),
    ("invalid_ids", 300, 16, 4, "softmax_topk", True),
    # more than 8192 assignments: the multi-workgroup form (chunks of 4096,
    # a ragged last chunk)
    ("multi_invalid", 3000, 64, 4, "softmax_topk", True),
    ("multi_e512", 2100, 512, 8, "zipf", False),
]


@pytest.mark.parametrize("name,T,E,k,routing,invalid", CASES, ids=[c[0] for c in CASES])
def test_route_bit_exact(name, T, E, k, routing, invalid):
    require_gpu()
    print(f"route case {name}", flush=True)
    cfg = synth.variant(synth.CONFIGS["tiny"], T=T, E=E, k=k, routing=routing, seed=11)
    ids, _ = synth.make_routing(cfg)
    if invalid:
        rng = np.random.default_rng(5)
        bad = rng.random(ids.shape) < 0.1
        ids = np.where(bad, rng.choice([-1, E, E + 7, -100], size=ids.shape), ids).astype(np.int32)
    p = moe.make_problem(T, E, k, 512, 512, 16)
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    c, o, sa, so = moe.route(p, torch.from_numpy(ids).cuda(), workspace=ws)
    torch.cuda.synchronize()
    rc, ro, rsa, rso = oracle.route(ids, E)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(sa.cpu().numpy(), rsa)
    assert np.array_equal(so.cpu().numpy(), rso)
    assert moe.dropped_assignments(ws) == int(np.sum((ids < 0) | (ids >= E)))
