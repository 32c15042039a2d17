"""Group16 -> group32 requantisation on the GPU vs the oracle, bit for bit:
random tensors, ragged sizes, ties, zero blocks, negative and absent global
scales, in-place use, and the full GLM-shaped layer (sampled)."""

import os

import numpy as np
import pytest
import torch

import block_scaled_fp4_topk_amd as moe
import oracle
import synth
from helpers import require_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, E, N, K, lo=-10.0, hi=-3.0):
    src = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = np.exp2(rng.uniform(lo, hi, size=(E, N, K // 16))).astype(np.float32)
    sf = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    gs = rng.uniform(0.5, 2.0, size=E).astype(np.float32)
    return src, sf, gs


def _gpu(src, sf, gs, inplace=False):
    s = torch.from_numpy(src).cuda()
    f = torch.from_numpy(sf).cuda()
    g = None if gs is None else torch.from_numpy(gs).cuda()
    d, dsf = moe.requant_gran_k(s, f, g, dst=s if inplace else None)
    torch.cuda.synchronize()
    return d.cpu().numpy(), dsf.cpu().numpy()


@pytest.mark.parametrize("E,N,K", [(3, 16, 512), (3, 5, 96), (1, 1, 32), (2, 33, 2080)])
def test_random_bit_exact(E, N, K):
    require_gpu()
    print(f"requant random E={E} N={N} K={K}", flush=True)
    rng = np.random.default_rng(E * 1000 + N)
    src, sf, gs = _rand(rng, E, N, K)
    d, dsf = _gpu(src, sf, gs)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, gs)
    assert np.array_equal(dsf, rdsf)
    assert np.array_equal(d, rd)


def test_no_global_negative_global_inplace():
    require_gpu()
    rng = np.random.default_rng(7)
    src, sf, gs = _rand(rng, 4, 32, 256)
    d, dsf = _gpu(src, sf, None)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, None)
    assert np.array_equal(d, rd) and np.array_equal(dsf, rdsf)
    gneg = -gs
    d, dsf = _gpu(src, sf, gneg)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, gneg)
    assert np.array_equal(d, rd) and np.array_equal(dsf, rdsf)
    d, dsf = _gpu(src.copy(), sf, gs, inplace=True)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, gs)
    assert np.array_equal(d, rd) and np.array_equal(dsf, rdsf)


def test_golden_blocks_on_gpu():
    require_gpu()
    rows = []
    with open(os.path.join(GOLDEN, "requant_blocks.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if ln:
                rows.append([x.strip() for x in ln.split("|")])
    for name, gs, s, src, exp, byte in rows:
        c = np.array([int(ch, 16) for ch in src], np.uint8)
        packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, None, :]
        sf = np.array([int(v, 16) for v in s.split()], np.uint8)[None, None, :]
        g = np.array([int(gs, 16)], np.uint32).view(np.float32)
        d, dsf = _gpu(packed, sf, g)
        got = np.empty(32, np.uint8)
        got[0::2] = d[0, 0] & 15
        got[1::2] = d[0, 0] >> 4
        assert "".join(f"{v:x}" for v in got) == exp, name
        assert int(dsf[0, 0, 0]) == int(byte), name


def test_tie_heavy_blocks():
    require_gpu()
    rng = np.random.default_rng(9)
    E, N, K = 2, 512, 256
    mags = rng.integers(0, 8, size=(E, N, K))
    mags = np.where(rng.random((E, N, K)) < 0.3, mags, 0)
    c = (mags | (rng.integers(0, 2, size=(E, N, K)) << 3)).astype(np.uint8)
    src = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    sf = rng.choice(np.array([0x38, 0x30, 0x40, 0x42, 0x46, 0x4A, 0x01, 0x7E], np.uint8),
                    size=(E, N, K // 16))
    gs = np.array([1.0, 1.5], np.float32)
    d, dsf = _gpu(src, sf, gs)
    rd, rdsf = oracle.requant_g16_to_g32(src, sf, gs)
    assert np.array_equal(d, rd) and np.array_equal(dsf, rdsf)


def test_full_layer_sampled():
    """The whole GLM-shaped layer (w13 [256, 4096, 6144], w2 [256, 6144, 2048])
    in one call per tensor, as the benchmark runs it; every scale byte and code
    of 3 whole experts plus 2 random rows of every expert checked bit-exactly."""
    require_gpu()
    cfg = synth.REQUANT_CONFIGS["requant"]
    rng = np.random.default_rng(3)
    for which in range(2):
        print(f"requant full layer tensor {which}: generating", flush=True)
        src, sf, gs = synth.make_requant_tensor(cfg, which)
        print("  running on GPU", flush=True)
        d, dsf = _gpu(src, sf, gs)
        E, N, _ = src.shape
        for e in (0, 129, E - 1):
            rd, rdsf = oracle.requant_g16_to_g32(src[e:e + 1], sf[e:e + 1], gs[e:e + 1])
            assert np.array_equal(dsf[e], rdsf[0]) and np.array_equal(d[e], rd[0]), f"expert {e}"
        rows = rng.integers(0, N, size=(E, 2))
        for e in range(E):
            rd, rdsf = oracle.requant_g16_to_g32(src[e:e + 1, rows[e]], sf[e:e + 1, rows[e]],
                                                 gs[e:e + 1])
            assert np.array_equal(d[e, rows[e]], rd[0]) and np.array_equal(dsf[e, rows[e]], rdsf[0])
        print("  ok", flush=True)
