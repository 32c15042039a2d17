"""The requantisation arithmetic of the HIP kernel (requant_core.h), built for
the host with g++ (-ffp-contract=off), must agree bit for bit with the FP64
oracle, including hand-built ties, exact boundaries, zero blocks, negative
global scales and the pages' scale ranges -- both the direct form and the
table-driven form the kernel runs (whose E2M1 encoder is the hardware
instruction on the GPU and its host equivalent here)."""

import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "requant_core_cpu.cpp")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("rqcore")
    out = str(d / "rqcore")
    r = subprocess.run(["g++", "-O2", "-ffp-contract=off", "-std=c++17", SRC, "-o", out],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr)
    return out


@pytest.fixture(params=["direct", "table"])
def variant(request):
    return request.param


def run_core(exe, codes, sf, gs, variant="direct"):
    """codes [n, 16] u8, sf [n, 2] u8, gs [n] f32 -> (codes [n,16], byte [n])."""
    n = codes.shape[0]
    rec = np.zeros((n, 22), np.uint8)
    rec[:, :16] = codes
    rec[:, 16:18] = sf
    rec[:, 18:22] = np.asarray(gs, np.float32).view(np.uint8).reshape(n, 4)
    with tempfile.TemporaryDirectory() as d:
        fi, fo = os.path.join(d, "in"), os.path.join(d, "out")
        rec.tofile(fi)
        subprocess.run([exe, fi, fo] + (["tab"] if variant == "table" else []), check=True)
        out = np.fromfile(fo, np.uint8).reshape(n, 17)
    return out[:, :16], out[:, 16]


def check(exe, codes, sf, gs, variant="direct"):
    got_c, got_b = run_core(exe, codes, sf, gs, variant)
    n = codes.shape[0]
    for g in np.unique(gs):
        idx = np.flatnonzero(gs == g)
        exp_c, exp_b = oracle.requant_g16_to_g32(codes[idx][None], sf[idx][None],
                                                 np.array([g], np.float32))
        bad = np.flatnonzero((got_b[idx] != exp_b[0, :, 0]) | np.any(got_c[idx] != exp_c[0], axis=1))
        assert bad.size == 0, (f"{bad.size}/{idx.size} blocks differ, first: codes "
                               f"{codes[idx[bad[0]]]} sf {sf[idx[bad[0]]]} gs {g}")
    return n


def test_random_blocks(exe, variant):
    rng = np.random.default_rng(0)
    n = 200000
    codes = rng.integers(0, 256, size=(n, 16), dtype=np.uint8)
    s = np.exp2(rng.uniform(-10, -3, size=(n, 2))).astype(np.float32)
    sf = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    gs = rng.choice(rng.uniform(0.5, 2.0, size=7).astype(np.float32), size=n)
    check(exe, codes, sf, gs, variant)


def test_all_scale_pairs_and_special_globals(exe, variant):
    rng = np.random.default_rng(1)
    b = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], np.uint8)
    sf = np.stack(np.meshgrid(b, b), -1).reshape(-1, 2)
    n = sf.shape[0]
    codes = rng.integers(0, 256, size=(n, 16), dtype=np.uint8)
    for g in [1.0, 0.5, 1.5, 1.0 + 2.0 ** -23, 1.9999999, -1.25, 3.0 / 7.0]:
        check(exe, codes, sf, np.full(n, g, np.float32), variant)


def test_ties_and_sparse_blocks(exe, variant):
    """Blocks with few distinct magnitudes and power-of-two scales land on
    E2M1 midpoints often."""
    rng = np.random.default_rng(2)
    n = 100000
    mags = rng.integers(0, 8, size=(n, 32))
    keep = rng.random((n, 32)) < rng.random((n, 1))
    mags = np.where(keep, mags, 0)
    sign = rng.integers(0, 2, size=(n, 32)) << 3
    c = (mags | sign).astype(np.uint8)
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    sfv = rng.choice(np.array([0x38, 0x30, 0x40, 0x42, 0x46, 0x4A, 0x34, 0x3C, 0x01, 0x7E], np.uint8),
                     size=(n, 2))
    gs = rng.choice(np.array([1.0, 0.75, 1.5, 2.0, 1.25], np.float32), size=n)
    check(exe, codes, sfv, gs, variant)
