"""Pins of the oracle's number formats against things other than itself:
the pages' printed constants (golden fixtures), torch's library decoders and
casts, closed forms and brute force."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_decode, rne_bf16, rne_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#")[0].strip() for ln in f if ln.split("#")[0].strip()]


def test_e2m1_table_golden():
    rows = [r.split() for r in _rows("e2m1_values.txt")]
    codes = np.array([int(c) for c, _ in rows])
    vals = np.array([float(v) for _, v in rows])
    got = oracle.e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))  # -0.0 for code 8


@pytest.mark.parametrize("dtype,sh_exp,sh_man", [(torch.bfloat16, 7, 6), (torch.float16, 10, 9)])
def test_e2m1_bias_identity(dtype, sh_exp, sh_man):
    """Placing s e1 e0 m into a 16-bit float's sign / two low exponent bits /
    top mantissa bit and decoding it with torch gives the E2M1 value times
    2**-bias, bias = 2**(t-1) - 2**(2-1) as printed on the pages."""
    consts = {r.split()[0]: (int(r.split()[1]), int(r.split()[2])) for r in _rows("bias_constants.txt")}
    t, bias = consts["bfloat16" if dtype == torch.bfloat16 else "float16"]
    assert bias == 2 ** (t - 1) - 2 ** (2 - 1)
    c = np.arange(16)
    bits = ((c >> 3) << 15) | (((c >> 1) & 3) << sh_exp) | ((c & 1) << sh_man)
    v = torch.from_numpy(bits.astype(np.int16)).view(dtype).double().numpy()
    assert np.array_equal(v * 2.0 ** bias, oracle.e2m1_decode(c))


def test_e4m3_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_decode(b)
    assert np.array_equal(got, ref, equal_nan=True)
    assert np.nanmax(got) == 448.0  # the E4M3 bound used by the pages' scale boost


def test_ue8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    got = oracle.ue8m0_decode(b)
    assert np.array_equal(got, ref, equal_nan=True)


def test_nibble_order_golden():
    for r in _rows("nibble_order.txt"):
        bs, cs = r.split("|")
        by = np.array([int(x, 16) for x in bs.split()], dtype=np.uint8)
        codes = np.array([int(x, 16) for x in cs.split()], dtype=np.uint8)
        assert np.array_equal(oracle.unpack_fp4(by), codes)
        # the pages' reading: int32 little-endian word, element pos at shift 4*pos
        word = int(by.view("<u4")[0])
        assert [(word >> (4 * p)) & 0xF for p in range(8)] == list(codes)
        assert np.array_equal(oracle.pack_fp4(codes), by)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(0)
    p = rng.integers(0, 256, size=(7, 48), dtype=np.uint8)
    assert np.array_equal(oracle.pack_fp4(oracle.unpack_fp4(p)), p)


def _brute_e2m1(x):
    """argmin |x - g| over the E2M1 magnitudes; ties to the even code."""
    g = oracle.E2M1_VALUES
    out = []
    for xv in x:
        d = np.abs(g - min(xv, 6.0))
        best = np.flatnonzero(d == d.min())
        out.append(best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0])
    return np.array(out, dtype=np.uint8)


def test_rne_e2m1_brute_force():
    rng = np.random.default_rng(1)
    x = np.concatenate([np.arange(0, 6 * 256 + 1) / 256.0, rng.uniform(0, 6, 4000),
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0]])
    assert np.array_equal(oracle.rne_e2m1_magnitude(x), _brute_e2m1(x))


def test_rne_e2m1_ties():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    # values 0, 1, 1, 2, 2, 4, 4 -> codes 0, 2, 2, 4, 4, 6, 6
    assert list(oracle.rne_e2m1_magnitude(ties)) == [0, 2, 2, 4, 4, 6, 6]


def test_rne_e4m3_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.standard_normal(20000) * 100.0,
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),
                        oracle.e4m3_decode(np.arange(0x7F)),   # grid points
                        (oracle.e4m3_decode(np.arange(0x7E)) + oracle.e4m3_decode(np.arange(1, 0x7F))) / 2,
                        [0.0, -0.0, 448.0, -448.0]]).astype(np.float32).astype(np.float64)
    y = np.clip(y, -448, 448)
    ref = torch.from_numpy(y).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rne_e4m3(y), ref)


def test_rne_e4m3_single_rounding():
    # 1 + 2**-4 is the midpoint of 1 and 1.125; just above it must round up
    # even though an intermediate FP32 rounding would land on the tie.
    assert rne_e4m3(np.array([1 + 2.0 ** -4 + 2.0 ** -40]))[0] == 0x39
    assert rne_e4m3(np.array([1 + 2.0 ** -4]))[0] == 0x38


def test_rne_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.standard_normal(20000) * 1e3, rng.standard_normal(2000) * 1e-30,
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = rne_bf16(y.astype(np.float64))
    assert np.array_equal(got, bf16_bits_decode(ref))


def test_rne_bf16_single_rounding():
    # just above the midpoint 1 + 2**-8 -> rounds up to 1 + 2**-7
    assert rne_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    assert rne_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0


def test_dequant_closed_form():
    # code 7 (6.0) with E4M3 448 and global 2 -> 5376; code 1 with the smallest
    # E4M3 subnormal 2**-9 -> 2**-10; code 15 -> -6 * scale.
    packed = oracle.pack_fp4(np.array([[7] * 16 + [1] * 16, [15] * 16 + [0] * 16], dtype=np.uint8))
    sf = np.array([[0x7E, 0x01], [0x38, 0x38]], dtype=np.uint8)
    w = oracle.dequant_fp4(packed, sf, 16, "e4m3", gs=2.0)
    assert np.all(w[0, :16] == 5376.0)
    assert np.all(w[0, 16:] == 2.0 ** -10 * 2)
    assert np.all(w[1, :16] == -12.0)
    w32 = oracle.dequant_fp4(packed, np.array([[120], [127]], dtype=np.uint8), 32, "ue8m0")
    assert w32[0, 0] == 6 * 2.0 ** -7 and w32[0, 20] == 0.5 * 2.0 ** -7 and w32[1, 0] == -6.0
