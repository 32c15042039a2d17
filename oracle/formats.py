"""Number formats of the block-scaled FP4 path, decoded and encoded in FP64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Every decoder is written from the bit layout of the format, every encoder is
"round to nearest, ties to even" (RNE) onto the format's grid, computed on
exact FP64 values (a power-of-two rescale followed by ``numpy.rint``, which
rounds half to even).  Nothing here is blocked or reordered.

Sources:
  * FP4 E2M1 layout ``s e1 e0 m`` and its value set follow from the bias
    identity in [P3] ``_process_nvfp4_packed_global_scale``: placing the two
    exponent bits of an FP4 code into the low exponent bits of a 16-bit float
    makes it 2**(2**(t-1) - 2**(f-1)) times too small, t the target exponent
    width and f = 2 the FP4 exponent width.  The value table is the usual
    OCP MX E2M1 table {0, .5, 1, 1.5, 2, 3, 4, 6}.
  * Nibble order: [P3] ``_repack_4bit_no_perm`` / ``_repack_weight`` read a
    row of packed bytes as little-endian int32 words and take element ``pos``
    of a word at bit shift ``4*pos``; so within a byte the even K element sits
    in bits 0-3 and the odd one in bits 4-7.
  * E4M3 ("float8_e4m3fn", bias 7, no infinities, max 448): [P3]
    ``_nvfp4_compute_scale_factor`` (the 448 bound) and
    ``_process_nvfp4_packed_scales`` (the torch dtype).
  * UE8M0 ("float8_e8m0fnu", value 2**(b-127), 0xFF = NaN): [P3]
    ``_validate_e8m0_k32_scales``; [P1]/[P2] "UE8M0 runtime scales".
"""

from __future__ import annotations

import numpy as np

# E2M1 magnitudes indexed by the 3 low bits of a code (OCP MX E2M1 table).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (values 0..15) to FP64.

    Bit layout s e1 e0 m: exponent field e = (c >> 1) & 3 with bias 1,
    one mantissa bit; e == 0 is subnormal with value m/2.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, (e - 1).astype(np.int64)))
    return np.where(s == 1, -mag, mag)


def e4m3_decode(b) -> np.ndarray:
    """Decode E4M3 (fn variant) bytes to FP64: bias 7, subnormal m*2**-9,
    0x7F / 0xFF are NaN, no infinities; largest finite value 448."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def ue8m0_decode(b) -> np.ndarray:
    """Decode UE8M0 bytes (unsigned power of two, bias 127) to FP64; 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, (b - 127).astype(np.int64))
    return np.where(b == 255, np.nan, v)


def bf16_bits_decode(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to FP64 (exact)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def unpack_fp4(packed) -> np.ndarray:
    """[..., K/2] uint8 -> [..., K] codes; element 2j in the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_fp4(codes) -> np.ndarray:
    """[..., K] codes (0..15) -> [..., K/2] uint8, inverse of :func:`unpack_fp4`."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even to pack two FP4 codes per byte")
    return (c[..., 0::2] & 0x0F) | ((c[..., 1::2] & 0x0F) << 4)


def _rne_to_format(y: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round exact FP64 values to a binary float format with ``mant_bits``
    fraction bits and minimum normal exponent ``emin`` (unbounded above),
    ties to even.  The quantum of a value with floor(log2|y|) = E is
    2**(max(E, emin) - mant_bits); dividing by it is exact, ``rint`` rounds
    half to even, and multiplying back is exact."""
    y = np.asarray(y, dtype=np.float64)
    _, ex = np.frexp(y)  # y = f * 2**ex, f in [0.5, 1) -> floor(log2|y|) = ex - 1
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, e - mant_bits)
    return np.rint(y / q) * q


def rne_e2m1_magnitude(x) -> np.ndarray:
    """Round non-negative FP64 values onto the E2M1 grid, RNE, saturating at 6.

    Returns the 3-bit magnitude code (0..7).  The grid has quantum 0.5 on
    [0, 2), 1 on [2, 4) and 2 on [4, 6]; a tie goes to the even integer
    multiple of the quantum, which is the code whose last bit is 0.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or np.any(np.isnan(x)):
        raise ValueError("rne_e2m1_magnitude expects non-negative, non-NaN input")
    r = _rne_to_format(np.minimum(x, 6.0), mant_bits=1, emin=0)
    r = np.minimum(r, 6.0)
    return np.searchsorted(E2M1_VALUES, r).astype(np.uint8)


_E4M3_POS = e4m3_decode(np.arange(0x7F))  # finite non-negative values, bytes 0..126


def rne_e4m3(y) -> np.ndarray:
    """Encode FP64 values to E4M3 (fn) bytes with RNE; |y| above 448 saturates
    to 448.  The sign of zero is kept."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("rne_e4m3: NaN input")
    a = np.minimum(np.abs(y), 448.0)
    r = _rne_to_format(a, mant_bits=3, emin=-6)
    r = np.minimum(r, 448.0)
    mag = np.searchsorted(_E4M3_POS, r).astype(np.uint8)
    if not np.array_equal(_E4M3_POS[mag], r):
        raise AssertionError("rne_e4m3: rounded value not on the E4M3 grid")
    return np.where(np.signbit(y), mag | 0x80, mag).astype(np.uint8)


def rne_bf16(y) -> np.ndarray:
    """Round FP64 values to bfloat16 (8 significant bits, min normal 2**-126),
    a single RNE rounding straight from FP64; returned as FP64 values."""
    return _rne_to_format(np.asarray(y, dtype=np.float64), mant_bits=7, emin=-126)


# Decode tables, built once from the bit-layout decoders above; indexing them
# is the same function, just fast enough for whole expert matrices.
_E2M1_TABLE = e2m1_decode(np.arange(16))
_E4M3_TABLE = e4m3_decode(np.arange(256))
_UE8M0_TABLE = ue8m0_decode(np.arange(256))


def dequant_fp4(packed, sf, gran: int, scale_kind: str, gs=None) -> np.ndarray:
    """Dequantise one block-scaled FP4 matrix to FP64.

    packed: [N, K/2] uint8 E2M1 codes, sf: [N, K/gran] scale bytes,
    scale_kind: "e4m3" (NVFP4 group16) or "ue8m0" (group32), gs: optional
    per-tensor FP32 global multiplier.
    W[n, k] = E2M1(code[n, k]) * S(sf[n, k // gran]) * gs   (exact in FP64:
    at most 2 + 4 + 24 significant bits).
    [P3] ``prepare_w4a16_modelopt_nvfp4_weights`` (K/16 E4M3 block scales with
    a per-expert global scale) and ``prepare_w4a16_fp4_e8m0_k32_weights``
    (K/32 E8M0 scales, global scale kept when given).
    """
    codes = unpack_fp4(packed)
    n, k = codes.shape
    sf = np.asarray(sf, dtype=np.uint8)
    if sf.shape != (n, k // gran) or k % gran:
        raise ValueError(f"scale shape {sf.shape} does not match [{n}, {k}/{gran}]")
    if scale_kind == "e4m3":
        s = _E4M3_TABLE[sf]
    elif scale_kind == "ue8m0":
        s = _UE8M0_TABLE[sf]
    else:
        raise ValueError(scale_kind)
    w = (_E2M1_TABLE[codes].reshape(n, k // gran, gran) * s[:, :, None]).reshape(n, k)
    if gs is not None:
        w = w * np.float64(np.float32(gs))
    return w
