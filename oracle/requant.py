"""Group16 (E4M3 + global scale) -> group32 (UE8M0) FP4 requantisation, FP64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes, in the order the pages give it ([P2] section
"Requantization path"; [P1] commit "Separate source and destination FP4 scale
packing in requant_fp4_to_gran_k ... always recomputes UE8M0 runtime scales"):

  1. dequantise the group16 FP4 values with their original scales:
     v = E2M1(code) * E4M3(sf16[k // 16]) * gs       (exact in FP64);
  2. requantise the restored values with group32 scales: for each block of 32
     consecutive K elements of a row, amax = max |v|, the UE8M0 exponent is
     e = ceil(log2(amax / 6)) -- the smallest integer with 6 * 2**e >= amax,
     found exactly -- and each code is RNE of |v| / 2**e onto the E2M1 grid
     with the sign of v kept;
  3. the group32 result is consumed by the existing recipe (1, 1, 32) kernel.

Readings where the pages are silent (each also listed in the design doc):
  * "restored values" include the global scale, so gs is folded into the
    group32 output (which carries no global scale);
  * amax == 0: the block keeps zero magnitudes (signs kept) and scale byte 0;
  * the exponent is clamped to [-127, 127] (bytes 0..254), magnitudes above 6
    after the clamp saturate to 6;
  * ties go to the even E2M1 code; a negative value that rounds to zero keeps
    its sign (code 0x8).
"""

from __future__ import annotations

import numpy as np

from .formats import dequant_fp4, pack_fp4, rne_e2m1_magnitude


def _ceil_log2_ratio(amax: np.ndarray, top: float) -> np.ndarray:
    """Smallest integer e with top * 2**e >= amax, for amax > 0, exactly.

    A floating ceil(log2(amax / top)) can be off by one near powers of two;
    it is corrected by comparing against the exact power-of-two products."""
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(amax / top)).astype(np.int64)
    for _ in range(2):
        e = np.where(np.ldexp(top, e) < amax, e + 1, e)
        e = np.where(np.ldexp(top, e - 1) >= amax, e - 1, e)
    return e


def requant_block(v: np.ndarray):
    """Requantise blocks of restored values.

    v: [..., 32] FP64 (exact restored values).  Returns (codes [..., 32]
    uint8 in 0..15, scale byte [...] uint8)."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=-1)
    nz = amax > 0
    e = np.where(nz, _ceil_log2_ratio(np.where(nz, amax, 1.0), 6.0), -127)
    e = np.clip(e, -127, 127)
    x = np.ldexp(np.abs(v), -e[..., None])
    mag = rne_e2m1_magnitude(np.minimum(x, 6.0))
    codes = np.where(np.signbit(v), mag | 0x8, mag).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def requant_g16_to_g32(src, src_sf, gs=None, experts=None):
    """Requantise a grouped FP4 tensor from group16 E4M3 (+ FP32 global scale
    per expert) to group32 UE8M0.

    src: [E, N, K/2] uint8, src_sf: [E, N, K/16] uint8 (E4M3), gs: [E] float32
    or None.  Returns (dst [E', N, K/2] uint8, dst_sf [E', N, K/32] uint8)
    for the experts listed in ``experts`` (default all)."""
    src = np.asarray(src, dtype=np.uint8)
    src_sf = np.asarray(src_sf, dtype=np.uint8)
    E, N, kh = src.shape
    K = kh * 2
    if K % 32:
        raise ValueError("requant g16->g32 needs K divisible by 32")
    if src_sf.shape != (E, N, K // 16):
        raise ValueError(f"src_sf shape {src_sf.shape} != {(E, N, K // 16)}")
    ex = range(E) if experts is None else list(experts)
    dst = np.empty((len(ex), N, kh), dtype=np.uint8)
    dst_sf = np.empty((len(ex), N, K // 32), dtype=np.uint8)
    for i, e in enumerate(ex):
        g = None if gs is None else np.asarray(gs, dtype=np.float32)[e]
        v = dequant_fp4(src[e], src_sf[e], 16, "e4m3", g).reshape(N, K // 32, 32)
        codes, sb = requant_block(v)
        dst[i] = pack_fp4(codes.reshape(N, K))
        dst_sf[i] = sb
    return dst, dst_sf
