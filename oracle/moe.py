"""Top-k routed MoE forward over block-scaled FP4 weights, FP64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The path, step by step (the MoE expert computation named on [P2] "Context"
-- the FP8xFP4 MegaMoE recipe (1, 1, 32) -- and on [P3] for the W4A16 form
with K/16 E4M3 or K/32 E8M0 scales):

  route    assignments a = t*k + j are grouped by expert id, stably (ties in
           a-order); counts n_e, exclusive offsets o_e, sorted_assign and its
           inverse slot_of;
  FC1      G[a, :] = sum_h xhat[t, h] * W13_e[:, h]   (W13 rows: gate then up
           in the kernel-native "w31"/"gate_up" order of [P3] module
           constants and ``_normalize_w13_layout``; "w13"/"up_gate" order is
           the same rows rotated by I, as in ``_prepare_w4a16_packed_weights``);
  SwiGLU   h = silu(gate) * up, silu(z) = z / (1 + exp(-z));
  h quant  A16: RNE to bfloat16 (one rounding from FP64);
           A8 : per assignment, per 32 consecutive I elements, UE8M0 exponent
                e = ceil(log2(amax / 448)) and E4M3 RNE of h / 2**e;
           A4 : per assignment, per 32 consecutive I elements, the block rule
                of the group32 requantisation ([P1] ``requant_fp4_to_gran_k``,
                [P2] "Requantization path"): UE8M0 e = ceil(log2(amax / 6))
                and E2M1 RNE of h / 2**e (the activations x arrive in the same
                MXFP4 form: "A4 prefill" of [P3] ``prepare_w4a16_modelopt_-
                native_weights``, read as the block-scaled FP4 format the
                matrix instruction consumes);
  FC2      Y[a, :] = sum_i hhat[a, i] * W2_e[:, i];
  combine  out[t] = sum_j topk_w[t, j] * Y[slot_of[t*k + j]], j ascending.

All arithmetic is FP64; dequantised weights are exact.  Assignments whose
expert id lies outside [0, E) are dropped (they contribute nothing), which
is the documented behaviour of the library for such ids.
"""

from __future__ import annotations

import numpy as np

from .formats import (
    bf16_bits_decode,
    dequant_fp4,
    e2m1_decode,
    e4m3_decode,
    pack_fp4,
    rne_bf16,
    rne_e2m1_magnitude,
    rne_e4m3,
    ue8m0_decode,
    unpack_fp4,
)
from .requant import _ceil_log2_ratio, requant_block


def route(topk_ids, E: int):
    """Counting sort of assignments by expert.

    Returns (counts [E], offsets [E+1], sorted_assign [A], slot_of [A]) as
    int32; entries past offsets[E] in sorted_assign and slot_of of dropped
    assignments are -1."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    A = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.zeros(E, dtype=np.int64)
    for a in range(A):
        if valid[a]:
            counts[ids[a]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    sorted_assign = np.full(A, -1, dtype=np.int64)
    slot_of = np.full(A, -1, dtype=np.int64)
    for a in range(A):
        if valid[a]:
            p = fill[ids[a]]
            fill[ids[a]] += 1
            sorted_assign[p] = a
            slot_of[a] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_assign.astype(np.int32), slot_of.astype(np.int32))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    # exp(-z) overflows to inf for z < -709; z / inf is then the exact
    # limit (-0.0), so the overflow is expected and not reported
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def quantize_h_a8(h):
    """Per row, per 32 consecutive elements: UE8M0 e = ceil(log2(amax/448))
    (smallest e with 448 * 2**e >= amax; amax == 0 -> e = -127), clamp to
    [-127, 127], then E4M3 RNE of h / 2**e.  Returns (hhat values FP64,
    fp8 bytes, scale bytes)."""
    h = np.asarray(h, dtype=np.float64)
    n, I = h.shape
    blk = h.reshape(n, I // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    nz = amax > 0
    e = np.where(nz, _ceil_log2_ratio(np.where(nz, amax, 1.0), 448.0), -127)
    e = np.clip(e, -127, 127)
    q = rne_e4m3(np.ldexp(blk, -e[..., None]))
    hhat = np.ldexp(e4m3_decode(q), e[..., None])
    return hhat.reshape(n, I), q.reshape(n, I), (e + 127).astype(np.uint8)


def quantize_a4(v):
    """MXFP4 rows: per row, per 32 consecutive elements, the requantisation
    block rule (UE8M0 e = ceil(log2(amax / 6)), amax == 0 -> e = -127, E2M1
    RNE of v / 2**e with the sign kept).  Returns (vhat values FP64, packed
    codes [n, K/2] uint8 with element 2j in the low nibble of byte j, scale
    bytes [n, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    codes, sb = requant_block(v.reshape(n, K // 32, 32))
    vhat = e2m1_decode(codes) * np.ldexp(1.0, sb.astype(np.int64) - 127)[..., None]
    return vhat.reshape(n, K), pack_fp4(codes.reshape(n, K)), sb


E2M1_POS = e2m1_decode(np.arange(8, dtype=np.uint8))  # magnitudes of codes 0..7


# A rounding decision of h is taken as undecided between its two
# neighbouring results when h lies within a decision radius times the maximum
# |h| of its 32-element block of the decision boundary.  The radius bounds how
# far the GPU's computation of h can land from the exact one.
#
# DECISION_RADIUS (bfloat16 activations on the bf16 / fp16 matrix
# instructions, and FP4 activations on the FP4 x FP4 block-scaled one):
#  * FC1 products are exact in FP32 (an E2M1 code times an E4M3 or power-of-
#    two block scale has at most 6 significant bits, a bfloat16 / fp16 / E2M1
#    activation at most 11), the global scale is one multiplication after the
#    sum, so the only FP32 error of G is its accumulation: at most K - 1
#    roundings of relative size <= 2**-24, fewest errors to the sequential
#    order's most;
#  * under the usual model of independent rounding errors the accumulated
#    error is about 2**-24 * sqrt(sum of squared partial sums) (Higham and
#    Mary, probabilistic rounding error analysis, 2019); for the workloads'
#    shapes the sequential FP32 order of K = 6144 exact products, followed by
#    SwiGLU in FP32, lands within 2**-19 of the block maximum of the exact h
#    (the CPU pin test_decision_radius_covers_fp32 checks this on decode,
#    prefill and tiny shapes);
#  * SwiGLU in FP32 with a hardware exp and reciprocal adds a few ulp of |h|
#    <= the block maximum, below 2**-21 of it.
# 2**-17 is four times the larger of those.
DECISION_RADIUS = 2.0 ** -17
# DECISION_RADIUS_FP8 (FP8 activations on the FP8 x FP4 block-scaled matrix
# instruction of the GPU): that instruction does not add its 128 products
# exactly -- measured on MI355X, one instruction's result is off by up to
# 2**-12.8 of its largest product on Gaussian FP8 data and 2**-10.9 on data
# spanning 16 binades, while FP4 x FP4 and bf16 products sum exactly there --
# so G carries errors far above FP32 rounding.  Over every FP8 parity case the
# GPU's quantised h differs from the exact one's only where h lies within
# 2**-14.8 of a block maximum of a boundary; 2**-13 is 3.5 times that.
DECISION_RADIUS_FP8 = 2.0 ** -13


def decision_radius(a8, a4=False):
    """The decision radius of the path: FP8 activations (a8 and not a4), or
    the FP32-accurate paths."""
    return DECISION_RADIUS_FP8 if a8 and not a4 else DECISION_RADIUS


def _grid_ambiguity(y, mant_bits, emin, radius):
    """|alternative rounding - RNE rounding| of each exact value y when y lies
    within ``radius`` (absolute, same units as y) of a rounding midpoint of the
    float grid with ``mant_bits`` fraction bits and minimum normal exponent
    ``emin``; 0 elsewhere."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, ex = np.frexp(y)
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, e - mant_bits)
    frac = y / quantum - np.floor(y / quantum)
    near = np.abs(frac - 0.5) * quantum <= radius
    return np.where(near, quantum, 0.0)


def h_decision_band(h, a8, radius=None, a4=False):
    """Per element, the largest change of the quantised h that a rounding
    decision within ``radius`` (default: the path's decision_radius) * (block
    max |h|) could make: one grid step
    where h is that close to a rounding midpoint and, for A8 / A4, the whole
    requantisation of a 32-block under the neighbouring exponent where amax
    is that close to 448 * 2**e (6 * 2**e).  Zero where every decision is
    clear."""
    if radius is None:
        radius = decision_radius(a8, a4)
    h = np.asarray(h, dtype=np.float64)
    n, I = h.shape
    blk = h.reshape(n, I // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    rad = radius * amax[..., None]
    if not a8 and not a4:
        return _grid_ambiguity(blk, 7, -126, rad).reshape(n, I)
    if a4:
        hhat, _, sb = quantize_a4(h)
        top, mant, emin = 6.0, 1, 0

        def requant_at(e2):
            y = np.clip(np.ldexp(np.abs(blk), -e2[..., None]), 0, 6)
            return np.copysign(E2M1_POS[rne_e2m1_magnitude(y)], blk) * np.ldexp(1.0, e2[..., None])
    else:
        hhat, _, sb = quantize_h_a8(h)
        top, mant, emin = 448.0, 3, -6

        def requant_at(e2):
            return np.ldexp(e4m3_decode(rne_e4m3(np.clip(np.ldexp(blk, -e2[..., None]), -448, 448))),
                            e2[..., None])
    hhat = hhat.reshape(n, I // 32, 32)
    e = sb.astype(np.int64) - 127
    band = _grid_ambiguity(np.ldexp(blk, -e[..., None]), mant, emin,
                           np.ldexp(rad, -e[..., None])) * np.ldexp(1.0, e[..., None])
    for de in (-1, 1):
        e2 = e + de
        lim = np.ldexp(top, np.minimum(e, e2))  # the boundary between e and e2
        close = (amax > 0) & (np.abs(amax - lim) <= radius * amax)
        if np.any(close):
            alt = requant_at(e2)
            band = np.where(close[..., None], np.maximum(band, np.abs(alt - hhat)), band)
    return band.reshape(n, I)


def h_decision_margin(h, a8, a4=False):
    """Per element, the distance from the exact h to the nearest boundary at
    which its quantisation decision changes, divided by the maximum |h| of
    its 32-element block: the rounding midpoint of its grid (bf16; or E4M3 /
    E2M1 after the block's UE8M0 scaling) and, for A8 / A4, the block's
    exponent boundaries 448 * 2**(e-1), 448 * 2**e (6 * 2**(e-1), 6 * 2**e)
    around max |h|.  An FP32 h closer than this to the exact one is
    quantised as the exact one is.  All-zero blocks get +inf."""
    h = np.asarray(h, dtype=np.float64)
    n, I = h.shape
    blk = np.abs(h.reshape(n, I // 32, 32))
    amax = np.max(blk, axis=-1)

    def grid_dist(y, mant_bits, emin):
        _, ex = np.frexp(y)
        e = np.maximum(ex.astype(np.int64) - 1, emin)
        quantum = np.ldexp(1.0, e - mant_bits)
        frac = y / quantum - np.floor(y / quantum)
        return np.abs(frac - 0.5) * quantum

    if not a8 and not a4:
        dist = grid_dist(blk, 7, -126)
    else:
        top, mant, emin = (6.0, 1, 0) if a4 else (448.0, 3, -6)
        _, _, sb = quantize_a4(h) if a4 else quantize_h_a8(h)
        e = sb.astype(np.int64) - 127
        dist = np.ldexp(grid_dist(np.ldexp(blk, -e[..., None]), mant, emin), e[..., None])
        lo, hi = np.ldexp(top, e - 1), np.ldexp(top, e)
        dexp = np.minimum(np.abs(amax - lo), np.abs(hi - amax))
        dist = np.minimum(dist, dexp[..., None])
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(amax[..., None] > 0, dist / amax[..., None], np.inf)
    return m.reshape(n, I)


def decode_activations(x, x_sf=None, a4=False):
    """A16: x is [T, H] bfloat16 bit patterns (uint16).  A8: x is [T, H]
    E4M3 bytes and x_sf [T, H/32] UE8M0 bytes; value = fp8 * 2**(sf - 127).
    A4: x is [T, H/2] packed E2M1 codes (element 2j in the low nibble of byte
    j) and x_sf [T, H/32] UE8M0 bytes; value = e2m1 * 2**(sf - 127)."""
    if x_sf is None:
        return bf16_bits_decode(x)
    xv = e2m1_decode(unpack_fp4(x)) if a4 else e4m3_decode(x)
    return xv * np.repeat(ue8m0_decode(x_sf), 32, axis=1)


def moe_forward(x, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs,
                gran: int, x_sf=None, w13_order: str = "gate_up",
                tokens=None, out_cols=None, return_parts=False, return_band=False, a4=False,
                return_h=False):
    """FP64 MoE forward.  Shapes: x [T, H] (see decode_activations),
    topk_ids/topk_w [T, k], w13 [E, 2I, H/2], w13_sf [E, 2I, H/gran],
    w2 [E, H, I/2], w2_sf [E, H, I/gran], gs [E] float32 or None.

    gran 16 -> E4M3 block scales, gran 32 -> UE8M0 block scales.
    x_sf given -> A8 activations, and h is quantised to FP8 + UE8M0 per 32;
    with a4=True as well -> A4 (MXFP4 x, h quantised to E2M1 + UE8M0 per 32);
    otherwise A16 (bfloat16 x, bfloat16 h).

    ``tokens`` / ``out_cols`` restrict the computation to a subset of output
    rows / columns (each output element is computed by the same definition);
    the result is then [len(tokens), len(out_cols)].

    ``return_h``: also return {slot: (h, hhat)}, the exact SwiGLU output and
    its quantised value (the FC2 input) per computed assignment.

    ``return_band``: also return, per output element, the largest change
    that near-tie rounding decisions of h (see h_decision_band) can cause:
    sum_j |w| * sum_i band_i * |W2[n, i]|.  Every result inside
    out +- band is an equally valid outcome of the quantisation rule.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    E, two_i, _ = np.asarray(w13).shape
    I = two_i // 2
    H = np.asarray(w2).shape[1]
    kind = {16: "e4m3", 32: "ue8m0"}[gran]
    if a4 and x_sf is None:
        raise ValueError("A4 activations need x_sf")
    a8 = x_sf is not None and not a4
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out_cols = np.arange(H) if out_cols is None else np.asarray(out_cols, dtype=np.int64)
    hrows = {}  # slot -> (exact h row, quantised h row), for return_h

    counts, offsets, sorted_assign, slot_of = route(ids, E)
    xv = decode_activations(x, x_sf, a4)
    want = np.zeros(T * k, dtype=bool)
    for t in tokens:
        want[t * k:(t + 1) * k] = True

    Y = {}  # slot -> FP64 row over out_cols
    YB = {}  # slot -> decision band row
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        assigns = [int(a) for a in sorted_assign[lo:hi] if want[a]]
        if not assigns:
            continue
        tok = np.array([a // k for a in assigns])
        X = xv[tok]
        gs1 = None if w13_gs is None else np.asarray(w13_gs, dtype=np.float32)[e]
        gs2 = None if w2_gs is None else np.asarray(w2_gs, dtype=np.float32)[e]
        W13 = dequant_fp4(w13[e], w13_sf[e], gran, kind, gs1)
        G = X @ W13.T
        if w13_order == "gate_up":
            gate, up = G[:, :I], G[:, I:]
        elif w13_order == "up_gate":
            up, gate = G[:, :I], G[:, I:]
        else:
            raise ValueError(w13_order)
        h = silu(gate) * up
        hhat = quantize_a4(h)[0] if a4 else quantize_h_a8(h)[0] if a8 else rne_bf16(h)
        if return_h:
            for r, a in enumerate(assigns):
                hrows[int(slot_of[a])] = (h[r], hhat[r])
        W2 = dequant_fp4(np.asarray(w2[e])[out_cols], np.asarray(w2_sf[e])[out_cols],
                         gran, kind, gs2)
        Ye = hhat @ W2.T
        if return_band:
            YBe = h_decision_band(h, a8, a4=a4) @ np.abs(W2).T
        for r, a in enumerate(assigns):
            Y[int(slot_of[a])] = Ye[r]
            if return_band:
                YB[int(slot_of[a])] = YBe[r]

    out = np.zeros((len(tokens), len(out_cols)), dtype=np.float64)
    band = np.zeros_like(out)
    for r, t in enumerate(tokens):
        for j in range(k):
            s = int(slot_of[t * k + j])
            if s >= 0:
                out[r] += w[t, j] * Y[s]
                if return_band:
                    band[r] += abs(w[t, j]) * YB[s]
    res = (out,)
    if return_parts:
        res += ((counts, offsets, sorted_assign, slot_of),)
    if return_band:
        res += (band,)
    if return_h:
        res += (hrows,)
    return res[0] if len(res) == 1 else res
