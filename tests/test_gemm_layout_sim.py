"""CPU simulation of the prefill GEMM's operand movement: global memory ->
LDS stage buffers (the direct-to-LDS loads of fc_gemm_a8_kernel) -> MFMA
operand fragments (its explicit LDS reads), for both weight layouts (RAW and
the GEMM layout written by moe_fp4_prepare_gemm_weights), FP8 and FP4
activations, and the UE8M0 scale bytes.

The index arithmetic of the kernel's loads and reads is restated here and
composed on labelled data; every lane of every MFMA must end up with the
elements the block-scaled MFMA operand layout assigns it (A: lane (r16, q) of
a 16-row group holds row r16, K elements 32q..32q+31 of the 128-K step; FP8
B: token r16, K bytes 16q..16q+15 and 64+16q..64+16q+15; FP4 B like A), and
the 16 lanes that share a 16-byte LDS read cycle must hit 16 distinct
16-byte bank groups (64 banks of 4 bytes).  A self-check in the manner of the
CuTeDSL W4A16 packer's own selftest (b12x moe/fused/w4a16/prepare.py,
_nf3_pack_selftest), which simulates its kernel's LDS staging and per-thread
reads in Python.  (The MFMA operand layout itself is exercised by the GPU
parity tests.)"""

import numpy as np
import pytest

GK = 128          # K per pipeline stage
WAVES = 4
LANES = 64


def roff(fc1, rg):
    """First row of wave row group rg relative to the wave's first row."""
    if fc1:
        return 16 * rg if rg < 4 else 256 + 16 * (rg - 4)
    return 16 * rg


def wrow0(fc1, w):
    return 64 * w if fc1 else 128 * w


def src_row(fc1, I, nb, r, order):
    """Global weight row of work-item-local row r (0..511) of row block nb."""
    if fc1:
        i0 = nb * 256 + (r & 255)
        return I + i0 if ((r >= 256) != (order != 0)) else i0
    return nb * 512 + r


def prepared_layout(codes, fc1, I, order):
    """The GEMM weight layout by its definition (moe_fp4_prepare_gemm_weights):
    piece j of (row block nb, stage s) = 16 bytes of source row j >> 2 at byte
    64 s + 16 ((j & 3) ^ ((j >> 4) & 3))."""
    N, KH = codes.shape
    K = 2 * KH
    ns, nblk = K // GK, N // 512
    out = np.zeros((nblk, ns, 2048, 16), np.uint8)
    for nb in range(nblk):
        for s in range(ns):
            for j in range(2048):
                piece = (j & 3) ^ ((j >> 4) & 3)
                r = src_row(fc1, I, nb, j >> 2, order)
                out[nb, s, j] = codes[r, 64 * s + 16 * piece: 64 * s + 16 * piece + 16]
    return out.reshape(-1)


def load_weight_stage(codes, prep, fc1, I, nb, s, order, flat_prep=None):
    """The stage's weight area in LDS (2048 16-byte slots) after the 8
    load instructions of each of the 4 waves."""
    N, KH = codes.shape
    K = 2 * KH
    lds = np.full((2048, 16), 255, np.uint8)
    for w in range(WAVES):
        for i in range(8):
            for lane in range(LANES):
                slot = 512 * w + 64 * i + lane
                if prep:
                    byte = nb * (K // GK) * 32768 + (512 * w + lane) * 16 + 1024 * i + 256 * (GK * s)
                    lds[slot] = flat_prep[byte: byte + 16]
                else:
                    r = 128 * w + (lane >> 2) + 16 * i
                    pw = (lane & 3) ^ ((lane >> 4) & 3)
                    row = src_row(fc1, I, nb, r, order)
                    b = 16 * pw + (GK * s) // 2
                    lds[slot] = codes[row, b: b + 16]
    return lds


def weight_fragment_slot(fc1, w, rg, lane):
    r16, q = lane & 15, lane >> 4
    return 4 * (wrow0(fc1, w) + roff(fc1, rg) + r16) + (q ^ ((r16 >> 2) & 3))


@pytest.mark.parametrize("fc1,order,prep", [(True, 0, False), (True, 1, False), (True, 0, True), (True, 1, True),
                                            (False, 0, False), (False, 0, True)])
def test_weight_fragments_reach_the_mfma_layout(fc1, order, prep):
    rng = np.random.default_rng(7)
    I, H = 512, 1024
    N, K = (2 * I, H) if fc1 else (H, I)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    flat = prepared_layout(codes, fc1, I, order) if prep else None
    nblk = I // 256 if fc1 else H // 512
    for nb in range(nblk):
        for s in (0, K // GK - 1):
            lds = load_weight_stage(codes, prep, fc1, I, nb, s, order, flat)
            for w in range(WAVES):
                for rg in range(8):
                    for lane in range(LANES):
                        r16, q = lane & 15, lane >> 4
                        got = lds[weight_fragment_slot(fc1, w, rg, lane)]
                        row = src_row(fc1, I, nb, wrow0(fc1, w) + roff(fc1, rg) + r16, order)
                        want = codes[row, (GK * s) // 2 + 16 * q: (GK * s) // 2 + 16 * q + 16]
                        assert np.array_equal(got, want), (nb, s, w, rg, lane)


def test_prepared_layout_is_a_permutation():
    rng = np.random.default_rng(3)
    I, H = 512, 1024
    codes = rng.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
    flat = prepared_layout(codes, True, I, 0)
    assert flat.size == codes.size
    assert np.array_equal(np.sort(flat), np.sort(codes.reshape(-1)))


def act_stage_fp8(x, rows, s):
    """FP8 activations: 4 load instructions per wave, stage slot S = 256 w +
    64 i + lane holds tile row S >> 3, piece (S & 7) ^ ((row >> 1) & 7)."""
    lds = np.full((1024, 16), 255, np.uint8)
    for w in range(WAVES):
        for i in range(4):
            for lane in range(LANES):
                S = 256 * w + 64 * i + lane
                t = S >> 3
                p = (S & 7) ^ ((t >> 1) & 7)
                lds[S] = x[rows[t], GK * s + 16 * p: GK * s + 16 * p + 16]
    return lds


def act_stage_fp4(x4, rows, s):
    """FP4 activations: 2 load instructions per wave, slot S = 128 w + 64 i +
    lane holds tile row S >> 2, piece (S & 3) ^ ((row >> 2) & 3)."""
    lds = np.full((512, 16), 255, np.uint8)
    for w in range(WAVES):
        for i in range(2):
            for lane in range(LANES):
                S = 128 * w + 64 * i + lane
                t = S >> 2
                p = (S & 3) ^ ((t >> 2) & 3)
                b = (GK * s) // 2 + 16 * p
                lds[S] = x4[rows[t], b: b + 16]
    return lds


def test_fp8_activation_fragments():
    rng = np.random.default_rng(11)
    T, H = 300, 512
    x = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    rows = rng.integers(0, T, size=128)  # the tile's gathered token rows
    for s in range(H // GK):
        lds = act_stage_fp8(x, rows, s)
        for tg in range(8):
            for lane in range(LANES):
                r16, q = lane & 15, lane >> 4
                xr = (r16 >> 1) & 7
                s0 = 8 * (16 * tg + r16) + (q ^ xr)
                s1 = 8 * (16 * tg + r16) + ((q + 4) ^ xr)
                t = 16 * tg + r16
                assert np.array_equal(lds[s0], x[rows[t], GK * s + 16 * q: GK * s + 16 * q + 16])
                assert np.array_equal(lds[s1], x[rows[t], GK * s + 64 + 16 * q: GK * s + 64 + 16 * q + 16])


def test_fp4_activation_fragments():
    rng = np.random.default_rng(12)
    T, H = 200, 512
    x4 = rng.integers(0, 256, size=(T, H // 2), dtype=np.uint8)
    rows = rng.integers(0, T, size=128)
    for s in range(H // GK):
        lds = act_stage_fp4(x4, rows, s)
        for tg in range(8):
            for lane in range(LANES):
                r16, q = lane & 15, lane >> 4
                slot = 4 * (16 * tg + r16) + (q ^ ((r16 >> 2) & 3))
                b = (GK * s) // 2 + 16 * q
                assert np.array_equal(lds[slot], x4[rows[16 * tg + r16], b: b + 16])


def perm_b32(s0, s1, sel):
    """v_perm_b32: byte k of the result is byte sel_k of the 8 bytes s0:s1
    (0..3 from s1, 4..7 from s0), 0x0C gives zero."""
    src = list(int(s1).to_bytes(4, "little")) + list(int(s0).to_bytes(4, "little"))
    out = 0
    for k in range(4):
        b = (sel >> (8 * k)) & 0xFF
        v = src[b] if b < 8 else (0 if b == 0x0C else None)
        assert v is not None
        out |= v << (8 * k)
    return out


def test_scale_byte_selection():
    """A lane keeps bytes q, 4 + q, 8 + q, 12 + q of its row's 16 group scale
    bytes in one word (three v_perm_b32); stage s of the group takes byte s
    after s shifts by 8 bits: the scale of K block 4 s + q, the block its MFMA
    operand covers."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        line = rng.integers(0, 256, size=16, dtype=np.uint8)
        v = np.frombuffer(line.tobytes(), dtype="<u4")
        for q in range(4):
            sel_lo = q | ((4 + q) << 8) | 0x0C0C0000
            lo = perm_b32(v[1], v[0], sel_lo)
            hi = perm_b32(v[3], v[2], sel_lo)
            word = perm_b32(hi, lo, 0x05040100)
            for s in range(4):
                assert (word >> (8 * s)) & 0xFF == line[4 * s + q]


def test_scale_line_placement_raw_and_prepared():
    """Weight scale lines: RAW rows 128 w + lane and 128 w + 64 + lane, or the
    prepared image (piece (nb * K/512 + g) * 512 + i = row i's bytes 16 g ..
    16 g + 15), both land as wsc[row * 16]; tile-row scale lines land in
    region tg >> 1 at lane (tg & 1) * 16 + r16 for tile row 16 tg + r16."""
    rng = np.random.default_rng(9)
    I, H = 512, 1024
    N, K = 2 * I, H
    sf = rng.integers(0, 256, size=(N, K // 32), dtype=np.uint8)
    ng = K // 512
    for order in (0, 1):
        prep = np.zeros(((N // 512) * ng * 512, 16), np.uint8)
        for nb in range(N // 512):
            for g in range(ng):
                for i in range(512):
                    prep[(nb * ng + g) * 512 + i] = sf[src_row(True, I, nb, i, order), 16 * g: 16 * g + 16]
        for nb in range(I // 256):
            for g in range(ng):
                raw_lds = np.zeros((512, 16), np.uint8)
                prep_lds = np.zeros((512, 16), np.uint8)
                for w in range(WAVES):
                    for j in range(2):
                        for lane in range(LANES):
                            r = 128 * w + 64 * j + lane
                            raw_lds[r] = sf[src_row(True, I, nb, r, order), 16 * g: 16 * g + 16]
                            piece = (nb * ng + g) * 512 + 128 * w + lane + 64 * j
                            prep_lds[r] = prep[piece]
                assert np.array_equal(raw_lds, prep_lds)
                for r in range(512):
                    assert np.array_equal(raw_lds[r], sf[src_row(True, I, nb, r, order), 16 * g: 16 * g + 16])
    # tile-row scale lines
    asc = np.zeros((WAVES, LANES), np.int64)
    for w in range(WAVES):
        for lane in range(LANES):
            asc[w, lane] = 32 * w + (lane & 31)
    for tg in range(8):
        for r16 in range(16):
            assert asc[tg >> 1, (tg & 1) * 16 + r16] == 16 * tg + r16


def bank_groups(slots):
    """16-byte bank group (64 banks of 4 bytes = 16 groups) of each slot."""
    return [s % 16 for s in slots]


@pytest.mark.parametrize("fc1", [True, False])
def test_operand_reads_are_bank_conflict_free(fc1):
    """Each ds_read_b128 serves 16 lanes per cycle: lanes 16 c .. 16 c + 15
    must read 16 distinct bank groups (weight, FP8 and FP4 activation
    fragments)."""
    for w in range(WAVES):
        for rg in range(8):
            for c in range(4):
                slots = [weight_fragment_slot(fc1, w, rg, lane) for lane in range(16 * c, 16 * c + 16)]
                assert len(set(bank_groups(slots))) == 16
    for tg in range(8):
        for c in range(4):
            for half in (0, 4):
                slots = []
                for lane in range(16 * c, 16 * c + 16):
                    r16, q = lane & 15, lane >> 4
                    slots.append(8 * (16 * tg + r16) + ((q + half) ^ ((r16 >> 1) & 7)))
                assert len(set(bank_groups(slots))) == 16
            slots = [4 * (16 * tg + (l & 15)) + ((l >> 4) ^ (((l & 15) >> 2) & 3)) for l in range(16 * c, 16 * c + 16)]
            assert len(set(bank_groups(slots))) == 16
