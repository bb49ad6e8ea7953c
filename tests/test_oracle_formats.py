"""Pins for oracle.formats: closed forms, hand-worked blocks, brute force and an
independent library route (torch's float8 / bfloat16 conversions)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _half_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def _block(scales=0, qs=0, d=0.0, dmin=0.0, d_bits=None, dmin_bits=None):
    b = np.zeros(84, dtype=np.uint8)
    b[0:16] = scales
    b[16:80] = qs
    db = _half_bits(d) if d_bits is None else d_bits
    mb = _half_bits(dmin) if dmin_bits is None else dmin_bits
    b[80], b[81] = db & 0xFF, db >> 8
    b[82], b[83] = mb & 0xFF, mb >> 8
    return b


# ------------------------------------------------------------------ Q2 hand-worked blocks


def test_q2_zero_block():
    assert np.all(formats.q2_dequant(_block()) == 0)


def test_q2_all_max_codes_scale15():
    # d = 1, dmin = 0, every scale nibble 15, every code 3 -> 1 * 15 * 3 = 45
    w = formats.q2_dequant(_block(scales=0x0F, qs=0xFF, d=1.0))
    assert np.all(w == 45.0)


def test_q2_min_only():
    # d = 0, dmin = 1, every min nibble 15 -> -15 regardless of codes
    w = formats.q2_dequant(_block(scales=0xF0, qs=0xA5, d=0.0, dmin=1.0))
    assert np.all(w == -15.0)


@pytest.mark.parametrize("i,byte,shift", [(0, 16, 0), (1, 17, 0), (31, 47, 0), (32, 16, 2),
                                          (63, 47, 2), (64, 16, 4), (127, 47, 6), (128, 48, 0),
                                          (160, 48, 2), (255, 79, 6)])
def test_q2_code_byte_map(i, byte, shift):
    # a single code 2 placed at (byte, shift): only weight i becomes 2 * d * sc
    assert formats.q2_code_location(i) == (byte, shift)
    b = _block(scales=0x01, d=1.0)
    b[byte] = 2 << shift
    w = formats.q2_dequant(b)
    expect = np.zeros(256)
    expect[i] = 2.0
    assert np.array_equal(w, expect)


def test_q2_every_code_slot_lights_one_weight():
    # exhaustive inverse check: each of the 64 bytes x 4 shifts owns exactly one weight,
    # and the 256 slots cover the 256 weights
    seen = set()
    for byte in range(16, 80):
        for shift in (0, 2, 4, 6):
            b = _block(scales=0x01, d=1.0)
            b[byte] = 1 << shift
            nz = np.flatnonzero(formats.q2_dequant(b))
            assert nz.size == 1
            seen.add(int(nz[0]))
    assert seen == set(range(256))


def test_q2_subblock_scale_map():
    # scale byte s governs weights 16s..16s+15: low nibble scale, high nibble min
    for s in range(16):
        b = _block(qs=0x55, d=1.0, dmin=1.0)  # all codes 1
        b[s] = 0x37  # scale 7, min 3
        w = formats.q2_dequant(b)
        expect = np.zeros(256)
        expect[16 * s:16 * s + 16] = 7 * 1 - 3
        assert np.array_equal(w, expect)


def test_q2_subnormal_d():
    # d = 0x0001 = 2^-24 (smallest half subnormal)
    b = _block(scales=0x0B, qs=0xFF, d_bits=0x0001, dmin_bits=0)
    w = formats.q2_dequant(b)
    assert np.all(w == 2.0 ** -24 * 11 * 3)


def test_q2_bruteforce_fraction():
    rng = np.random.default_rng(0)
    for d_bits, m_bits in [(0x3C00, 0x3800), (0x2E66, 0x1A3F), (0x0001, 0x7BFF), (0x211F, 0x0003)]:
        d = Fraction(float(np.array([d_bits], np.uint16).view(np.float16)[0]))
        dm = Fraction(float(np.array([m_bits], np.uint16).view(np.float16)[0]))
        for sc in range(16):
            for mn in range(16):
                b = _block(scales=(mn << 4) | sc, d_bits=d_bits, dmin_bits=m_bits)
                qs = rng.integers(0, 256, 64, dtype=np.uint8)
                b[16:80] = qs
                w = formats.q2_dequant(b)
                for i in range(0, 256, 37):
                    byte, shift = formats.q2_code_location(i)
                    q = (int(b[byte]) >> shift) & 3
                    assert Fraction(w[i]) == d * sc * q - dm * mn


def test_q2_fp32_single_rounding_any_order():
    # w in float32 is one rounding of the exact value whether computed as
    # (d*sc)*q - dmin*m or with a fused multiply-add: every product is exact.
    rng = np.random.default_rng(1)
    for _ in range(200):
        d = np.float32(np.float16(abs(rng.normal(0, 0.01))))
        dm = np.float32(np.float16(abs(rng.normal(0, 0.01))))
        sc, mn, q = rng.integers(0, 16), rng.integers(0, 16), rng.integers(0, 4)
        a = np.float32(d * np.float32(sc))
        prod = np.float32(a * np.float32(q))
        mm = np.float32(dm * np.float32(mn))
        assert Fraction(float(a)) == Fraction(float(d)) * sc  # exact
        assert Fraction(float(prod)) == Fraction(float(d)) * sc * q
        assert Fraction(float(mm)) == Fraction(float(dm)) * mn
        exact = Fraction(float(d)) * sc * q - Fraction(float(dm)) * mn
        assert np.float32(prod - mm) == np.float32(float(exact))


def test_q2_matrix_flat_tiling():
    # rows shorter than a block: a 4 x 128 matrix is two blocks, block 0 = rows 0-1
    rng = np.random.default_rng(2)
    raw = rng.integers(0, 256, 2 * 84, dtype=np.uint8)
    raw[80:84] = [0, 0x3C, 0, 0]
    raw[84 + 80:84 + 84] = [0, 0x3C, 0, 0]
    m = formats.q2_matrix(raw, 4, 128)
    flat = formats.q2_dequant(raw.reshape(2, 84))
    assert np.array_equal(m[0], flat[0:128]) and np.array_equal(m[1], flat[128:256])
    assert np.array_equal(m[2], flat[256:384]) and np.array_equal(m[3], flat[384:512])


def test_q2_matrix_rows_along_k():
    # a 2 x 512 matrix: row r holds blocks 2r, 2r+1
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, 4 * 84, dtype=np.uint8)
    m = formats.q2_matrix(raw, 2, 512)
    flat = formats.q2_dequant(raw.reshape(4, 84)).reshape(4, 256)
    assert np.array_equal(m[1, 256:], flat[3])


# ------------------------------------------------------------------ Q8_0


def test_q8_0_hand_block():
    b = np.zeros(34, dtype=np.uint8)
    b[0], b[1] = 0x00, 0x38  # d = 0.5
    q = np.arange(-16, 16, dtype=np.int8)
    b[2:] = q.view(np.uint8)
    w = formats.q8_0_dequant(b)
    assert np.array_equal(w, q.astype(np.float64) * 0.5)


def test_q8_0_extremes():
    b = np.zeros(34, dtype=np.uint8)
    b[0], b[1] = 0x00, 0x3C  # d = 1
    b[2] = 0x80  # -128
    b[3] = 0x7F  # 127
    w = formats.q8_0_dequant(b)
    assert w[0] == -128 and w[1] == 127 and np.all(w[2:] == 0)


def test_q8_0_matches_torch_route():
    rng = np.random.default_rng(4)
    blocks = rng.integers(0, 256, (64, 34), dtype=np.uint8)
    blocks[:, 1] &= 0x3F  # finite d
    w = formats.q8_0_dequant(blocks).reshape(64, 32)
    d = torch.from_numpy(blocks[:, :2].copy()).view(torch.float16).double()
    q = torch.from_numpy(blocks[:, 2:].copy()).view(torch.int8).double()
    assert np.array_equal(w, (d * q).numpy())


# ------------------------------------------------------------------ E4M3 / E8M0 / BF16


def test_e4m3_closed_form_landmarks():
    assert formats.e4m3_to_f64(0x7E) == 448.0
    assert formats.e4m3_to_f64(0x08) == 2.0 ** -6
    assert formats.e4m3_to_f64(0x01) == 2.0 ** -9
    assert formats.e4m3_to_f64(0x07) == 7 * 2.0 ** -9
    assert np.isnan(formats.e4m3_to_f64(0x7F)) and np.isnan(formats.e4m3_to_f64(0xFF))
    assert formats.e4m3_to_f64(0x80) == 0.0 and np.signbit(formats.e4m3_to_f64(0x80))


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([formats.e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_monotone_positive_codes():
    v = [formats.e4m3_to_f64(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(v, v[1:]))


def test_e8m0_matches_torch():
    xs = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = xs.view(torch.float8_e8m0fnu).double().numpy()
    for x in range(255):
        assert 2.0 ** formats.e8m0_exponent(x) == ref[x]
    assert formats.e8m0_exponent(255) is None and np.isnan(ref[255])


def _load_anchors():
    rows = []
    with open(os.path.join(GOLDEN, "engram_decode_anchors.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            c, s, v = line.split()
            rows.append((int(c, 16), int(s), None if v == "NaN" else int(v, 16)))
    return rows


def test_engram_decode_golden_anchors():
    rows = _load_anchors()
    assert len(rows) >= 20
    for code, scale, expect in rows:
        got = formats.engram_decode_value(code, scale)
        if expect is None:
            assert formats.is_bf16_nan(np.uint16(got)), (hex(code), scale)
        else:
            assert got == expect, (hex(code), scale, hex(got), hex(expect))


def test_engram_decode_table_all_65536_vs_torch():
    """Every (code, scale): E4M3 x E8M0 through torch's own float8 decoders, the
    product (exact: <= 4 significant bits, inside binary32's range incl.
    subnormals, or beyond it and then also beyond BF16's) rounded by torch's
    binary32 -> bfloat16 conversion."""
    t = formats.engram_decode_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    v = codes.view(torch.float8_e4m3fn).double()
    s = codes.view(torch.float8_e8m0fnu).double()
    prod = (v[:, None] * s[None, :]).float()
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    nan_ref = torch.isnan(prod).numpy()
    nan_mine = formats.is_bf16_nan(t)
    assert np.array_equal(nan_ref, nan_mine)
    assert np.array_equal(t[~nan_mine], ref[~nan_ref])
    # survey of the edges: inexact subnormal roundings and overflows exist in the full range
    finite = ~nan_mine
    n_inf = int(np.sum(finite & ((t & 0x7FFF) == 0x7F80)))
    assert n_inf == 560
    # within the synthetic tables' scale range 110..140 every product is exact
    sub = t[:, 110:141]
    vals = v.numpy()[:, None] * 2.0 ** (np.arange(110, 141) - 127)[None, :]
    ok = ~np.isnan(vals)
    assert np.array_equal(formats.bf16_to_f64(sub)[ok], vals[ok])


def test_bf16_rounding_vs_torch_random():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    mine = formats.bf16_array_from_f64(f.astype(np.float64))
    assert np.array_equal(mine, ref)


def test_bf16_rounding_ties_and_edges():
    assert formats.bf16_from_f64(1.0 + 2.0 ** -8) == 0x3F80  # tie -> even
    assert formats.bf16_from_f64(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (up)
    assert formats.bf16_from_f64(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # above the tie
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127  # halfway between max finite and 2^128
    assert formats.bf16_from_f64(big) == 0x7F80
    assert formats.bf16_from_f64(np.nextafter(big, 0)) == 0x7F7F
    assert formats.bf16_from_f64(-0.0) == 0x8000
    assert formats.bf16_from_f64(2.0 ** -133) == 0x0001
    assert formats.bf16_from_f64(2.0 ** -126) == 0x0080
    assert formats.bf16_from_f64(float("inf")) == 0x7F80
