"""Comparator self-tests (planted mistakes must fail) and input-generator pins."""
import numpy as np
import pytest

import synthdata
from oracle import compare, engram, formats


# ------------------------------------------------------------------ comparators


def test_rel_error_detects_planted_error():
    rng = np.random.default_rng(0)
    y = rng.normal(size=(4, 64))
    assert compare.max_rel_error(y, y) == 0.0
    bad = y.copy()
    bad[2, 5] += 2e-2 * max(abs(y[2, 5]), np.sqrt(np.mean(y[2] ** 2)))
    assert compare.max_rel_error(bad, y) > 1e-2 - 1e-12
    nan = y.copy()
    nan[1, 1] = np.nan
    assert compare.max_rel_error(nan, y) == np.inf
    inf = y.copy()
    inf[0, 0] = np.inf
    assert compare.max_rel_error(inf, y) == np.inf


def test_rel_error_small_noise_passes():
    rng = np.random.default_rng(1)
    y = rng.normal(size=(4, 64))
    assert compare.max_rel_error(y * (1 + 1e-3), y) < 1.1e-3


def test_tie_rule():
    L = np.array([5.0, 4.0, 3.0, 3.0 + 5e-6, 1.0])
    assert compare.valid_selection([0, 1, 3], L, 3)
    assert compare.valid_selection([0, 1, 2], L, 3)  # within 1e-5 of the boundary
    assert not compare.valid_selection([0, 1, 4], L, 3)
    assert not compare.valid_selection([0, 0, 1], L, 3)
    assert not compare.valid_selection([1, 0, 3], L, 3)  # order broken by far more than 1e-5
    L2 = np.array([5.0, 4.0, 3.0, 2.9, 1.0])
    assert not compare.valid_selection([0, 1, 3], L2, 3)
    ex, ties, bad = compare.compare_ids(np.array([[0, 1, 2], [0, 1, 4]]), np.array([[0, 1, 3], [0, 1, 3]]),
                                        np.stack([L, L]))
    assert (ex, ties, bad) == (0, 1, [1])


def test_bf16_bits_equal_nan_aware():
    a = np.array([0x7FC0, 0x3F80, 0x8000], np.uint16)
    b = np.array([0xFFC1, 0x3F80, 0x8000], np.uint16)
    assert compare.bf16_bits_equal(a, b)
    c = np.array([0x7FC0, 0x3F80, 0x0000], np.uint16)
    assert not compare.bf16_bits_equal(a, c)


# ------------------------------------------------------------------ generators


def test_splitmix_reference_values():
    # SplitMix64 seeded with 0: published first outputs of the reference generator
    w = synthdata.words(0, 0, 3)
    assert [hex(int(v)) for v in w] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def test_half_normal_lut():
    lut = synthdata.half_normal_lut()
    v = lut.view(np.float16).astype(np.float64)
    assert np.all(v >= 0) and np.all(np.diff(v) >= 0)
    assert abs(np.median(v) - 0.01 * 0.6744897501960817) < 1e-5
    assert 0.04 < v[-1] < 0.05


def test_q2_generator_deterministic_and_sliced():
    k = synthdata.tensor_key(1, synthdata.KIND_GATE, 3)
    full = synthdata.q2_bytes(k, 0, 10)
    part = synthdata.q2_bytes(k, 4, 3)
    assert np.array_equal(full[4:7], part)
    w = formats.q2_dequant(full)
    assert np.all(np.isfinite(w)) and np.abs(w).max() < 1.0


def test_engram_rows_valid_codes():
    k = synthdata.tensor_key(1, synthdata.KIND_ENGRAM, 0)
    rows = synthdata.engram_rows(k, np.arange(200) * 9973)
    vals = rows[:, :256]
    assert not np.any((vals & 0x7F) == 0x7F)  # no NaN codes
    sc = rows[:, 256:]
    assert sc.min() >= 110 and sc.max() <= 140
    assert len(np.unique(vals)) == 254
    dec = engram.decode_rows(rows)
    assert not np.any(formats.is_bf16_nan(dec))


def test_engram_gather_out_of_range_raises():
    with pytest.raises(ValueError):
        engram.gather(lambda ids: np.zeros((len(ids), 264), np.uint8), 10, [3, 10])


def test_engram_hash_ids_range_and_chunk_equivalence():
    toks = synthdata.token_ids(1, 0, 40)
    ids_all = synthdata.engram_row_ids(1, toks, 0)
    assert ids_all.shape == (40, 2, 8)
    assert ids_all.min() >= 0 and ids_all.max() < 1 << 22
    # token-by-token on growing prefixes equals one pass over the chunk
    for p in (0, 1, 2, 3, 17, 39):
        one = synthdata.engram_row_ids(1, toks[:p + 1], p)
        assert np.array_equal(one[0], ids_all[p])
    # history before the start is the pad id: position 0 equals a sequence
    # whose preceding tokens are explicitly the pad value
    padded = np.concatenate([[synthdata.VOCAB] * 3, toks[:1]])
    assert np.array_equal(synthdata.engram_row_ids(1, padded, 3)[0], ids_all[0])


def test_engram_hash_uniformity_chi2():
    toks = synthdata.token_ids(2, 0, 4000)
    ids = synthdata.engram_row_ids(2, toks, 0).reshape(-1)
    buckets = np.bincount(ids >> 16, minlength=64)  # 64 buckets of 2^16 rows
    exp = ids.size / 64
    chi2 = float(((buckets - exp) ** 2 / exp).sum())
    assert chi2 < 120  # 63 dof: p ~ 1e-5 threshold
