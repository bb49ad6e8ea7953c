"""Pins of the oracle's Engram injection: the gate's closed forms and sign
symmetry, masking, a zero value, invariance of the gate under scaling of the
branch or of the keys, a projection by unit rows, and a hand-worked case."""
import math

import numpy as np

from oracle import engram_inject as ei, formats


def _bf16(a):
    return formats.bf16_array_from_f64(np.asarray(a, dtype=np.float64))


def _case(T=3, n_rows=2, W=8, seed=0):
    rng = np.random.default_rng(seed)
    K = n_rows * 256
    rows = _bf16(rng.standard_normal((T, n_rows, 256)))
    w = _bf16(rng.standard_normal((5 * W, K)) / math.sqrt(K))
    qn = 1.0 + 0.1 * rng.standard_normal((4, W))
    kn = 1.0 + 0.1 * rng.standard_normal((4, W))
    res = _bf16(rng.standard_normal((T, 4, W)))
    return rows, w, qn, kn, res


def test_gate_closed_forms_and_symmetry():
    g = ei.gate_of([0.0, -4.0, 4.0, 1e-9, -1e-9, 0.25])
    assert abs(g[0] - 1.0 / (1.0 + math.exp(-1e-3))) < 1e-15  # |dot| floored at 1e-6, sign of +0
    assert abs(g[1] - 1.0 / (1.0 + math.exp(2.0))) < 1e-15
    assert abs(g[1] + g[2] - 1.0) < 1e-15 and abs(g[3] + g[4] - 1.0) < 1e-15
    assert abs(g[5] - 1.0 / (1.0 + math.exp(-0.5))) < 1e-15


def test_masked_positions_keep_their_residual():
    rows, w, qn, kn, res = _case()
    new, g = ei.inject(rows, w, qn, kn, 1e-6, res, mask=np.array([1, 0, 1]))
    assert np.array_equal(new[1], res[1]) and np.all(g[1] == 0)
    assert not np.array_equal(new[0], res[0])


def test_zero_value_leaves_residual_unchanged():
    rows, w, qn, kn, res = _case()
    W = res.shape[2]
    w[4 * W:] = 0  # value rows
    new, g = ei.inject(rows, w, qn, kn, 1e-6, res)
    assert np.array_equal(new, res) and np.all((g > 0) & (g < 1))


def test_gate_invariant_under_scaling_branch_or_keys():
    rows, w, qn, kn, res = _case(seed=1)
    W = res.shape[2]
    _, g = ei.inject(rows, w, qn, kn, 0.0, res)
    res2 = _bf16(2.0 * formats.bf16_to_f64(res))  # exact doubling
    _, g2 = ei.inject(rows, w, qn, kn, 0.0, res2)
    assert np.allclose(g, g2, rtol=1e-13)
    w3 = w.copy()
    w3[:4 * W] = _bf16(4.0 * formats.bf16_to_f64(w[:4 * W]))  # keys x 4, value unchanged
    _, g3 = ei.inject(rows, w3, qn, kn, 0.0, res)
    assert np.allclose(g, g3, rtol=1e-13)


def test_projection_by_unit_rows():
    rows, w, qn, kn, res = _case(T=2, n_rows=2, W=4)
    K = 512
    sel = np.array([3, 100, 511, 0, 256, 7, 300, 1, 2, 5, 9, 11, 13, 17, 19, 23, 29, 31, 37, 41])
    w = np.zeros((20, K), dtype=np.uint16)
    w[np.arange(20), sel] = 0x3F80  # BF16 1.0
    kv = ei.kv_projection(rows, w)
    flat = formats.bf16_to_f64(rows).reshape(2, K)
    assert np.array_equal(kv, flat[:, sel])


def test_hand_worked_case():
    # W = 4, one token: branch 0 = (1,1,1,1), its key = (1,1,1,1), norms 1, eps 0:
    # dot = 4 / 1 / 1 / 2 = 2, gate = logistic(sqrt 2); value = 0.5 everywhere
    W, K = 4, 512
    rows = np.zeros((1, 2, 256), dtype=np.uint16)
    rows[0, 0, 0] = 0x3F80  # 1.0
    rows[0, 0, 1] = 0x3F00  # 0.5
    w = np.zeros((5 * W, K), dtype=np.uint16)
    w[0:W, 0] = 0x3F80       # key of branch 0 = input[0] = 1
    w[W:4 * W, 1] = 0x3F80   # keys of branches 1..3 = input[1] = 0.5
    w[4 * W:, 1] = 0x3F80    # value = input[1] = 0.5
    res = np.full((1, 4, W), 0x3F80, dtype=np.uint16)  # every branch = 1.0
    new, g = ei.inject(rows, w, np.ones((4, W)), np.ones((4, W)), 0.0, res)
    # branches 1..3: dot = (4 * 0.5) / 1 / 0.5 / 2 = 2 as well
    want_g = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    assert np.allclose(g[0], want_g, rtol=1e-15)
    want = formats.bf16_from_f64(1.0 + 0.5 * want_g)  # 1.402..: BF16 1.3984375 (0x3FB3)
    assert want == 0x3FB3
    assert np.all(new == want)
