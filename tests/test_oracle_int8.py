"""Pins for oracle.int8_mode: quantiser bounds and ties (closed forms), the
integer row dots against the dot of the dequantised operands, a hand-worked
super-block, and the int8 layer against the float64 layer."""
import math
from fractions import Fraction

import numpy as np

import synthdata
from oracle import formats, int8_mode, moe


def test_quantizer_bounds_and_zero_block():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((6, 256)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    v[2, 32:64] = 0.0  # one all-zero block
    q, d, s = int8_mode.quantize_blocks(v)
    assert q.dtype == np.int8 and d.shape == (6, 8) and s.shape == (6, 16)
    qb = q.astype(np.int64).reshape(6, 8, 32)
    vb = v.astype(np.float64).reshape(6, 8, 32)
    amax = np.abs(vb).max(-1)
    live = amax > 0
    # the largest magnitude of every live block maps to +-127, nothing beyond
    assert np.all(np.abs(qb).max(-1)[live] == 127) and np.abs(qb).max() <= 127
    # reconstruction within half a step (plus the float32 rounding of v / d)
    dd = d.astype(np.float64)[..., None]
    assert np.all(np.abs(vb - dd * qb) <= dd * (0.5 + 128 * 2.0 ** -24) + 1e-30)
    # scale: the float32 value nearest amax / 127
    assert np.all(np.abs(d.astype(np.float64) - amax / 127) <= amax / 127 * 2.0 ** -24)
    # zero block: zero scale, zero codes, zero sums
    assert d[2, 1] == 0 and np.all(qb[2, 1] == 0) and np.all(s[2, 2:4] == 0)
    # stored sums: the float32 nearest d * (sum of the 16 codes)
    exact = np.repeat(d.astype(np.float64), 2, axis=-1) * q.astype(np.int64).reshape(6, 16, 16).sum(-1)
    assert np.all(np.abs(s.astype(np.float64) - exact) <= np.abs(exact) * 2.0 ** -24)


def test_quantizer_rounds_halves_to_even():
    v = np.zeros(32, np.float32)
    v[0] = 127.0  # amax 127 -> d = 1 exactly, q = v where v is an integer
    v[1:9] = [2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, -125.5]
    q, d, _ = int8_mode.quantize_blocks(v)
    assert d[0] == 1.0
    assert q[:9].tolist() == [127, 2, 4, -2, 0, 2, 0, 126, -126]


def _random_activation(rng, n):
    x = rng.standard_normal(n).astype(np.float32)
    q, dx, _ = int8_mode.quantize_blocks(x)
    s_exact = np.repeat(dx.astype(np.float64), 2) * q.astype(np.int64).reshape(-1, 16).sum(-1)
    x_deq = np.repeat(dx.astype(np.float64), 32) * q.astype(np.float64)
    return q, dx, s_exact, x_deq


def test_q2_rows_dot_is_the_dequantised_dot():
    rng = np.random.default_rng(1)
    rows, cols = 12, 1024
    raw = synthdata.q2_bytes(synthdata.tensor_key(5, synthdata.KIND_GATE), 0, rows * cols // 256)
    q, dx, s_exact, x_deq = _random_activation(rng, cols)
    got = int8_mode.q2_rows_dot(raw, rows, cols, q, dx, s_exact)
    want = formats.q2_matrix(raw, rows, cols) @ x_deq
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_q8_0_rows_dot_is_the_dequantised_dot():
    rng = np.random.default_rng(2)
    rows, cols = 9, 512
    raw = synthdata.q8_0_bytes(synthdata.tensor_key(5, synthdata.KIND_SH_UP), 0, rows * cols // 32)
    q, dx, _, x_deq = _random_activation(rng, cols)
    got = int8_mode.q8_0_rows_dot(raw, rows, cols, q, dx)
    want = formats.q8_0_matrix(raw, rows, cols) @ x_deq
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_hand_worked_super_block():
    # d = 1/4, dmin = 1/2, every scale nibble 2, every min nibble 1, every
    # code 3: every weight is 1/4 * 2 * 3 - 1/2 * 1 = 1.  Against 256 ones
    # (quantised to 127 steps of fp32(1/127)) the row sums to 256.
    blk = np.zeros(84, np.uint8)
    blk[0:16] = 0x12
    blk[16:80] = 0xFF
    blk[80:82] = [0x00, 0x34]  # fp16 0.25
    blk[82:84] = [0x00, 0x38]  # fp16 0.5
    x = np.ones(256, np.float32)
    q, dx, s = int8_mode.quantize_blocks(x)
    assert np.all(q == 127) and np.all(dx == np.float32(1 / 127))
    got = int8_mode.q2_rows_dot(blk, 1, 256, q, dx, s)[0]
    assert abs(got - 256.0) < 256.0 * 1e-6
    # the minimum term uses the stored sums: 16 sub-blocks of 1/2 * 1 * s
    step = Fraction(float(np.float32(1 / 127)))
    main = Fraction(1, 4) * 16 * 2 * step * 16 * 3 * 127
    mins = Fraction(1, 2) * 16 * Fraction(float(s[0]))
    assert got == float(main - mins) or math.isclose(got, float(main - mins), rel_tol=1e-15)


def _layer_with_shared(seed=3):
    cfg = synthdata.Config("int8", 4, 256, 128, 16, 2, "bf16", True)
    ld = synthdata.LayerData(cfg, seed)
    return ld, moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(), ld.expert_bytes,
                         ld.shared_bytes)


def test_int8_layer_tracks_the_float_layer():
    ld, layer = _layer_with_shared()
    x = ld.x_values(0, 4)
    ref = moe.moe_layer(layer, x)
    got = int8_mode.moe_layer_int8(layer, x)
    assert np.array_equal(got.ids, ref.ids)
    err = np.sqrt(np.mean((got.out - ref.out) ** 2)) / np.sqrt(np.mean(ref.out ** 2))
    # two 8-bit quantisations (x and h): about 0.5 % relative, never exact
    assert 1e-4 < err < 0.03, err


def test_int8_ffn_single_expert_matches_dense_int8_route():
    # the layer's expert outputs equal ffn_int8 run by hand, and the shared
    # expert path uses the Q8_0 dot (no planning or combine involved)
    ld, layer = _layer_with_shared(4)
    x = ld.x_values(1, 2)
    res = int8_mode.moe_layer_int8(layer, x)
    t = 1
    y = [int8_mode.ffn_int8(layer, int(e), x[t])[0] for e in res.ids[t]]
    ysh = int8_mode.ffn_int8(layer, -1, x[t])[0]
    out = sum(w * yy for w, yy in zip(res.weights[t], y)) + ysh
    assert np.allclose(res.out[t], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())


def _q2_block(codes: dict, sc0: int, d_bits: int) -> np.ndarray:
    """One 84-byte Q2 super-block: sub-block 0 scale sc0 (min 0), the given
    {weight index: code}, fp16 d = d_bits, dmin = 0."""
    blk = np.zeros(84, np.uint8)
    blk[0] = sc0
    for i, q in codes.items():
        byte, shift = formats.q2_code_location(i)
        blk[byte] |= q << shift
    blk[80], blk[81] = d_bits & 0xFF, d_bits >> 8
    return blk


def test_ffn_int8_requantises_h_hand_worked():
    # d_model = d_ff = 256, one expert, x = 127 everywhere: x quantises
    # exactly (d = 1, q = 127).  Gate rows 0 and 1 have weight 0 = 2^-10 (d =
    # 2^-10 = fp16 0x1400, sc 1, code 1): g = 127/1024 for both.  Up row 0 has
    # code 3 at weight 0 (u = 381/1024), up row 1 code 1 (u = 127/1024); all
    # other rows are zero, so h = silu(127/1024) * (3, 1, 0, ...) * 127/1024.
    # h quantises in block 0 with d_h = fp32(h_0/127): q_0 = 127 and
    # q_1 = rint(127/3) = rint(42.33) = 42.  Down row 0 has weights 1 at
    # columns 0 and 1 (d = 1.0 = 0x3C00, sc 1, code 1), the other rows zero:
    # y_0 = d_h * (127 + 42) = 169 d_h, where the unquantised h would give
    # h_0 + h_1 = 169.33 d_h.
    D = F = 256
    zero = np.zeros(84, np.uint8)
    gate = np.concatenate([_q2_block({0: 1}, 1, 0x1400)] * 2 + [zero] * (F - 2))
    up = np.concatenate([_q2_block({0: 3}, 1, 0x1400), _q2_block({0: 1}, 1, 0x1400)] + [zero] * (F - 2))
    down = np.concatenate([_q2_block({0: 1, 1: 1}, 1, 0x3C00)] + [zero] * (D - 1))
    mats = {"gate": gate, "up": up, "down": down}
    layer = moe.Layer(D, F, 1, 1, np.zeros((1, D), np.float32), lambda kind, e: mats[kind])
    y, h = int8_mode.ffn_int8(layer, 0, np.full(D, 127.0, np.float32))
    g = 127 / 1024
    s = g / (1 + math.exp(-g))
    h0 = s * 381 / 1024
    assert math.isclose(h[0], h0, rel_tol=1e-15) and math.isclose(h[1], h0 / 3, rel_tol=1e-15)
    assert np.all(h[2:] == 0)
    d_h = float(np.float32(np.float32(h0) / np.float32(127)))
    assert math.isclose(y[0], 169 * d_h, rel_tol=1e-12), (y[0], 169 * d_h)
    assert abs(y[0] - (h0 + h0 / 3)) > 1e-3 * abs(y[0])  # h is not used unquantised
    assert np.all(y[1:] == 0)


def test_ffn_int8_rows_equals_per_token_ffn():
    # the batched form parses each matrix once and runs the same arithmetic
    cfg = synthdata.Config("i8rows", 3, 256, 256, 4, 2, "f32", False)
    ld = synthdata.LayerData(cfg, 5)
    layer = moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(), ld.expert_bytes)
    X = ld.x_values(2).astype(np.float32)
    got = int8_mode.ffn_int8_rows(layer, 2, X)
    for i in range(len(X)):
        assert np.array_equal(got[i], int8_mode.ffn_int8(layer, 2, X[i])[0])
