"""Int8 activation numerics of the expert FFN (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

"Strata-DSV4.1" README, §Results and the decode notes of its
"DeepSeek-V4-Flash (0731) engine" section: the expert products there run on
integer dot products (dp4a for decode, int8 tensor cores for the prompt)
against activations quantised to 8-bit blocks of 32 values with one scale
each ("q8_1"), which moves results slightly against the float path.  The
pages name the block format but print neither the quantiser nor the integer
formulation, so this module fixes them (the design notes list each reading):

* quantiser, per block of 32 float32 values v: amax = max |v|,
  d = float32(amax / 127), q = round-half-even(float32(v / d)) (all q = 0
  when amax = 0), and per 16-value half b the stored sum
  s_b = float32(d * sum_{k in b} q_k); the float32 decisions are those of
  IEEE division and rounding, so any implementation reproduces them bit for
  bit;
* a 2-bit super-block row against quantised activations, per super-block:
  d_w * sum_b sc_b dx_c(b) sum_{k in b} q2_k q_k  -  dmin_w * sum_b m_b s_b,
  the integer sums exact, sub-block b (16 weights) inside activation block
  c(b) = b // 2; this is the dot product of the dequantised weights with the
  dequantised activations d * q, except that the minimum term uses the
  stored s_b;
* a Q8_0 row: sum over blocks of d_w dx sum qw qx (exact integer sums);
* the FFN: x (float32) quantised, gate and up rows dotted, h = silu(g) * u
  in float64, h rounded to float32 and quantised, down rows dotted; routing
  and the combine are those of the float path.

The arithmetic on integers is exact here (int64); the float combination is
float64.
"""
from __future__ import annotations

import numpy as np

from . import formats, moe

QBLOCK = 32     # activation values per quantisation block
HALF = 16       # values per stored sum (one 2-bit sub-block)


def quantize_blocks(v) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """float32 [..., C] (C a multiple of 32) -> (q int8 [..., C],
    d float32 [..., C/32], s float32 [..., C/16])."""
    v = np.asarray(v, dtype=np.float32)
    if v.shape[-1] % QBLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    lead = v.shape[:-1]
    blk = v.reshape(*lead, -1, QBLOCK)
    amax = np.max(np.abs(blk), axis=-1)
    d = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1))
    with np.errstate(invalid="ignore"):
        r = np.rint((blk / safe[..., None]).astype(np.float32))
    q = np.where(d[..., None] > 0, r, 0).astype(np.int64)
    if np.any(np.abs(q) > 127):
        raise AssertionError("quantised value outside [-127, 127]")
    halves = q.reshape(*lead, -1, HALF).sum(axis=-1)  # exact integers
    d_half = np.repeat(d, QBLOCK // HALF, axis=-1).astype(np.float64)
    s = (d_half * halves).astype(np.float32)  # one rounding of the exact product
    return q.reshape(*lead, -1).astype(np.int8), d, s


def _q2_parse(raw: np.ndarray, n_rows: int, n_cols: int):
    """The fields of a row-major [n_rows][n_cols] Q2 matrix, per sub-block of
    the flattened matrix: codes [nsub][16], sc, m, and d, dmin of its
    super-block."""
    if n_cols % QBLOCK:
        raise ValueError("n_cols must be a multiple of 32")
    qw, sc, m, d, dmin = formats.q2_fields(np.asarray(raw, dtype=np.uint8).reshape(-1, formats.Q2_BLOCK_BYTES))
    nsub = n_rows * n_cols // HALF                       # sub-blocks of the flattened matrix
    sb = np.arange(nsub) // 16                             # super-block of each sub-block
    return (qw.reshape(nsub, HALF).astype(np.int64), sc.reshape(-1).astype(np.float64),
            m.reshape(-1).astype(np.float64), d[sb], dmin[sb], n_rows, n_cols)


def _q2_dot(parsed, q, dx, s) -> np.ndarray:
    qw, sc, m, d, dmin, n_rows, n_cols = parsed
    nsub = qw.shape[0]
    per_row = n_cols // HALF
    j = np.arange(nsub) % per_row                          # sub-block's column group in its row
    qa = np.asarray(q, dtype=np.int64).reshape(per_row, HALF)
    dots = np.einsum("bk,bk->b", qw, qa[j])              # exact integer sums
    dxb = np.asarray(dx, dtype=np.float64)[j // 2]
    sj = np.asarray(s, dtype=np.float64)[j]
    term = d * (sc * dxb * dots) - dmin * (m * sj)
    return term.reshape(n_rows, per_row).sum(-1)


def q2_rows_dot(raw: np.ndarray, n_rows: int, n_cols: int, q, dx, s) -> np.ndarray:
    """Rows of a row-major [n_rows][n_cols] Q2 matrix against one quantised
    activation vector (q [n_cols] int8, dx [n_cols/32], s [n_cols/16]).
    Returns float64 [n_rows].

    The super-blocks tile the flattened matrix (a row narrower than 256
    shares a super-block with the next row); every 16-weight sub-block lies in
    one row, and its columns in one activation block since n_cols is a
    multiple of 32."""
    return _q2_dot(_q2_parse(raw, n_rows, n_cols), q, dx, s)


def q8_0_rows_dot(raw: np.ndarray, n_rows: int, n_cols: int, q, dx) -> np.ndarray:
    """Rows of a row-major [n_rows][n_cols] Q8_0 matrix against one quantised
    activation vector.  Returns float64 [n_rows]."""
    nb = n_cols // formats.Q8_BLOCK_WEIGHTS
    blocks = np.asarray(raw, dtype=np.uint8).reshape(n_rows, nb, formats.Q8_BLOCK_BYTES)
    dw = formats.half_bits_to_f64(blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8))
    qw = blocks[..., 2:].view(np.int8).astype(np.int64)                   # [row][block][32]
    qa = np.asarray(q, dtype=np.int64).reshape(nb, formats.Q8_BLOCK_WEIGHTS)
    dots = np.einsum("rbk,bk->rb", qw, qa)
    return (dw * np.asarray(dx, dtype=np.float64)[None, :] * dots).sum(-1)


def _matrix_dot(layer: moe.Layer, kind: str, e: int, act) -> np.ndarray:
    rows, cols = (layer.d_model, layer.d_ff) if kind == "down" else (layer.d_ff, layer.d_model)
    q, dx, s = act
    if e < 0:
        return q8_0_rows_dot(layer.shared_bytes(kind), rows, cols, q, dx)
    return q2_rows_dot(layer.expert_bytes(kind, e), rows, cols, q, dx, s)


def ffn_int8(layer: moe.Layer, e: int, x_row) -> tuple[np.ndarray, np.ndarray]:
    """One token through expert e (-1: the shared expert) in int8 numerics.
    x_row: the token's float32 values.  Returns (y float64 [d_model],
    h float64 [d_ff] before its quantisation)."""
    xa = quantize_blocks(np.asarray(x_row, dtype=np.float32))
    g = _matrix_dot(layer, "gate", e, xa)
    u = _matrix_dot(layer, "up", e, xa)
    h = moe.silu(g) * u
    ha = quantize_blocks(h.astype(np.float32))
    return _matrix_dot(layer, "down", e, ha), h


def ffn_int8_rows(layer: moe.Layer, e: int, X) -> np.ndarray:
    """ffn_int8 of routed expert e for each row of X (float32 values), each
    matrix parsed once.  Returns y float64 [rows][d_model]."""
    D, F = layer.d_model, layer.d_ff
    pg = _q2_parse(layer.expert_bytes("gate", e), F, D)
    pu = _q2_parse(layer.expert_bytes("up", e), F, D)
    pd = _q2_parse(layer.expert_bytes("down", e), D, F)
    out = np.zeros((len(X), D))
    for i, x_row in enumerate(X):
        xa = quantize_blocks(np.asarray(x_row, dtype=np.float32))
        h = moe.silu(_q2_dot(pg, *xa)) * _q2_dot(pu, *xa)
        out[i] = _q2_dot(pd, *quantize_blocks(h.astype(np.float32)))
    return out


def moe_layer_int8(layer: moe.Layer, x: np.ndarray, bias=None, ids=None) -> moe.LayerResult:
    """Steps 1-5 with the expert FFNs in int8 numerics; routing (float64 from
    the same inputs) and the combine as in :func:`moe.moe_layer`.  x holds the
    float values of the inputs (BF16 or float32 values, exact in float32)."""
    x = np.asarray(x, dtype=np.float64)
    r_ids, r_w, L = moe.route(x, layer.w_router, layer.top_k, bias)
    if ids is not None:
        r_ids = np.asarray(ids, dtype=np.int64)
        r_w = moe.weights_for_selection(L, r_ids)
    T, k = r_ids.shape
    y = np.zeros((T, k, layer.d_model))
    for t in range(T):
        for j in range(k):
            y[t, j] = ffn_int8(layer, int(r_ids[t, j]), x[t])[0]
    ysh = np.zeros((T, layer.d_model))
    if layer.shared_bytes is not None:
        for t in range(T):
            ysh[t] = ffn_int8(layer, -1, x[t])[0]
    return moe.LayerResult(r_ids, r_w, L, moe.combine(r_w, y, ysh))
