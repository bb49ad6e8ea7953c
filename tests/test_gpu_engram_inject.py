"""GPU parity of engram_inject against the oracle: every updated BF16 value
within one BF16 step of the oracle's (the GPU sums in float32) and nearly all
identical, gates within 1e-5, masked positions untouched bit for bit."""
import math

import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import engram, engram_inject as ei, formats

pytestmark = pytest.mark.gpu


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.uint16).view(np.int16)).cuda()


def _ulp_diff(a, b):
    """Distance in BF16 steps between bit patterns of the same sign."""
    a = np.asarray(a, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ka - kb)


def _inputs(T, n_rows, W, seed, rows=None):
    if rows is None:
        rows = synthdata.activations_bf16(seed, 83, T * n_rows, 256).reshape(T, n_rows, 256)
    # scale the weight so the keys have about unit RMS over these rows
    row_rms = math.sqrt(float(np.mean(formats.bf16_to_f64(rows) ** 2))) or 1.0
    w = synthdata.engram_kv_weight(seed, n_rows, W, scale=1.0 / row_rms)
    qn, kn = synthdata.engram_branch_norms(seed, W)
    res = synthdata.residual_branches(seed, T, W)
    return rows, w, qn, kn, res


def _run(rows, w, qn, kn, eps, res, mask):
    out = _bits_dev(res)
    gate = torch.empty((res.shape[0], 4), dtype=torch.float32, device="cuda")
    bm.engram_inject(_bits_dev(rows), _bits_dev(w), torch.from_numpy(qn).cuda(), torch.from_numpy(kn).cuda(), eps,
                     out, mask=None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda(),
                     gate_out=gate)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), gate.cpu().numpy()


def _bf16_step(x):
    """Spacing of BF16 values at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _compare(got, g_got, want, g_want, rows, w, res):
    """The GPU sums the projection in float32, so its BF16 value can sit one
    step off the oracle's near a rounding boundary, and its gate carries float32
    error; the exact updates then differ by at most gate * step(value) +
    |gate error| * |value|, and each side rounds once more (half a step of the
    result each).  Nearly every element must still be identical."""
    d = _ulp_diff(got, want)
    T, H, W = res.shape
    v = formats.bf16_to_f64(formats.bf16_array_from_f64(ei.kv_projection(rows, w)[:, H * W:]))[:, None, :]
    g = g_want[:, :, None]
    want_f = formats.bf16_to_f64(want)
    got_f = formats.bf16_to_f64(got)
    bound = g * _bf16_step(v) + 1e-5 * np.abs(v) + np.maximum(_bf16_step(want_f), _bf16_step(got_f))
    err = np.abs(got_f - want_f)
    assert np.all(err <= bound), (d.max(), float(np.max(err - bound)))
    assert np.mean(d == 0) > 0.999, np.mean(d == 0)
    assert np.allclose(g_got, g_want, rtol=0, atol=1e-5)
    print(f"[parity] identical {np.mean(d == 0):.6f}, max steps apart {d.max()}")


@pytest.mark.parametrize("T,n_rows,W", [(1, 8, 4096), (5, 8, 4096), (13, 2, 256), (9, 24, 512),
                                         (16, 2, 256), (17, 4, 256), (64, 2, 512), (130, 2, 256),
                                         (1, 24, 5120), (5, 24, 5120), (37, 24, 5120),
                                         (1, 32, 8192), (20, 32, 8192)])  # largest rows and width
def test_inject_matches_oracle(T, n_rows, W):
    rows, w, qn, kn, res = _inputs(T, n_rows, W, 100 + T)
    mask = np.ones(T, dtype=bool)
    if T > 2:
        mask[1] = False  # one masked position
    got, g = _run(rows, w, qn, kn, 1e-6, res, mask)
    want, gw = ei.inject(rows, w, qn.astype(np.float64), kn.astype(np.float64), 1e-6, res, mask=mask)
    _compare(got, g, want, gw, rows, w, res)
    if T > 2:
        assert np.array_equal(got[1], res[1]) and g[1].tolist() == [0.0] * 4
    print(f"[parity] engram_inject T={T} rows={n_rows} W={W}: gates {g.min():.3f}..{g.max():.3f}")


def test_inject_on_gathered_engram_rows():
    # rows decoded by the library's own gather from a table in the verify format
    n_tab, T, n_rows, W = 4096, 5, 8, 4096
    lut = torch.from_numpy(synthdata.half_normal_lut().view(np.int16).copy()).cuda()
    table = torch.empty(n_tab * 264, dtype=torch.uint8, device="cuda")
    bm.fill(table, synthdata.tensor_key(3, synthdata.KIND_ENGRAM, 0), bm.FILL_ENGRAM, lut)
    table = table.view(n_tab, 264)
    ids = torch.from_numpy(np.random.default_rng(4).integers(0, n_tab, size=(T, n_rows))).cuda()
    rows_dev = bm.engram_gather(table, ids.view(-1)).view(T, n_rows, 256)
    torch.cuda.synchronize()
    rows = rows_dev.cpu().numpy().view(np.uint16)
    # the oracle decodes the same table rows itself
    host = table.cpu().numpy()
    assert np.array_equal(engram.decode_rows(host[ids.cpu().numpy().reshape(-1)]).reshape(T, n_rows, 256), rows)
    _, w, qn, kn, res = _inputs(T, n_rows, W, 7, rows=rows)
    got, g = _run(rows, w, qn, kn, 1e-6, res, None)
    want, gw = ei.inject(rows, w, qn.astype(np.float64), kn.astype(np.float64), 1e-6, res)
    _compare(got, g, want, gw, rows, w, res)


def test_inject_large_batch_sampled_tokens():
    # the real model's shape at a prefill-sized batch (64-token tiles and a
    # ragged last tile): every position is computed on the device, the oracle
    # recomputes a sample of them (positions are independent of each other)
    T, n_rows, W = 1000, 24, 5120
    rows, w, qn, kn, res = _inputs(T, n_rows, W, 9)
    mask = np.ones(T, dtype=bool)
    mask[[3, 700]] = False
    got, g = _run(rows, w, qn, kn, 1e-6, res, mask)
    idx = np.array([0, 1, 3, 63, 64, 127, 511, 700, 959, 960, 999])
    want, gw = ei.inject(rows[idx], w, qn.astype(np.float64), kn.astype(np.float64), 1e-6, res[idx],
                         mask=mask[idx])
    _compare(got[idx], g[idx], want, gw, rows[idx], w, res[idx])
    for t in (3, 700):
        assert np.array_equal(got[t], res[t]) and g[t].tolist() == [0.0] * 4
    # run twice: the same inputs give the same bits (residual and gates)
    got2, g2 = _run(rows, w, qn, kn, 1e-6, res, mask)
    assert np.array_equal(got2, got) and np.array_equal(g2.view(np.uint32), g.view(np.uint32))


def test_inject_every_position_masked():
    # the projection still runs (wide kernel at T = 20); no residual element
    # changes and every gate reads 0
    T, n_rows, W = 20, 2, 256
    rows, w, qn, kn, res = _inputs(T, n_rows, W, 31)
    got, g = _run(rows, w, qn, kn, 1e-6, res, np.zeros(T, dtype=bool))
    assert np.array_equal(got, res) and not g.any()
