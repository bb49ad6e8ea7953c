"""GPU parity of the router variants (moe_route_ex) against the oracle:
selection-only bias, sqrt-softplus scores, hash-routed rows, and the bad
token / table entry records.  Selections must be valid top-k of the oracle's
selection scores under the tie rule (exact for table rows); weights within
2e-5 of the oracle's weights for the device's selection."""
import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import compare, moe

from gpu_util import device_layer, x_device

pytestmark = pytest.mark.gpu


def _check(ld, T, tag, score, select_bias=None, logit_bias=None, table=None, tok=None):
    cfg = ld.cfg
    layer = device_layer(ld, host_bytes=cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    ws = bm.workspace(layer, T)
    cuda = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a).astype(dt)).cuda()
    ids, w = bm.route_ex(layer, x, ws, score=score, logit_bias=cuda(logit_bias, np.float32),
                         select_bias=cuda(select_bias, np.float32), hash_table=cuda(table, np.int32),
                         token_ids=cuda(tok, np.int32))
    torch.cuda.synchronize()
    ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy()
    xv = ld.x_values(tag, T)
    sname = moe.SCORE_SOFTMAX if score == bm.SCORE_SOFTMAX else moe.SCORE_SQRT_SOFTPLUS
    hash_ids = None if table is None else table[tok]
    r_ids, _, L, sel = moe.route_variant(xv, ld.router(), cfg.top_k, logit_bias=logit_bias, select_bias=select_bias,
                                         score=sname, hash_ids=hash_ids)
    if table is None:
        for t in range(T):
            assert compare.valid_selection(ids_h[t], sel[t], cfg.top_k), (t, ids_h[t], r_ids[t])
    else:
        assert np.array_equal(ids_h, r_ids)
    sc = moe.route_scores(L, sname)
    g = np.take_along_axis(sc, ids_h.astype(np.int64), axis=1)
    want = g / g.sum(axis=1, keepdims=True)
    assert np.allclose(w_h, want, rtol=2e-5, atol=1e-7)
    return ids_h, ws


@pytest.mark.parametrize("cfg_name,T", [("decode", 1), ("verify", 5), ("tiny", 8)])
@pytest.mark.parametrize("score", [bm.SCORE_SOFTMAX, bm.SCORE_SQRT_SOFTPLUS])
def test_selection_bias(cfg_name, T, score):
    ld = synthdata.LayerData(synthdata.CONFIGS[cfg_name], 21)
    E = ld.cfg.n_experts
    rng = np.random.default_rng(100 + T)
    # a bias of the size of the scores, so that it changes some selections
    scale = 2.0 / E if score == bm.SCORE_SOFTMAX else 0.02
    b = rng.standard_normal(E) * scale
    ids_b, _ = _check(ld, T, 40 + T, score, select_bias=b)
    ids_0, _ = _check(ld, T, 40 + T, score)
    if cfg_name != "tiny":
        assert not np.array_equal(ids_b, ids_0)  # the bias changed the selection somewhere


def test_selection_bias_with_logit_bias_prefill_shape():
    # T = 300 (router tile kernel), Zipf logit bias on top of a selection bias
    cfg = synthdata.Config("pf_route", 300, 4096, 2048, 384, 6, "bf16", True, zipf_lambda=1.0)
    ld = synthdata.LayerData(cfg, 22)
    rng = np.random.default_rng(3)
    _check(ld, 300, 5, bm.SCORE_SQRT_SOFTPLUS, select_bias=rng.standard_normal(384) * 0.02,
           logit_bias=ld.bias())


@pytest.mark.parametrize("score", [bm.SCORE_SOFTMAX, bm.SCORE_SQRT_SOFTPLUS])
def test_hash_routed_rows(score):
    ld = synthdata.LayerData(synthdata.CONFIGS["verify"], 23)
    E, k, T, vocab = 384, 6, 5, 1000
    rng = np.random.default_rng(9)
    table = np.stack([rng.choice(E, size=k, replace=False) for _ in range(vocab)])
    tok = rng.integers(0, vocab, size=T)
    _, ws = _check(ld, T, 50, score, table=table, tok=tok)
    assert bm.read_status(bm.ws_status(ws))[0] == 0


def test_hash_bad_token_and_table_entry():
    ld = synthdata.LayerData(synthdata.CONFIGS["verify"], 24)
    layer = device_layer(ld)
    E, k, T, vocab = 384, 6, 5, 16
    rng = np.random.default_rng(10)
    table = np.stack([rng.choice(E, size=k, replace=False) for _ in range(vocab)]).astype(np.int32)
    table[3, 2] = E + 5  # an entry outside the experts
    tok = np.array([1, 3, vocab + 2, 0, -4], dtype=np.int32)
    x = x_device(ld, 51, T)
    ws = bm.workspace(layer, T)
    ids, w = bm.route_ex(layer, x, ws, hash_table=torch.from_numpy(table).cuda(),
                         token_ids=torch.from_numpy(tok).cuda())
    code, detail = bm.read_status(bm.ws_status(ws))
    ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy()
    assert code == bm.DEV_BAD_EXPERT | bm.DEV_BAD_TOKEN
    assert detail == 2  # the smallest recorded index (token 2; pair 1*6+2 = 8 is larger)
    assert np.all(ids_h[2] == -1) and np.all(w_h[2] == 0) and np.all(ids_h[4] == -1)
    assert w_h[1, 2] == 0 and ids_h[1, 2] == E + 5
    assert np.allclose(w_h[[0, 1, 3]].sum(axis=1), 1.0, rtol=1e-6)
