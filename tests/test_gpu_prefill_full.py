"""Prefill parity at the full prefill-chunk shape (T = 4096, d_model 4096,
384 experts top-6, d_ff 2048), element by element on sampled pairs.

The routed experts are checked per (token, slot) pair: with a layer that has
no shared expert and one-hot mixing weights on slot j, the float32 output of
a token is exactly that pair's expert output y[t, j] (the combine adds one
term).  Every pair of a few chosen experts is compared with the oracle: the
most and the least loaded expert (ragged tails of the largest and smallest
groups), the median one, and two drawn at random -- together they hold the
first and last row of many 48-token gate/up chunks and 32-pair down chunks.
The shared expert is checked the same way with all routed weights zero."""
import dataclasses

import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import moe

from gpu_util import device_layer, oracle_layer, x_device

pytestmark = pytest.mark.gpu

# float32 outputs: exact weights and activations, float32 accumulation, h as
# a bf16 hi + lo pair (relative rounding 2^-17)
TOL_F32 = 1e-4


def _setup(lam, shared):
    cfg = dataclasses.replace(synthdata.CONFIGS["prefill"], zipf_lambda=lam, shared=shared)
    ld = synthdata.LayerData(cfg, 1)
    layer = device_layer(ld)
    x = x_device(ld)
    ws = bm.workspace(layer, cfg.T, bm.MODE_PREFILL)
    bias = torch.from_numpy(ld.bias()).cuda()
    ids, _ = bm.route(layer, x, ws, bias=bias)
    return cfg, ld, layer, x, ws, ids


def _slot_outputs(layer, x, ids, ws, j):
    T, k = ids.shape
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    w[:, j] = 1.0
    y = bm.expert_ffn(layer, x, ids, w, ws, out_dtype=torch.float32, mode=bm.MODE_PREFILL)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("lam", [0.3, 1.0])
def test_prefill_routed_pairs_full_shape(lam):
    cfg, ld, layer, x, ws, ids = _setup(lam, shared=False)
    ids_h = ids.cpu().numpy()
    k = cfg.top_k
    counts = np.bincount(ids_h.reshape(-1), minlength=cfg.n_experts)
    used = np.nonzero(counts)[0]
    rng = np.random.default_rng(17)
    chosen = [int(used[np.argmax(counts[used])]), int(used[np.argmin(counts[used])]),
              int(used[np.argsort(counts[used])[len(used) // 2]])]
    chosen += [int(e) for e in rng.choice(np.setdiff1d(used, chosen), size=2, replace=False)]
    print(f"[prefill-full] lam={lam} experts {chosen} group sizes {[int(counts[e]) for e in chosen]}", flush=True)
    Y = np.stack([_slot_outputs(layer, x, ids, ws, j).cpu().numpy() for j in range(k)], axis=1)  # [T][k][D]
    # determinism: the same call again gives the same bits
    again = _slot_outputs(layer, x, ids, ws, 0).cpu().numpy()
    assert np.array_equal(again.view(np.uint32), Y[:, 0].view(np.uint32))
    ol = oracle_layer(ld)
    xv = ld.x_values()
    n_pairs, worst = 0, 0.0
    for e in chosen:
        toks, slots = np.nonzero(ids_h == e)
        ref = moe.ffn(xv[toks], ol.expert_matrix("gate", e), ol.expert_matrix("up", e), ol.expert_matrix("down", e))
        err = moe_err = float(np.max(np.abs(Y[toks, slots] - ref) / np.maximum(
            np.abs(ref), np.sqrt(np.mean(ref * ref, axis=1, keepdims=True)))))
        print(f"[parity] expert {e}: {len(toks)} pairs, max rel err {moe_err:.3e}", flush=True)
        worst = max(worst, err)
        n_pairs += len(toks)
        ol._cache.clear()
    assert n_pairs >= 200
    assert worst < TOL_F32


def test_prefill_shared_expert_full_shape():
    cfg, ld, layer, x, ws, ids = _setup(0.3, shared=True)
    w = torch.zeros((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
    y = bm.expert_ffn(layer, x, ids, w, ws, out_dtype=torch.float32, mode=bm.MODE_PREFILL)
    torch.cuda.synchronize()
    # tokens at the edges of 64-token M-tiles and a random draw
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, 63, 64, 127, 2048, cfg.T - 64, cfg.T - 1],
                                       rng.choice(cfg.T, size=57, replace=False)]))
    ol = oracle_layer(ld)
    ref = moe.shared_output(ol, ld.x_values()[sample])
    yv = y.cpu().numpy()[sample].astype(np.float64)
    err = float(np.max(np.abs(yv - ref) / np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref, axis=1, keepdims=True)))))
    print(f"[parity] shared expert: {len(sample)} tokens, max rel err {err:.3e}", flush=True)
    assert err < TOL_F32
