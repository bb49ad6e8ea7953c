"""GPU parity when a token names one expert in two slots (a hash-routing table
row or a caller's ids can): the expert is served once per token, at its first
slot, the later slot contributes nothing, and BITMOE_DEV_DUP_EXPERT is recorded
with the smallest such pair index.  Runs the plan alone, the decode path (T=1,
T=5), the prefill path (T=300, several M-tiles per group), and a hash-routed
layer whose table repeats an entry; each against the oracle on the same ids and
weights."""
import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import compare, moe

from gpu_util import device_layer, oracle_layer, x_device

pytestmark = pytest.mark.gpu


def _repeat_ids(rng, T, k, E, every=3):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    for t in range(0, T, every):
        j = 1 + t % (k - 1)
        ids[t, j] = ids[t, (j - 1) // 2]  # repeat an earlier slot
    return ids


def _first_repeat(ids):
    T, k = ids.shape
    for t in range(T):
        for j in range(k):
            if ids[t, j] in ids[t, :j]:
                return t * k + j
    return None


def test_plan_with_repeats_bit_exact():
    rng = np.random.default_rng(1)
    T, k, E = 300, 6, 384
    ids = _repeat_ids(rng, T, k, E)
    status = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = bm.plan(torch.from_numpy(ids).cuda(), E, status=status)
    ref = moe.plan(ids, E)
    n = ref.perm.size
    assert n < T * k
    assert np.array_equal(out["counts"].cpu().numpy(), ref.counts)
    assert np.array_equal(out["offsets"].cpu().numpy(), ref.offsets)
    assert np.array_equal(out["perm"].cpu().numpy()[:n], ref.perm)
    code, detail = bm.read_status(status)
    assert code == bm.DEV_DUP_EXPERT and detail == _first_repeat(ids)


def _ffn_check(ld, ids_h, w_h, tag, mode, out_dtype=torch.float32):
    T = ids_h.shape[0]
    layer = device_layer(ld, host_bytes=ld.cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    ws = bm.workspace(layer, T, mode)
    y = bm.expert_ffn(layer, x, torch.from_numpy(ids_h.astype(np.int32)).cuda(),
                      torch.from_numpy(w_h.astype(np.float32)).cuda(), ws, out_dtype=out_dtype, mode=mode)
    code, detail = bm.read_status(bm.ws_status(ws))
    ol = oracle_layer(ld)
    xv = ld.x_values(tag, T)
    y_pairs = moe.expert_outputs(ol, xv, ids_h)          # zero for the repeated slots
    want = moe.combine(w_h.astype(np.float64), y_pairs, moe.shared_output(ol, xv))
    err = compare.max_rel_error(y.float().cpu().numpy().astype(np.float64), want)
    print(f"[parity] repeats {ld.cfg.name} T={T} mode={mode} max rel err {err:.3e}", flush=True)
    return err, code, detail


@pytest.mark.parametrize("T,mode", [(1, bm.MODE_DECODE), (5, bm.MODE_DECODE), (5, bm.MODE_DECODE_INT8)])
def test_decode_with_repeats(T, mode):
    ld = synthdata.LayerData(synthdata.CONFIGS["verify"], 31)
    xv = ld.x_values(60 + T, T)
    ids_h, w, L = moe.route(xv, ld.router(), 6)
    ids_h = ids_h.astype(np.int32)
    ids_h[0, 3] = ids_h[0, 1]
    if T > 1:
        ids_h[T - 1, 5] = ids_h[T - 1, 0]
        ids_h[1, 2] = ids_h[0, 0]  # another token's expert: a legitimate share, not a repeat
    if mode == bm.MODE_DECODE_INT8:
        from oracle import int8_mode
        layer = device_layer(ld)
        x = x_device(ld, 60 + T, T)
        ws = bm.workspace(layer, T, mode)
        y = bm.expert_ffn(layer, x, torch.from_numpy(ids_h).cuda(), torch.from_numpy(w.astype(np.float32)).cuda(),
                          ws, out_dtype=torch.float32, mode=mode)
        code, detail = bm.read_status(bm.ws_status(ws))
        ol = oracle_layer(ld)
        served = moe.served_pairs(ids_h, 384)
        y_pairs = np.zeros((T, 6, 4096))
        for t in range(T):
            for j in range(6):
                if served[t, j]:
                    y_pairs[t, j] = int8_mode.ffn_int8(ol, int(ids_h[t, j]), xv[t])[0]
        ysh = np.stack([int8_mode.ffn_int8(ol, -1, xv[t])[0] for t in range(T)])
        want = moe.combine(w.astype(np.float32).astype(np.float64), y_pairs, ysh)
        err = compare.max_rel_error(y.cpu().numpy().astype(np.float64), want)
        assert err < 5e-3
    else:
        err, code, detail = _ffn_check(ld, ids_h, w, 60 + T, mode)
        assert err < 1e-4
    assert code == bm.DEV_DUP_EXPERT and detail == _first_repeat(ids_h)


@pytest.mark.parametrize("T,lam", [(300, 1.0), (70, 0.0)])
def test_prefill_with_repeats(T, lam):
    cfg = synthdata.Config("pf_rep", T, 1024, 512, 16, 4, "bf16", True, zipf_lambda=lam)
    ld = synthdata.LayerData(cfg, 32)
    xv = ld.x_values(0, T)
    ids_h, w, _ = moe.route(xv, ld.router(), 4, ld.bias())
    ids_h = ids_h.astype(np.int32)
    for t in range(0, T, 4):
        ids_h[t, 1 + t % 3] = ids_h[t, 0]  # popular experts repeated across several M-tiles
    err, code, detail = _ffn_check(ld, ids_h, w, 0, bm.MODE_PREFILL)
    assert err < 1e-4
    assert code == bm.DEV_DUP_EXPERT and detail == _first_repeat(ids_h)


@pytest.mark.parametrize("mode", [bm.MODE_DECODE, bm.MODE_PREFILL])
def test_hash_table_row_with_repeat(mode):
    ld = synthdata.LayerData(synthdata.CONFIGS["verify"], 33)
    E, k, T, vocab = 384, 6, 5, 64
    rng = np.random.default_rng(11)
    table = np.stack([rng.choice(E, size=k, replace=False) for _ in range(vocab)]).astype(np.int32)
    table[7, 4] = table[7, 1]
    tok = np.array([7, 2, 7, 9, 0], dtype=np.int32)
    layer = device_layer(ld)
    x = x_device(ld, 70, T)
    ws = bm.workspace(layer, T, mode)
    ids, w = bm.route_ex(layer, x, ws, hash_table=torch.from_numpy(table).cuda(),
                         token_ids=torch.from_numpy(tok).cuda())
    code, detail = bm.read_status(bm.ws_status(ws))
    assert code == bm.DEV_DUP_EXPERT and detail == 0 * k + 4
    ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy()
    xv = ld.x_values(70, T)
    r_ids, r_w, _, _ = moe.route_variant(xv, ld.router(), k, hash_ids=table[tok])
    assert np.array_equal(ids_h, r_ids)
    assert w_h[0, 4] == 0 and w_h[2, 4] == 0
    assert np.allclose(w_h, r_w, rtol=2e-5, atol=1e-7)
    ws2 = bm.workspace(layer, T, mode)
    y = bm.expert_ffn(layer, x, ids, w, ws2, out_dtype=torch.float32, mode=mode)
    code2, detail2 = bm.read_status(bm.ws_status(ws2))
    assert code2 == bm.DEV_DUP_EXPERT and detail2 == 4
    ol = oracle_layer(ld)
    want = moe.combine(w_h.astype(np.float64), moe.expert_outputs(ol, xv, ids_h), moe.shared_output(ol, xv))
    assert compare.max_rel_error(y.cpu().numpy().astype(np.float64), want) < 1e-4
