"""Pins for oracle.moe: brute-force sorts, library softmax, dense brute-force MoE,
special cases that reduce to textbook routines, and plan invariants."""
import numpy as np
import pytest
import scipy.special
import torch

import synthdata
from oracle import formats, moe


def _tiny_layer(seed=1, cfg=None, shared=False):
    cfg = cfg or synthdata.CONFIGS["tiny"]
    ld = synthdata.LayerData(cfg, seed)
    return ld, moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(),
                         ld.expert_bytes, ld.shared_bytes if shared else None)


# ------------------------------------------------------------------ routing


def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    L = rng.normal(0, 3, (7, 50))
    assert np.allclose(moe.softmax(L), scipy.special.softmax(L, axis=1), rtol=1e-14, atol=0)


def test_topk_matches_full_sort_bruteforce():
    rng = np.random.default_rng(1)
    for _ in range(50):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        # coarse values force exact ties
        L = rng.integers(-5, 5, (3, E)).astype(np.float64)
        ids = moe.topk_ids(L, k)
        for t in range(3):
            brute = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
            assert list(ids[t]) == brute


def test_route_weights_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(6, 32))
    wr = rng.normal(0, 0.5, (20, 32))
    ids, w, L = moe.route(x, wr, 4)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(np.take_along_axis(L, ids, 1), axis=1) <= 0)
    ids2, w2, _ = moe.route(x, wr, 4, bias=np.full(20, 3.25))
    assert np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=1e-12)


def test_route_topk_by_prob_equals_topk_by_logit():
    rng = np.random.default_rng(3)
    L = rng.normal(size=(5, 30))
    p = moe.softmax(L)
    assert np.array_equal(moe.topk_ids(L, 6), moe.topk_ids(p, 6))


def test_route_equal_logits():
    x = np.ones((2, 8))
    wr = np.zeros((10, 8))
    ids, w, _ = moe.route(x, wr, 3)
    assert np.array_equal(ids, [[0, 1, 2], [0, 1, 2]])
    assert np.allclose(w, 1.0 / 3, atol=1e-15)


def test_route_weights_closed_form():
    # renormalised softmax over S equals exp(L_i) / sum_{j in S} exp(L_j)
    rng = np.random.default_rng(4)
    x = rng.normal(size=(4, 16))
    wr = rng.normal(size=(12, 16))
    ids, w, L = moe.route(x, wr, 5)
    ls = np.take_along_axis(L, ids, 1)
    ref = np.exp(ls) / np.exp(ls).sum(1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-12)


# ------------------------------------------------------------------ plan


def test_plan_invariants_and_bruteforce():
    rng = np.random.default_rng(5)
    for _ in range(30):
        E, T, k = int(rng.integers(1, 30)), int(rng.integers(1, 20)), None
        k = int(rng.integers(1, E + 1))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        pl = moe.plan(ids, E)
        assert pl.counts.sum() == T * k
        assert pl.offsets[0] == 0 and np.array_equal(np.diff(pl.offsets), pl.counts)
        assert np.array_equal(np.sort(pl.perm), np.arange(T * k))
        assert pl.n_union == np.count_nonzero(pl.counts) <= min(E, k * T)
        assert np.all(np.diff(pl.union) > 0)
        flat = ids.reshape(-1)
        for e in range(E):
            brute = [p for p in range(T * k) if flat[p] == e]
            assert list(pl.perm[pl.offsets[e]:pl.offsets[e + 1]]) == brute


# ------------------------------------------------------------------ FFN / layer


def test_sparse_layer_equals_dense_bruteforce_tiny():
    ld, layer = _tiny_layer(seed=7)
    x = ld.x_values()
    res = moe.moe_layer(layer, x)
    dense = moe.dense_moe(layer, x)
    assert np.allclose(res.out, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_sparse_layer_equals_dense_with_shared_and_bias():
    cfg = synthdata.Config("t2", 5, 256, 256, 12, 3, "f32", True, zipf_lambda=1.0)
    ld = synthdata.LayerData(cfg, 11)
    layer = moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(), ld.expert_bytes,
                      ld.shared_bytes)
    x = ld.x_values()
    bias = ld.bias()
    res = moe.moe_layer(layer, x, bias=bias)
    dense = moe.dense_moe(layer, x, bias=bias)
    assert np.allclose(res.out, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_single_expert_is_plain_swiglu_ffn_torch():
    # E = k = 1: weight 1, the layer is one SwiGLU FFN (checked with torch float64)
    cfg = synthdata.Config("one", 3, 256, 128, 1, 1, "f32", False)
    ld = synthdata.LayerData(cfg, 3)
    layer = moe.Layer(256, 128, 1, 1, ld.router(), ld.expert_bytes, None)
    x = ld.x_values()
    out = moe.moe_layer(layer, x).out
    wg = torch.from_numpy(formats.q2_matrix(ld.expert_bytes("gate", 0), 128, 256))
    wu = torch.from_numpy(formats.q2_matrix(ld.expert_bytes("up", 0), 128, 256))
    wd = torch.from_numpy(formats.q2_matrix(ld.expert_bytes("down", 0), 256, 128))
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_all_experts_equal_logits_is_mean():
    cfg = synthdata.Config("mean", 2, 256, 128, 4, 4, "f32", False)
    ld = synthdata.LayerData(cfg, 5)
    layer = moe.Layer(256, 128, 4, 4, np.zeros((4, 256), np.float32), ld.expert_bytes, None)
    x = ld.x_values()
    out = moe.moe_layer(layer, x).out
    ys = [moe.ffn(x, layer.expert_matrix("gate", e), layer.expert_matrix("up", e),
                  layer.expert_matrix("down", e)) for e in range(4)]
    assert np.allclose(out, np.mean(ys, axis=0), rtol=1e-12, atol=1e-12)


def test_shared_expert_adds_with_weight_one():
    cfg = synthdata.Config("sh", 2, 256, 128, 4, 2, "f32", True)
    ld = synthdata.LayerData(cfg, 9)
    with_sh = moe.Layer(256, 128, 4, 2, ld.router(), ld.expert_bytes, ld.shared_bytes)
    without = moe.Layer(256, 128, 4, 2, ld.router(), ld.expert_bytes, None)
    x = ld.x_values()
    wsg = torch.from_numpy(formats.q8_0_matrix(ld.shared_bytes("gate"), 128, 256))
    wsu = torch.from_numpy(formats.q8_0_matrix(ld.shared_bytes("up"), 128, 256))
    wsd = torch.from_numpy(formats.q8_0_matrix(ld.shared_bytes("down"), 256, 128))
    xt = torch.from_numpy(x)
    sh = ((torch.nn.functional.silu(xt @ wsg.T) * (xt @ wsu.T)) @ wsd.T).numpy()
    diff = moe.moe_layer(with_sh, x).out - moe.moe_layer(without, x).out
    assert np.allclose(diff, sh, rtol=1e-11, atol=1e-11 * np.abs(sh).max())


def test_forced_selection_weights():
    ld, layer = _tiny_layer(seed=2)
    x = ld.x_values()
    res = moe.moe_layer(layer, x)
    alt = res.ids[:, ::-1].copy()
    res2 = moe.moe_layer(layer, x, ids=alt)
    # same set in another order: same output
    assert np.allclose(res.out, res2.out, rtol=1e-12, atol=1e-12)


def test_residual_rescale_hand_worked():
    # r = x + out per token row, x' = bf16(r / sqrt(mean(r^2) + 1e-6)), worked by hand:
    # row 0: r = (1, 1), mean 1: 1/sqrt(1.000001) = 0.9999995 -> bf16 1.0 = 0x3F80 twice
    # row 1: r = (3, 4), mean 12.5, rms = 3.5355339: 0.848528 -> 217/256 = 0x3F59,
    #        1.131371 -> 145/128 = 0x3F91 (steps 2^-8 below 1, 2^-7 above)
    # (dropping x gives (0, 1.414) = (0x0000, 0x3FB5); x - out flips the second sign)
    x = np.array([[1.0, 0.0], [3.0, 0.0]])
    out = np.array([[0.0, 1.0], [0.0, 4.0]])
    assert moe.residual_rescale(x, out).tolist() == [[0x3F80, 0x3F80], [0x3F59, 0x3F91]]
    # tiny rows: eps matters.  r = (2^-10, 2^-10), mean r^2 = 2^-20, so
    # r/rms = 1/sqrt(1 + 1e-6 * 2^20) = 1/sqrt(2.048576) = 0.698673 -> 179/256 = 0x3F33
    # (eps = 0 would give 1.0 = 0x3F80, eps = 1e-5 gives 0.29507 = 0x3E97)
    tiny = np.full((1, 2), 2.0 ** -10)
    assert moe.residual_rescale(tiny, np.zeros((1, 2))).tolist() == [[0x3F33, 0x3F33]]


def test_residual_rescale_unit_rms():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 4096))
    out = rng.normal(size=(3, 4096)) * 5
    bits = moe.residual_rescale(x, out)
    v = formats.bf16_to_f64(bits)
    assert np.allclose(np.sqrt(np.mean(v * v, axis=1)), 1.0, rtol=1e-2)


# ------------------------------------------------------------------ repeated experts


def test_served_pairs_hand_cases():
    ids = np.array([[0, 1, 0, 3], [2, 2, 2, 2], [5, -1, 4, 1], [3, 1, 1, 0]])
    want = [[1, 1, 0, 1], [1, 0, 0, 0], [0, 0, 1, 1], [1, 1, 0, 1]]
    assert moe.served_pairs(ids, 5).astype(int).tolist() == want


def test_plan_leaves_out_repeats_and_bad_ids():
    ids = np.array([[0, 1, 0], [1, 1, 2], [7, 2, 0]])
    pl = moe.plan(ids, 3)
    # served pairs: 0 (e0), 1 (e1), 3 (e1), 5 (e2), 7 (e2), 8 (e0)
    assert pl.counts.tolist() == [2, 2, 2]
    assert pl.perm.tolist() == [0, 8, 1, 3, 5, 7]
    assert pl.union.tolist() == [0, 1, 2]


def test_repeated_expert_contributes_once():
    # a token that names expert e twice gets FFN_e once, at its first slot:
    # the later slot's output is zero, the others equal a selection without
    # the repeat
    ld, layer = _tiny_layer(seed=4)
    x = ld.x_values()[:2]
    dup = np.array([[3, 5], [7, 7]])
    alt = np.array([[3, 5], [7, 8]])
    y_dup = moe.expert_outputs(layer, x, dup)
    y_alt = moe.expert_outputs(layer, x, alt)
    assert np.all(y_dup[1, 1] == 0)
    assert np.array_equal(y_dup[0], y_alt[0]) and np.array_equal(y_dup[1, 0], y_alt[1, 0])
    # hash-routed rows: the repeated entry gets weight 0, the others share 1
    xv = ld.x_values()[:1]
    ids, w, L, _ = moe.route_variant(xv, layer.w_router, 2, hash_ids=np.array([[6, 6]]))
    assert w.tolist() == [[1.0, 0.0]]
    ids, w, L, _ = moe.route_variant(xv, layer.w_router, 2, hash_ids=np.array([[16, 6]]))  # E = 16
    assert w.tolist() == [[0.0, 1.0]]
