"""GPU parity of the libbitmoe kernels against the CPU oracle (through the C ABI).

Bars: bit-exact for dequantised weights, Engram rows, plans and the seeded
device fill; expert ids exact up to the routing tie rule; MoE outputs within
the per-element relative error 1e-2 (oracle.compare.rowwise_rel_error)."""
import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import compare, engram, formats, moe

from gpu_util import device_layer, lut_device, oracle_layer, x_device

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ Engram


def test_engram_every_code_scale_pair():
    # row s: 256 codes 0..255, all 8 scales = s  -> all 65536 combinations
    rows = np.zeros((256, 264), np.uint8)
    rows[:, :256] = np.arange(256, dtype=np.uint8)[None, :]
    rows[:, 256:] = np.arange(256, dtype=np.uint8)[:, None]
    table = torch.from_numpy(rows).cuda()
    ids = torch.arange(256, dtype=torch.int64, device="cuda")
    out = _bits(bm.engram_gather(table, ids))
    ref = formats.engram_decode_table().T  # [scale][code]
    assert compare.bf16_bits_equal(out, ref)


def test_engram_verify_tables_and_hashed_rows():
    cfg = synthdata.CONFIGS["verify"]
    n_rows = synthdata.ENGRAM_ROWS
    lut = lut_device()
    keys = [synthdata.tensor_key(1, synthdata.KIND_ENGRAM, tb) for tb in range(2)]
    tables = []
    for key in keys:
        t = torch.empty(n_rows * 264, dtype=torch.uint8, device="cuda")
        bm.fill(t, key, bm.FILL_ENGRAM, lut)
        tables.append(t.view(n_rows, 264))
    toks = synthdata.token_ids(1, 0, cfg.history + cfg.T)
    ids = synthdata.engram_row_ids(1, toks, cfg.history)  # [T][2][8]
    for tb in range(2):
        rid = torch.from_numpy(ids[:, tb, :].copy()).cuda()
        out = _bits(bm.engram_gather(tables[tb], rid))
        ref = engram.gather(lambda r, k=keys[tb]: synthdata.engram_rows(k, r), n_rows, ids[:, tb, :])
        assert out.shape == ref.shape == (cfg.T, 8, 256)
        assert compare.bf16_bits_equal(out, ref)
    # the device fill equals the host generator on sampled rows (incl. both ends)
    sample = np.array([0, 1, 12345, n_rows // 2, n_rows - 1])
    dev = tables[0][torch.from_numpy(sample).cuda()].cpu().numpy()
    assert np.array_equal(dev, synthdata.engram_rows(keys[0], sample))


def test_engram_gather_tables_verify_batch():
    # both tables of a verify batch in one launch: the oracle's rows, and the
    # two single-table calls' rows, bit for bit
    cfg = synthdata.CONFIGS["verify"]
    n_rows = synthdata.ENGRAM_ROWS
    lut = lut_device()
    keys = [synthdata.tensor_key(1, synthdata.KIND_ENGRAM, tb) for tb in range(2)]
    tables = []
    for key in keys:
        t = torch.empty(n_rows * 264, dtype=torch.uint8, device="cuda")
        bm.fill(t, key, bm.FILL_ENGRAM, lut)
        tables.append(t.view(n_rows, 264))
    toks = synthdata.token_ids(1, 3, cfg.history + cfg.T)
    ids = synthdata.engram_row_ids(1, toks, cfg.history)  # [T][2][8]
    out = _bits(bm.engram_gather_tables(tables, torch.from_numpy(ids.copy()).cuda()))
    assert out.shape == (cfg.T, 2, 8, 256)
    for tb in range(2):
        ref = engram.gather(lambda r, k=keys[tb]: synthdata.engram_rows(k, r), n_rows, ids[:, tb, :])
        assert compare.bf16_bits_equal(out[:, tb], ref)
        single = _bits(bm.engram_gather(tables[tb], torch.from_numpy(ids[:, tb, :].copy()).cuda()))
        assert np.array_equal(out[:, tb], single)


def test_engram_gather_tables_bad_ids_and_sizes():
    # three tables of different row counts; an id valid in one table and out of
    # range in another is zero-filled there and recorded with its flat index
    rng = np.random.default_rng(4)
    host = []
    for n in (5, 9, 3):
        r = rng.integers(0, 256, (n, 264), dtype=np.uint8)
        r[:, 256:] = rng.integers(110, 140, (n, 8), dtype=np.uint8)
        host.append(r)
    tables = [torch.from_numpy(r).cuda() for r in host]
    ids = np.array([[[0, 4], [8, 1], [2, 0]],
                    [[4, 3], [5, 6], [3, -1]]], dtype=np.int64)  # [2 groups][3 tables][2]
    status = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = _bits(bm.engram_gather_tables(tables, torch.from_numpy(ids).cuda(), status=status))
    for g in range(2):
        for j in range(3):
            for s in range(2):
                i = ids[g, j, s]
                if 0 <= i < host[j].shape[0]:
                    assert compare.bf16_bits_equal(out[g, j, s][None], engram.decode_rows(host[j][[i]]))
                else:
                    assert np.all(out[g, j, s] == 0)
    code, detail = bm.read_status(status)
    assert code == bm.DEV_BAD_ROW and detail == 10  # group 1, table 2, slot 0: 3 >= 3 rows
    empty = bm.engram_gather_tables(tables, torch.zeros((0, 3, 2), dtype=torch.int64, device="cuda"))
    assert empty.shape == (0, 3, 2, 256)


def test_engram_bad_ids_zero_fill_and_status():
    rows = np.random.default_rng(0).integers(0, 256, (10, 264), dtype=np.uint8)
    rows[:, 256:] = 120
    table = torch.from_numpy(rows).cuda()
    ids = torch.tensor([3, -1, 9, 10, 2], dtype=torch.int64, device="cuda")
    status = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = _bits(bm.engram_gather(table, ids, status=status))
    assert np.all(out[1] == 0) and np.all(out[3] == 0)
    ref = engram.decode_rows(rows[[3, 9, 2]])
    assert compare.bf16_bits_equal(out[[0, 2, 4]], ref)
    code, detail = bm.read_status(status)
    assert code == bm.DEV_BAD_ROW and detail == 1


def test_engram_empty():
    table = torch.zeros((4, 264), dtype=torch.uint8, device="cuda")
    out = bm.engram_gather(table, torch.zeros(0, dtype=torch.int64, device="cuda"))
    assert out.shape == (0, 256)


# ------------------------------------------------------------------ dequant / fill


@pytest.mark.parametrize("n_blocks", [1, 37, 4096])
def test_dequant_q2_bit_exact(n_blocks):
    key = synthdata.tensor_key(3, synthdata.KIND_GATE, n_blocks)
    raw = synthdata.q2_bytes(key, 0, n_blocks)
    dev = torch.from_numpy(raw.reshape(-1)).cuda()
    exact = formats.q2_dequant(raw)
    f32 = bm.dequant(dev, bm.WFMT_Q2SB, n_blocks * 256, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), exact.astype(np.float32).view(np.uint32))
    b16 = _bits(bm.dequant(dev, bm.WFMT_Q2SB, n_blocks * 256, torch.bfloat16))
    assert np.array_equal(b16, formats.bf16_array_from_f64(exact.astype(np.float32).astype(np.float64)))


def test_dequant_q8_bit_exact():
    key = synthdata.tensor_key(3, synthdata.KIND_SH_GATE, 0)
    raw = synthdata.q8_0_bytes(key, 0, 999)
    dev = torch.from_numpy(raw.reshape(-1)).cuda()
    exact = formats.q8_0_dequant(raw)
    f32 = bm.dequant(dev, bm.WFMT_Q8_0, 999 * 32, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), exact.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("kind,unit", [(bm.FILL_RAW, 1), (bm.FILL_Q2, 84), (bm.FILL_Q8, 34)])
def test_device_fill_equals_host_generator(kind, unit):
    key = synthdata.tensor_key(9, 5, kind)
    n_units = 20011
    t = torch.empty(n_units * unit, dtype=torch.uint8, device="cuda")
    bm.fill(t, key, kind, lut_device())
    dev = t.cpu().numpy()
    if kind == bm.FILL_RAW:
        host = synthdata.raw_bytes(key, 0, n_units)
    elif kind == bm.FILL_Q2:
        host = synthdata.q2_bytes(key, 0, n_units).reshape(-1)
    else:
        host = synthdata.q8_0_bytes(key, 0, n_units).reshape(-1)
    assert np.array_equal(dev, host)


# ------------------------------------------------------------------ router


def _route_check(ld, T=None, tag=0, bias=None):
    layer = device_layer(ld, host_bytes=ld.cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    ws = bm.workspace(layer, x.shape[0])
    b = None if bias is None else torch.from_numpy(bias).cuda()
    ids, w = bm.route(layer, x, ws, bias=b)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    r_ids, r_w, L = moe.route(ld.x_values(tag, T), ld.router(), ld.cfg.top_k, bias)
    exact, ties, bad = compare.compare_ids(ids, r_ids, L)
    assert not bad, f"invalid selections at tokens {bad[:10]}"
    # weights: those of the device's own (valid) selection
    ref_w = moe.weights_for_selection(L, ids)
    assert np.allclose(w, ref_w, rtol=2e-5, atol=1e-7)
    return exact, ties


def test_router_tiny():
    exact, ties = _route_check(synthdata.LayerData(synthdata.CONFIGS["tiny"], 1))
    assert exact + ties == 8


@pytest.mark.parametrize("T", [1, 5, 8, 9, 64, 200])
def test_router_decode_shapes(T):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 2)
    exact, ties = _route_check(ld, T=T, tag=T)
    assert exact + ties == T


@pytest.mark.parametrize("T,d,E,k,xd", [(9, 256, 16, 2, "bf16"), (33, 1024, 100, 6, "bf16"), (130, 512, 1000, 8, "bf16"),
                                        (70, 4096, 64, 1, "bf16"), (40, 256, 100, 4, "f32")])
def test_router_ragged_shapes(T, d, E, k, xd):
    # T > 8 with bf16 x runs the logits on MFMA over the router matrix's three
    # bf16 parts (token tiles of 16, expert tiles of 64, ragged ends on both
    # sides); float32 x keeps the float32 tile kernel
    cfg = synthdata.Config(f"router-{T}-{d}-{E}", T, d, 256, E, k, xd, False)
    exact, ties = _route_check(synthdata.LayerData(cfg, 9), tag=T)
    assert exact + ties == T


def test_router_prefill_zipf_bias():
    ld = synthdata.LayerData(synthdata.CONFIGS["prefill"], 1)
    exact, ties = _route_check(ld, bias=ld.bias())
    assert exact + ties == 4096 and exact > 4000


@pytest.mark.parametrize("T", [1, 8, 64])
def test_router_exact_ties_and_nan_row(T):
    """Experts 3g, 3g+1, 3g+2 share one router row, so their logits are equal
    bit for bit on the device as in the oracle: a selected expert's lower
    group mates must be selected before it.  Expert 5's row is NaN: never
    selected (the oracle sees it as -inf)."""
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 3)
    cfg = ld.cfg
    E, k = cfg.n_experts, cfg.top_k
    base = ld.router()
    wr = base[np.arange(E) // 3].copy()
    wr[5] = np.nan
    layer = device_layer(ld, host_bytes=False)
    layer.w_router = torch.from_numpy(wr).cuda()
    x = x_device(ld, 7, T)
    ws = bm.workspace(layer, T)
    ids, w = bm.route(layer, x, ws)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert not np.any(ids == 5)
    wr_ref = wr.copy()
    wr_ref[5] = 0.0
    L = moe.router_logits(ld.x_values(7, T), wr_ref)
    L[:, 5] = -np.inf
    r_ids = moe.topk_ids(L, k)
    exact, ties, bad = compare.compare_ids(ids, r_ids, L)
    assert not bad and exact + ties == T
    for t in range(T):
        pos = {int(e): j for j, e in enumerate(ids[t])}
        for e, j in pos.items():
            for e2 in range(3 * (e // 3), e):
                if e2 == 5:
                    continue
                assert e2 in pos and pos[e2] < j, (t, ids[t])
    assert np.allclose(w, moe.weights_for_selection(L, ids), rtol=2e-5, atol=1e-7)


# ------------------------------------------------------------------ plan


@pytest.mark.parametrize("T,k,E,skew", [(1, 6, 384, 0.0), (5, 6, 384, 0.0), (300, 6, 384, 1.5), (4096, 6, 384, 1.1),
                                        (70, 2, 16, 0.0)])
def test_plan_bit_exact(T, k, E, skew):
    rng = np.random.default_rng(T + E)
    p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    out = bm.plan(torch.from_numpy(ids).cuda(), E)
    ref = moe.plan(ids, E)
    assert np.array_equal(out["counts"].cpu().numpy(), ref.counts)
    assert np.array_equal(out["offsets"].cpu().numpy(), ref.offsets)
    assert np.array_equal(out["perm"].cpu().numpy()[:T * k], ref.perm)
    U = int(out["n_union"].item())
    assert U == ref.n_union
    assert np.array_equal(out["union"].cpu().numpy()[:U], ref.union)


def test_plan_bad_ids_recorded():
    ids = np.array([[0, 3], [5, 1], [2, 7]], dtype=np.int32)
    status = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = bm.plan(torch.from_numpy(ids).cuda(), 6, status=status)
    assert out["counts"].cpu().numpy().tolist() == [1, 1, 1, 1, 0, 1]
    code, detail = bm.read_status(status)
    assert code == bm.DEV_BAD_EXPERT and detail == 5


# ------------------------------------------------------------------ decode layer


def _layer_check(ld, T=None, tag=0, mode=bm.MODE_AUTO, out_dtype=torch.bfloat16, ids_override=None):
    cfg = ld.cfg
    layer = device_layer(ld, host_bytes=cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    Tn = x.shape[0]
    ws = bm.workspace(layer, Tn, mode)
    bias = ld.bias()
    bias_t = None if bias is None else torch.from_numpy(bias).cuda()
    ids, w = bm.route(layer, x, ws, bias=bias_t)
    if ids_override is not None:
        ids = torch.from_numpy(ids_override).cuda()
    y = bm.expert_ffn(layer, x, ids, w, ws, out_dtype=out_dtype, mode=mode)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    ol = oracle_layer(ld)
    xv = ld.x_values(tag, T)
    ref = moe.moe_layer(ol, xv, bias=bias, ids=ids_h)
    r_ids, _, L = moe.route(xv, ld.router(), cfg.top_k, bias)
    if ids_override is None:
        _, _, bad = compare.compare_ids(ids_h, r_ids, L)
        assert not bad
    yv = y.float().cpu().numpy().astype(np.float64)
    err = compare.max_rel_error(yv, ref.out)
    print(f"[parity] {cfg.name} T={Tn} mode={mode} max rel err {err:.3e} "
          f"normwise {compare.normwise_rel_error(yv, ref.out):.3e}")
    return err, y, ws


def test_decode_tiny_f32():
    ld = synthdata.LayerData(synthdata.CONFIGS["tiny"], 1)
    err, _, _ = _layer_check(ld, mode=bm.MODE_DECODE, out_dtype=torch.float32)
    assert err < 1e-4  # float32 activations and hidden values travel as exact bf16 hi + lo pairs


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_decode_full_layer(T):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 4)
    err, _, _ = _layer_check(ld, T=T, tag=100 + T, mode=bm.MODE_DECODE)
    assert err < TOL


def test_decode_deterministic():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 5)
    layer = device_layer(ld)
    x = x_device(ld, 7, 5)
    ws = bm.workspace(layer, 5)
    ids, w = bm.route(layer, x, ws)
    y1 = bm.expert_ffn(layer, x, ids, w, ws).clone()
    y2 = bm.expert_ffn(layer, x, ids, w, ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_decode_bad_expert_id_skipped_and_recorded():
    ld = synthdata.LayerData(synthdata.CONFIGS["tiny"], 3)
    layer = device_layer(ld, host_bytes=True)
    x = x_device(ld)
    ws = bm.workspace(layer, 8, bm.MODE_DECODE)
    ids, w = bm.route(layer, x, ws)
    ids_bad = ids.clone()
    ids_bad[2, 1] = 99
    y = bm.expert_ffn(layer, x, ids_bad, w, ws, out_dtype=torch.float32, mode=bm.MODE_DECODE)
    code, detail = bm.read_status(bm.ws_status(ws))
    assert code == bm.DEV_BAD_EXPERT and detail == 2 * 2 + 1
    # oracle: the same layer without that pair
    ol = oracle_layer(ld)
    xv = ld.x_values()
    ids_h = ids.cpu().numpy()
    res = moe.moe_layer(ol, xv, ids=ids_h)
    y_pairs = moe.expert_outputs(ol, xv, ids_h)
    ref = res.out.copy()
    ref[2] -= res.weights[2, 1] * y_pairs[2, 1]
    assert compare.max_rel_error(y.cpu().numpy(), ref) < 1e-4


def _forced_selection_check(ld, ids_h, tag, T):
    """Experts on a given selection (weights renormalised over it, from the
    oracle's logits) against the oracle on the same selection."""
    layer = device_layer(ld)
    x = x_device(ld, tag, T)
    xv = ld.x_values(tag, T)
    _, _, L = moe.route(xv, ld.router(), ld.cfg.top_k)
    w_h = moe.weights_for_selection(L, ids_h).astype(np.float32)
    ws = bm.workspace(layer, T, bm.MODE_DECODE)
    y = bm.expert_ffn(layer, x, torch.from_numpy(ids_h.astype(np.int32)).cuda(), torch.from_numpy(w_h).cuda(), ws,
                      mode=bm.MODE_DECODE)
    torch.cuda.synchronize()
    return y, ws, moe.moe_layer(oracle_layer(ld), xv, ids=ids_h)


@pytest.mark.parametrize("T", [2, 5, 8])
def test_decode_tokens_sharing_experts(T):
    # every token picks the same six experts (in rotated orders) and one of its
    # own: jobs of T pairs run in passes of two tokens next to one-pair jobs
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 8)
    common = np.array([3, 77, 150, 211, 300, 383])
    ids_h = np.stack([np.roll(common, t) for t in range(T)])
    ids_h[:, 5] = 10 + 37 * np.arange(T)  # one expert of its own per token
    y, ws, ref = _forced_selection_check(ld, ids_h, 300 + T, T)
    err = compare.max_rel_error(y.float().cpu().numpy().astype(np.float64), ref.out)
    print(f"[parity] shared-expert jobs T={T} max rel err {err:.3e}")
    assert err < TOL
    assert bm.read_status(bm.ws_status(ws))[0] == 0


def test_decode_streamed_bad_expert_ids():
    # out-of-range ids at T=5 (streamed kernels): those pairs contribute nothing
    # and the smallest offending pair index is recorded
    ld = synthdata.LayerData(synthdata.CONFIGS["verify"], 9)
    T, k = 5, 6
    xv = ld.x_values(310, T)
    r_ids, _, L = moe.route(xv, ld.router(), k)
    ids_h = r_ids.copy()
    ids_h[1, 4] = 384
    ids_h[3, 0] = -1
    valid = ids_h.clip(0, 383)  # the oracle runs the clipped selection; those two terms are removed below
    w_h = moe.weights_for_selection(L, valid).astype(np.float32)
    layer = device_layer(ld)
    x = x_device(ld, 310, T)
    ws = bm.workspace(layer, T, bm.MODE_DECODE)
    y = bm.expert_ffn(layer, x, torch.from_numpy(ids_h.astype(np.int32)).cuda(), torch.from_numpy(w_h).cuda(), ws,
                      out_dtype=torch.float32, mode=bm.MODE_DECODE)
    code, detail = bm.read_status(bm.ws_status(ws))
    assert code == bm.DEV_BAD_EXPERT and detail == 1 * k + 4
    ol = oracle_layer(ld)
    ref = moe.moe_layer(ol, xv, ids=valid)
    y_pairs = moe.expert_outputs(ol, xv, valid)
    want = ref.out.copy()
    want[1] -= ref.weights[1, 4] * y_pairs[1, 4]
    want[3] -= ref.weights[3, 0] * y_pairs[3, 0]
    err = compare.max_rel_error(y.cpu().numpy().astype(np.float64), want)
    print(f"[parity] streamed bad ids max rel err {err:.3e}")
    assert err < 1e-4


# ------------------------------------------------------------------ prefill (grouped GEMM)


def test_prefill_tiny_shape_refused():
    ld = synthdata.LayerData(synthdata.CONFIGS["tiny"], 1)
    layer = device_layer(ld, host_bytes=True)
    x = x_device(ld)
    ws = bm.workspace(layer, 8, bm.MODE_PREFILL)
    ids, w = bm.route(layer, x, ws)
    with pytest.raises(bm.BitmoeError) as ei:
        bm.expert_ffn(layer, x, ids, w, ws, mode=bm.MODE_PREFILL)
    assert ei.value.code == bm.EUNSUPPORTED


@pytest.mark.parametrize("T", [8, 5])
def test_prefill_equals_oracle_decode_shapes(T):
    # the same layer through the grouped-GEMM path at decode sizes
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 6)
    err, _, _ = _layer_check(ld, T=T, tag=200 + T, mode=bm.MODE_PREFILL)
    assert err < TOL


@pytest.mark.parametrize("T,lam", [(300, 1.0), (129, 0.0), (64, 0.3)])
def test_prefill_ragged_groups(T, lam):
    # 16 experts top-2: groups span several 64-token M-tiles with ragged tails
    cfg = synthdata.Config("pf_small", T, 1024, 512, 16, 2, "bf16", True, zipf_lambda=lam)
    ld = synthdata.LayerData(cfg, 7)
    err, _, ws = _layer_check(ld, mode=bm.MODE_PREFILL)
    assert err < TOL
    code, _ = bm.read_status(bm.ws_status(ws))
    assert code == 0


def test_prefill_chunk_sampled_tokens():
    """Prefill chunk (T=4096, Zipf(1.1) router bias): every output finite, and
    sampled tokens against the oracle recomputed with the device's selection."""
    cfg = synthdata.CONFIGS["prefill"]
    ld = synthdata.LayerData(cfg, 1)
    layer = device_layer(ld)
    x = x_device(ld)
    ws = bm.workspace(layer, cfg.T, bm.MODE_PREFILL)
    bias = torch.from_numpy(ld.bias()).cuda()
    ids, w = bm.route(layer, x, ws, bias=bias)
    y = bm.expert_ffn(layer, x, ids, w, ws, mode=bm.MODE_PREFILL)
    code, _ = bm.read_status(bm.ws_status(ws))
    assert code == 0
    yv = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yv))
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=cfg.n_experts)
    assert counts.max() > 64  # several M-tiles for the popular experts
    ids_h = ids.cpu().numpy()
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(cfg.T, size=10, replace=False))
    sample[0] = 0
    sample[-1] = cfg.T - 1
    ol = oracle_layer(ld)
    xv = ld.x_values()[sample]
    ref = moe.moe_layer(ol, xv, bias=ld.bias(), ids=ids_h[sample])
    assert compare.max_rel_error(yv[sample], ref.out) < TOL


# ------------------------------------------------------------------ launch timing


def test_profiled_launches_give_identical_results_and_timings():
    # with timing on, every kernel is launched through hipExtLaunchKernel with
    # its event pair: the outputs must not change, and every kernel of the
    # decode layer is counted once per call with a positive duration
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 12)
    layer = device_layer(ld)
    x = x_device(ld, 3, 1)
    ws = bm.workspace(layer, 1)
    ids0, w0 = bm.route(layer, x, ws)
    y0 = bm.expert_ffn(layer, x, ids0, w0, ws).clone()
    torch.cuda.synchronize()
    bm.profile_start()
    ids1, w1 = bm.route(layer, x, ws)
    y1 = bm.expert_ffn(layer, x, ids1, w1, ws)
    torch.cuda.synchronize()
    prof = bm.profile_stop()
    assert torch.equal(ids0, ids1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    for name in ("router_gemv_kernel", "topk_kernel", "ffn_gateup_kernel", "ffn_down_kernel", "combine_kernel"):
        ms, n = prof[name]
        assert n == 1 and 0.0 < ms < 50.0, (name, ms, n)
    # timing off again: nothing more is recorded
    bm.profile_start()
    assert bm.profile_stop() == {}
