"""moe_layer (router + experts + combine in one call) and moe_layer_residual
(the same with the stack's residual step in the combine launch) through the C
ABI.

Its results are moe_route's followed by moe_expert_ffn's, bit for bit: the
one-token decode arrangement (the top-k inside the routed gate/up blocks, no
launch of its own) runs the same arithmetic per row and output.  Each case compares the ids, weights and y of one moe_layer call with
those of the two separate calls on the same inputs, and the layer output with
the oracle."""
import numpy as np
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from oracle import compare, formats, moe

from gpu_util import device_layer, oracle_layer, x_device

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()


def _both(ld, tag, T, out_dtype, bias=None, mode=bm.MODE_AUTO):
    cfg = ld.cfg
    layer = device_layer(ld, host_bytes=cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    Tn = x.shape[0]
    ws = bm.workspace(layer, Tn, mode)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    ids1, w1 = bm.route(layer, x, ws, bias=b)
    y1 = bm.expert_ffn(layer, x, ids1, w1, ws, out_dtype=out_dtype, mode=mode)
    torch.cuda.synchronize()
    ids1, w1, y1 = ids1.clone(), w1.clone(), y1.clone()
    ws.zero_()
    ids2, w2, y2 = bm.layer(layer, x, ws, bias=b, out_dtype=out_dtype, mode=mode)
    torch.cuda.synchronize()
    return (ids1, w1, y1), (ids2, w2, y2), x


def _check(ld, tag, T=None, out_dtype=torch.bfloat16, bias=None, mode=bm.MODE_AUTO, oracle=True):
    (ids1, w1, y1), (ids2, w2, y2), x = _both(ld, tag, T, out_dtype, bias, mode)
    assert np.array_equal(ids1.cpu().numpy(), ids2.cpu().numpy())
    assert np.array_equal(_bits(w1), _bits(w2))
    assert np.array_equal(_bits(y1), _bits(y2))
    if oracle:
        ids_h = ids2.cpu().numpy()
        xv = ld.x_values(tag, T)
        r_ids, _, L = moe.route(xv, ld.router(), ld.cfg.top_k, bias)
        _, _, bad = compare.compare_ids(ids_h, r_ids, L)
        assert not bad
        ref = moe.moe_layer(oracle_layer(ld), xv, bias=bias, ids=ids_h)
        err = compare.max_rel_error(y2.float().cpu().numpy().astype(np.float64), ref.out)
        print(f"[parity] moe_layer {ld.cfg.name} T={x.shape[0]} max rel err {err:.3e}")
        assert err < (1e-4 if out_dtype == torch.float32 else 1e-2)


@pytest.mark.parametrize("tag", [0, 1, 2])
def test_layer_one_token_decode_shape(tag):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 11 + tag)
    _check(ld, 300 + tag)


def test_layer_one_token_f32_bias_no_shared():
    # float32 x and y, a logit bias, no shared expert, 1000 experts top-8
    # (the 16-logits-per-lane top-k), d_model 1024, d_ff 512
    cfg = synthdata.Config("layer_f32", 1, 1024, 512, 1000, 8, "f32", False)
    ld = synthdata.LayerData(cfg, 3)
    bias = np.random.default_rng(5).normal(0, 0.5, cfg.n_experts).astype(np.float32)
    _check(ld, 7, out_dtype=torch.float32, bias=bias)


def test_layer_one_token_small_shared():
    cfg = synthdata.Config("layer_small", 1, 256, 128, 16, 2, "bf16", True)
    ld = synthdata.LayerData(cfg, 4)
    _check(ld, 9)
    _check(ld, 10, out_dtype=torch.float32)


@pytest.mark.parametrize("T", [2, 5])
def test_layer_batches_run_the_two_calls(T):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 6)
    _check(ld, 40 + T, T=T)


def test_layer_prefill_mode_runs_the_two_calls():
    cfg = synthdata.Config("layer_pf", 40, 512, 256, 16, 2, "bf16", True)
    ld = synthdata.LayerData(cfg, 2)
    _check(ld, 3, mode=bm.MODE_PREFILL, oracle=False)


def test_layer_repeated_calls_and_graph_replay():
    # a run of tokens through one resident layer, eager and replayed from a
    # HIP graph, each against the two-call results
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 8)
    layer = device_layer(ld)
    xs = [x_device(ld, 500 + i, 1) for i in range(4)]
    ws = bm.workspace(layer, 1)
    ref = []
    for x in xs:
        ids, w = bm.route(layer, x, ws)
        y = bm.expert_ffn(layer, x, ids, w, ws)
        torch.cuda.synchronize()
        ref.append((ids.clone(), w.clone(), y.clone()))
    ids = torch.empty((1, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((1, 6), dtype=torch.float32, device="cuda")
    y = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
    xin = torch.empty_like(xs[0])
    for i, x in enumerate(xs):
        xin.copy_(x)
        bm.layer(layer, xin, ws, ids=ids, weights=w, y=y)
        torch.cuda.synchronize()
        assert torch.equal(ids, ref[i][0]) and np.array_equal(_bits(w), _bits(ref[i][1]))
        assert np.array_equal(_bits(y), _bits(ref[i][2]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        bm.layer(layer, xin, ws, ids=ids, weights=w, y=y, stream=s)  # warm-up outside capture
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            bm.layer(layer, xin, ws, ids=ids, weights=w, y=y, stream=s)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, x in enumerate(xs):
            xin.copy_(x)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ids, ref[i][0]), (rep, i)
            assert np.array_equal(_bits(w), _bits(ref[i][1])), (rep, i)
            assert np.array_equal(_bits(y), _bits(ref[i][2])), (rep, i)


def test_layer_empty_and_argument_errors():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 9)
    layer = device_layer(ld)
    x = x_device(ld, 1, 1)
    ws = bm.workspace(layer, 1)
    ids, w, y = bm.layer(layer, x[:0], ws)
    assert ids.shape == (0, 6) and y.shape == (0, 4096)
    with pytest.raises(bm.BitmoeError):
        bm.layer(layer, x, ws[:1024])  # workspace too small
    with pytest.raises(bm.BitmoeError):
        bm.layer(layer, x, ws, mode=9)


# ---- moe_layer_residual: moe_layer then bitmoe_residual_rescale, bit for bit ----

def _residual_check(ld, tag, T=None, out_dtype=torch.bfloat16, mode=bm.MODE_AUTO, in_place=False, oracle=False):
    cfg = ld.cfg
    layer = device_layer(ld, host_bytes=cfg.n_experts * ld.blocks_per_expert < 200000)
    x = x_device(ld, tag, T)
    Tn = x.shape[0]
    ws = bm.workspace(layer, Tn, mode)
    ids1, w1, y1 = bm.layer(layer, x, ws, out_dtype=out_dtype, mode=mode)
    xn1 = bm.residual_rescale(x, y1)
    torch.cuda.synchronize()
    ids1, w1, y1, xn1 = ids1.clone(), w1.clone(), y1.clone(), xn1.clone()
    ws.zero_()
    xin = x.clone()
    xn2 = xin if in_place else torch.empty_like(x)
    ids2, w2, y2 = bm.layer(layer, xin, ws, out_dtype=out_dtype, mode=mode, x_next=xn2)
    torch.cuda.synchronize()
    assert np.array_equal(ids1.cpu().numpy(), ids2.cpu().numpy())
    assert np.array_equal(_bits(w1), _bits(w2))
    assert np.array_equal(_bits(y1), _bits(y2))
    assert np.array_equal(_bits(xn1), _bits(xn2))
    code, _ = bm.read_status(bm.ws_status(ws))
    assert code == 0
    if oracle:  # the residual step against the oracle's, on the layer output as stored
        xv = formats.bf16_to_f64(_bits(x).view(np.uint16))
        yv = y2.double().cpu().numpy()
        assert np.array_equal(_bits(xn2).view(np.uint16), moe.residual_rescale(xv, yv))
    print(f"[parity] moe_layer_residual {cfg.name} T={Tn} mode={mode} y={out_dtype} in_place={in_place}: bit-equal")


@pytest.mark.parametrize("tag", [0, 1])
def test_layer_residual_one_token_decode_shape(tag):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 21 + tag)
    _residual_check(ld, 600 + tag, oracle=True)


def test_layer_residual_float32_output_and_in_place():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 23)
    _residual_check(ld, 610, out_dtype=torch.float32, oracle=True)
    _residual_check(ld, 611, in_place=True)


@pytest.mark.parametrize("T", [3, 5])
def test_layer_residual_decode_batches(T):
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 24)
    _residual_check(ld, 620 + T, T=T, oracle=True)


@pytest.mark.parametrize("mode", [bm.MODE_PREFILL, bm.MODE_PREFILL_INT8])
def test_layer_residual_prefill_paths(mode):
    cfg = synthdata.Config("layer_pf", 40, 512, 256, 16, 2, "bf16", True)
    ld = synthdata.LayerData(cfg, 2)
    _residual_check(ld, 630, mode=mode)


def test_layer_residual_int8_decode():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 25)
    _residual_check(ld, 640, mode=bm.MODE_DECODE_INT8)
    _residual_check(ld, 641, T=4, mode=bm.MODE_DECODE_INT8)


def test_layer_residual_graph_replay():
    # one token through a resident layer from a replayed HIP graph, each
    # replay against the eager two-step results
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 26)
    layer = device_layer(ld)
    xs = [x_device(ld, 650 + i, 1) for i in range(3)]
    ws = bm.workspace(layer, 1)
    ref = []
    for x in xs:
        _, _, y = bm.layer(layer, x, ws)
        ref.append((y.clone(), bm.residual_rescale(x, y).clone()))
    torch.cuda.synchronize()
    ids = torch.empty((1, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((1, 6), dtype=torch.float32, device="cuda")
    y = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
    xin = torch.empty_like(xs[0])
    xn = torch.empty_like(xs[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        bm.layer(layer, xin, ws, ids=ids, weights=w, y=y, stream=s, x_next=xn)  # warm-up outside capture
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            bm.layer(layer, xin, ws, ids=ids, weights=w, y=y, stream=s, x_next=xn)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, x in enumerate(xs):
            xin.copy_(x)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(_bits(y), _bits(ref[i][0])), (rep, i)
            assert np.array_equal(_bits(xn), _bits(ref[i][1])), (rep, i)


def test_layer_residual_argument_errors():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 27)
    layer = device_layer(ld)
    x = x_device(ld, 1, 1)
    ws = bm.workspace(layer, 1)
    y = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bm.BitmoeError):
        bm.layer(layer, x, ws, y=y, x_next=y)  # x_next aliases y
    with pytest.raises(TypeError):
        bm.layer(layer, x.float(), ws, x_next=torch.empty_like(x))  # x must be bf16
