"""moe_route_noalloc (per-device scratch, no workspace) against moe_route."""
import pytest
import torch

import bit_moe_amd as bm
import synthdata
from gpu_util import device_layer, x_device

pytestmark = pytest.mark.gpu


def test_route_noalloc_equals_route_twice():
    ld = synthdata.LayerData(synthdata.CONFIGS["decode"], 3)
    layer = device_layer(ld)
    bias = torch.linspace(-0.5, 0.5, ld.cfg.n_experts, dtype=torch.float32, device="cuda")
    # two calls in a row, the second with fewer tokens: the scratch keeps the
    # first call's logits, which the second must not read
    for T, b in ((bm.NOALLOC_MAX_T, None), (3, bias)):
        print(f"[noalloc] T={T} bias={'yes' if b is not None else 'no'}", flush=True)
        x = x_device(ld, 60 + T, T)
        ws = bm.workspace(layer, T)
        ids_a, w_a = bm.route(layer, x, ws, bias=b)
        ids_b, w_b = bm.route_noalloc(layer, x, bias=b)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(w_a, w_b)  # same kernels and order: bit for bit


def test_route_noalloc_rejects_large_T():
    ld = synthdata.LayerData(synthdata.CONFIGS["tiny"], 3)
    layer = device_layer(ld, host_bytes=True)
    x = x_device(ld, 1, bm.NOALLOC_MAX_T + 1)
    with pytest.raises(bm.BitmoeError) as ei:
        bm.route_noalloc(layer, x)
    assert ei.value.code == bm.EUNSUPPORTED
