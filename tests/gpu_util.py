"""Helpers shared by the GPU parity tests: device copies of the seeded inputs
(host generators or the library's own fill of the same byte stream) and the
matching oracle views."""
from __future__ import annotations

import numpy as np
import torch

import bit_moe_amd as bm
import synthdata
from oracle import moe


def lut_device() -> torch.Tensor:
    return torch.from_numpy(synthdata.half_normal_lut().view(np.int16).copy()).cuda()


def x_device(ld: synthdata.LayerData, tag: int = 0, T=None) -> torch.Tensor:
    x = ld.x(tag, T)
    if ld.cfg.x_dtype == "f32":
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)


def device_layer(ld: synthdata.LayerData, host_bytes: bool = False) -> bm.Layer:
    """Device tensors of a layer: from the host generator (small layers) or
    from the library's device fill of the same stream."""
    cfg = ld.cfg
    E = cfg.n_experts
    nb = ld.blocks_per_expert * E

    def q2(kind):
        if host_bytes:
            return torch.from_numpy(ld.all_expert_bytes(kind)).cuda()
        t = torch.empty(nb * 84, dtype=torch.uint8, device="cuda")
        return bm.fill(t, ld.key(kind), bm.FILL_Q2, lut_device())

    def q8(kind):
        if host_bytes:
            return torch.from_numpy(ld.shared_bytes(kind)).cuda()
        t = torch.empty(ld.q8_blocks * 34, dtype=torch.uint8, device="cuda")
        return bm.fill(t, ld.shared_key(kind), bm.FILL_Q8, lut_device())

    router = torch.from_numpy(ld.router()).cuda()
    sh = [q8(k) for k in ("gate", "up", "down")] if cfg.shared else [None, None, None]
    return bm.Layer(cfg.d_model, cfg.d_ff, E, cfg.top_k, q2("gate"), q2("up"), q2("down"), router, *sh)


def oracle_layer(ld: synthdata.LayerData) -> moe.Layer:
    cfg = ld.cfg
    return moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(), ld.expert_bytes,
                     ld.shared_bytes if cfg.shared else None)
