#!/usr/bin/env python3
"""Benchmark: one routed-MoE decode layer on one MI355X.

Workload (the single-layer decode configuration): T = 1 token, d_model 4096,
384 routed experts top-6 (softmax then renormalise), expert FFN width 2048,
every expert matrix in the 2-bit super-block format, one Q8_0 shared expert,
bf16 activations.  A step is one pass of the hot path for one token: router
(logits, top-6, weights) + gate/up GEMV with SwiGLU + down GEMV + combine, all
HIP kernels of libbitmoe behind its C ABI, issued by one moe_layer call (four
launches: router, gate/up whose routed blocks select their experts from the
logits, down, combine).

Inputs are seeded and synthetic and resident in HBM before timing.  To keep
the 256 MB Infinity Cache from serving re-reads, the steps rotate through 16
independent layer instances (router, experts and shared expert each; about
51 GB) and every step has a fresh token.

Timed regions (HIP events on the stream the library launches on):
  1. graph replay of K steps captured in one HIP graph  -> value
  2. the same K steps launched eagerly  -> eager_ms_per_step
  3. K more eager steps with every launch timed by an event pair that
     hipExtLaunchKernel stamps from the kernel's own dispatch
     -> per-kernel average durations (roofline of the dominant kernel)

Also measured (fields "verify" and "prefill"): the verify batch (T=5) with
its Engram gathers, and a 4096-token prefill chunk through the grouped-GEMM
path.  Prints ONE JSON line.  ``--gpus N`` with N > 1 exits: this build uses one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode T=1/5), TFLOP/s (prefill)"
HBM_PEAK_GBPS = 8000.0
Q2_MAT = 4096 * 2048 // 256 * 84  # 2,752,512 B
Q8_MAT = 4096 * 2048 // 32 * 34  # 8,912,896 B
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "ffn_gateup_kernel__decode_T1.txt")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(T: int, U: float, D: int = 4096, F: int = 2048, E: int = 384, k: int = 6) -> dict:
    """Bytes the method must move per launch of each decode kernel that runs at
    T tokens with U distinct experts (moe_route + moe_expert_ffn): the router,
    the top-k, the gate/up and down GEMV launches (each holding the routed
    experts' and the shared expert's rows) and the combine.  h travels as bf16
    hi + lo."""
    P = T * k
    x = T * D * 2
    h_pairs, h_tok = P * F * 2 * 2, T * F * 2 * 2
    return {
        "router_gemv_kernel": E * D * 4 + x + T * E * 4,
        "topk_kernel": T * E * 4 + P * 8,
        "ffn_gateup_kernel": U * 2 * Q2_MAT + 2 * Q8_MAT + x + h_pairs + h_tok,
        "ffn_down_kernel": U * Q2_MAT + Q8_MAT + h_pairs + h_tok + (P + T) * D * 4,
        "combine_kernel": (P + T) * D * 4 + P * 8 + T * D * 2,
    }


def algorithmic_bytes_layer(U: float, D: int = 4096, F: int = 2048, E: int = 384, k: int = 6) -> dict:
    """The same for moe_layer at T = 1: no top-k launch; the gate/up launch also
    reads the logits (its routed blocks select the experts) and writes the
    selection."""
    two = algorithmic_bytes(1, U, D, F, E, k)
    return {
        "router_gemv_kernel": two["router_gemv_kernel"],
        "ffn_gateup_kernel": two["ffn_gateup_kernel"] + E * 4 + k * 8,
        "ffn_down_kernel": two["ffn_down_kernel"],
        "combine_kernel": two["combine_kernel"],
    }


# the decode GEMV kernels' own sources: the stored counter figures describe these
DECODE_KERNEL_SOURCES = ("gemv.hip", "gemv_units.h", "decode_job.h", "router_units.h")


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_src: str, label: str):
    """HBM bytes per launch of the kernel launched as `label`, from the
    committed rocprofv3 counter summary, or None when the summary covers
    another kernel or the kernel source changed since the counters were taken."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    text = open(PROFILE_SUMMARY).read()
    want = source_hash(kernel_src)
    vals = {}
    for line in text.splitlines():
        if line.startswith("<!--") and "=" in line:
            for kv in line.strip("<!-> ").split():
                if "=" in kv:
                    a, b = kv.split("=", 1)
                    vals[a] = b
    if vals.get("source_sha") != want or "traffic_bytes" not in vals or vals.get("label") != label:
        return None
    return float(vals["traffic_bytes"])


def _host_cpu() -> dict:
    """Host threads available to this process and the CPU model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "model": model}


def _oracle_pass(moe, cfg, ld, x, bias=None):
    """One timed pass of the whole fp64 layer on tokens x.  A fresh oracle
    Layer per pass (its matrix memo starts empty), so every selected expert's
    three matrices and the shared expert are dequantised inside the timed
    region, as the layer must; the raw input bytes are generated before."""
    ids, _, _ = moe.route(x, ld.router(), cfg.top_k, bias)
    raw = {(kd, int(e)): ld.expert_bytes(kd, int(e)) for e in np.unique(ids) for kd in ("gate", "up", "down")}
    sh = {kd: ld.shared_bytes(kd) for kd in ("gate", "up", "down")}
    layer = moe.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, ld.router(), lambda kd, e: raw[(kd, e)],
                      lambda kd: sh[kd])
    t0 = time.perf_counter()
    moe.moe_layer(layer, x, bias=bias)
    return time.perf_counter() - t0, len(np.unique(ids))


def cpu_baseline(seed: int, n_tokens: int, repeats: int) -> dict:
    """The fp64 oracle on the host for bounded samples.  Headline: decode
    tokens (the single-layer T=1 workload), each token one full layer pass
    (router, its 6 experts dequantised + SwiGLU FFN, the Q8_0 shared expert
    dequantised + FFN, combine) `repeats` times with a fresh oracle layer per
    pass, so nothing carries over between passes.  Beside it: one verify
    batch (T=5, the union of its experts) and a sample of prefill-chunk tokens
    (Zipf-biased routing), timed the same way.  BLAS may use every host
    thread; NumPy's elementwise work (most of the dequantisation) runs on
    one."""
    import threadpoolctl

    import synthdata
    from oracle import moe

    host = _host_cpu()
    with threadpoolctl.threadpool_limits(limits=host["nproc"]):
        blas_threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
        cfg = synthdata.CONFIGS["decode"]
        ld = synthdata.LayerData(cfg, seed, 0)
        total = 0.0
        for t in range(n_tokens):
            x = ld.x_values(10_000 + t, 1)
            for _ in range(repeats):
                dt, _ = _oracle_pass(moe, cfg, ld, x)
                total += dt
        n = n_tokens * repeats
        vcfg = synthdata.CONFIGS["verify"]
        vld = synthdata.LayerData(vcfg, seed, 0)
        v_dt, v_u = _oracle_pass(moe, vcfg, vld, vld.x_values(20_000, 5))
        pcfg = synthdata.CONFIGS["prefill"]
        pld = synthdata.LayerData(pcfg, seed, 0)
        n_pf = 4
        p_dt, p_u = _oracle_pass(moe, pcfg, pld, pld.x_values()[np.linspace(0, pcfg.T - 1, n_pf).astype(int)],
                                 bias=pld.bias())
    return {"value": round(n / total, 4), "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "host": host,
            "sample": f"{n_tokens} decode tokens (T=1, layer instance 0), each through the whole fp64 layer "
                      f"(router, 6 experts dequantised + SwiGLU FFN, Q8_0 shared expert, combine) {repeats} "
                      f"time(s) with a fresh oracle layer per pass: {n} layer passes in {total:.1f} s; BLAS on "
                      f"{blas_threads} thread(s) of {host['nproc']}, elementwise NumPy on one",
            "verify_T5": {"tokens_per_s": round(5 / v_dt, 4), "s_per_step": round(v_dt, 2), "experts": v_u,
                          "sample": "one verify batch of 5 tokens through the whole fp64 layer"},
            "prefill_sample": {"tokens_per_s": round(n_pf / p_dt, 4), "s": round(p_dt, 2), "experts": p_u,
                               "sample": f"{n_pf} tokens spread over the 4096-token chunk (Zipf-biased "
                                         f"routing) through the whole fp64 layer; a full chunk would "
                                         f"dequantise every expert once and is not timed"}}


def make_layer(bm, torch, synthdata, cfg, seed: int, layer: int, lut, dev):
    ld = synthdata.LayerData(cfg, seed, layer)
    q2 = []
    for kind in ("gate", "up", "down"):
        t = torch.empty(cfg.n_experts * ld.blocks_per_expert * 84, dtype=torch.uint8, device=dev)
        bm.fill(t, ld.key(kind), bm.FILL_Q2, lut)
        q2.append(t)
    q8 = []
    for kind in ("gate", "up", "down"):
        t = torch.empty(ld.q8_blocks * 34, dtype=torch.uint8, device=dev)
        bm.fill(t, ld.shared_key(kind), bm.FILL_Q8, lut)
        q8.append(t)
    router = torch.from_numpy(ld.router()).to(dev)
    return bm.Layer(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, *q2, router, *q8), ld


def time_steps(bm, torch, step, K: int, W: int, graph: bool):
    """Warm up, then time K steps (graph replay if requested), K eager steps,
    and K more eager steps with per-kernel timing (each launch's event pair
    stamped by its own dispatch).  Returns (graph_ms or None, eager_ms, prof)."""
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph_ms = None
    if graph:
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(K):
                    step(W + i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1)
        del g
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(K):
        step(W + i)
    e1.record()
    torch.cuda.synchronize()
    # per-kernel durations from a second eager pass with timed launches (the
    # timed launch path costs host time, so it stays out of the step timing)
    bm.profile_start()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    prof = bm.profile_stop()
    return graph_ms, e0.elapsed_time(e1), prof


def kernel_table(prof: dict, alg: dict, flops: dict = None) -> dict:
    out = {}
    for name, (ms, n) in prof.items():
        avg_s = ms / n * 1e-3
        row = {"avg_us": round(avg_s * 1e6, 3), "launches": n}
        if name in alg:
            row["alg_bytes"] = alg[name]
            row["gbps"] = round(alg[name] / avg_s / 1e9, 1)
        if flops and name in flops:
            row["tflops"] = round(flops[name] / avg_s / 1e12, 1)
        out[name] = row
    return out


def bench_verify(bm, torch, np, synthdata, args, lut, dev) -> dict:
    """Verify batch (1 token + 4 drafts) through one layer, plus the Engram
    gather of its 2 x 8 rows per token from two 2^22-row tables."""
    cfg = synthdata.CONFIGS["verify"]
    NI = args.instances
    layers = [make_layer(bm, torch, synthdata, cfg, args.seed, i, lut, dev)[0] for i in range(NI)]
    tables = []
    for tb in range(2):
        t = torch.empty(synthdata.ENGRAM_ROWS * 264, dtype=torch.uint8, device=dev)
        bm.fill(t, synthdata.tensor_key(args.seed, synthdata.KIND_ENGRAM, tb), bm.FILL_ENGRAM, lut)
        tables.append(t.view(synthdata.ENGRAM_ROWS, 264))
    K, W = args.verify_steps, 10
    T = cfg.T
    n_seq = K + W
    toks = synthdata.token_ids(args.seed, 7, n_seq * (T + cfg.history))
    rid = np.stack([synthdata.engram_row_ids(args.seed, toks[i * (T + cfg.history):(i + 1) * (T + cfg.history)],
                                             cfg.history) for i in range(n_seq)])  # [n][T][2][8]
    rid_t = torch.from_numpy(np.ascontiguousarray(rid)).to(dev)  # [n][T][2][8]
    xs = torch.from_numpy(synthdata.activations_bf16(args.seed, 2, n_seq * T, cfg.d_model).view(np.int16)).to(dev)
    xs = xs.view(torch.bfloat16).view(n_seq, T, cfg.d_model)
    ws = bm.workspace(layers[0], T)
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((T, cfg.d_model), dtype=torch.bfloat16, device=dev)
    rows = torch.empty((T, 2, 8, 256), dtype=torch.int16, device=dev)

    def step(i):
        L = layers[i % NI]
        bm.route(L, xs[i], ws, ids=ids, weights=wts)
        bm.expert_ffn(L, xs[i], ids, wts, ws, y=y, mode=bm.MODE_DECODE)
        bm.engram_gather_tables(tables, rid_t[i], out=rows)  # both tables in one launch

    graph_ms, eager_ms, prof = time_steps(bm, torch, step, K, W, not args.no_graph)
    # union size per timed step (routing recomputed outside the timed regions)
    U = []
    for i in range(W, W + K):
        bm.route(layers[i % NI], xs[i], ws, ids=ids, weights=wts)
        U.append(len(np.unique(ids.cpu().numpy())))
    U_mean = float(np.mean(U))
    step_ms = (graph_ms if graph_ms is not None else eager_ms) / K
    alg = algorithmic_bytes(T, U_mean)
    alg["engram_gather_kernel"] = 2 * (T * 8 * (264 + 512) + T * 8 * 8)  # both tables, one launch
    step_bytes = sum(alg[n] * prof[n][1] for n in prof if n in alg) / K
    return {"workload": "verify batch T=5 (+3 history tokens) through one decode layer, plus 2 x 8 Engram rows "
                        "per token gathered from two 2^22-row tables",
            "tokens_per_s": round(T / (step_ms * 1e-3), 1), "ms_per_step": round(step_ms, 5),
            "union_mean": round(U_mean, 2), "hbm_gbps_step": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
            "eager_ms_per_step": round(eager_ms / K, 5), "kernels": kernel_table(prof, alg)}


def bench_int8_decode(bm, torch, np, synthdata, args, lut, dev) -> dict:
    """The decode layer in int8 activation numerics (moe_expert_ffn mode
    DECODE_INT8) at T=1 (as the decode line) and T=5 (a verify batch without
    the Engram gathers), HIP-graph replay over the same 16 layer instances."""
    cfg = synthdata.CONFIGS["decode"]
    NI = args.instances
    layers = [make_layer(bm, torch, synthdata, cfg, args.seed, i, lut, dev)[0] for i in range(NI)]
    out = {}
    for T, K in ((1, args.steps), (5, args.verify_steps)):
        W = 10
        n_x = K + W
        xs = torch.from_numpy(synthdata.activations_bf16(args.seed, 30 + T, n_x * T, cfg.d_model).view(np.int16))
        xs = xs.to(dev).view(torch.bfloat16).view(n_x, T, cfg.d_model)
        ws = bm.workspace(layers[0], T, bm.MODE_DECODE_INT8)
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
        y = torch.empty((T, cfg.d_model), dtype=torch.bfloat16, device=dev)

        def step(i):
            L = layers[i % NI]
            bm.route(L, xs[i], ws, ids=ids, weights=wts)
            bm.expert_ffn(L, xs[i], ids, wts, ws, y=y, mode=bm.MODE_DECODE_INT8)

        graph_ms, eager_ms, prof = time_steps(bm, torch, step, K, W, not args.no_graph)
        U = []
        for i in range(W, W + K):
            bm.route(layers[i % NI], xs[i], ws, ids=ids, weights=wts)
            U.append(len(np.unique(ids.cpu().numpy())))
        U_mean = float(np.mean(U))
        P = T * cfg.top_k
        alg = algorithmic_bytes(T, U_mean)
        D, F = cfg.d_model, cfg.d_ff
        # h travels as float32 (the quantiser's input)
        alg["ffn_i8_gateup_kernel"] = U_mean * 2 * Q2_MAT + 2 * Q8_MAT + T * D * 2 + (P + T) * F * 4
        alg["ffn_i8_down_kernel"] = U_mean * Q2_MAT + Q8_MAT + (P + T) * F * 4 + (P + T) * D * 4
        step_ms = (graph_ms if graph_ms is not None else eager_ms) / K
        step_bytes = sum(alg[n] * prof[n][1] for n in prof if n in alg) / K
        out[f"T{T}"] = {"tokens_per_s": round(T / (step_ms * 1e-3), 1), "ms_per_step": round(step_ms, 5),
                        "union_mean": round(U_mean, 2), "hbm_gbps_step": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                        "eager_ms_per_step": round(eager_ms / K, 5), "kernels": kernel_table(prof, alg)}
        log(f"[bench] int8 decode T={T}: {step_ms * 1000:.2f} us/step")
    out["workload"] = ("the decode layer (T=1) and a T=5 batch in int8 activation numerics: x and h quantised "
                       "to 8-bit blocks of 32 values, integer dot products against the 2-bit and Q8_0 codes")
    return out


def bench_prefill(bm, torch, np, synthdata, args, lut, dev, lam=None, mode=None) -> dict:
    """Prefill chunk T=4096 through one layer with the Zipf router bias (lambda
    = lam, else --zipf-lambda), in the bf16 path or (mode) the int8 numerics."""
    mode = bm.MODE_PREFILL if mode is None else mode
    import dataclasses
    lam = args.zipf_lambda if lam is None else lam
    cfg = dataclasses.replace(synthdata.CONFIGS["prefill"], zipf_lambda=lam)
    L, ld = make_layer(bm, torch, synthdata, cfg, args.seed, 0, lut, dev)
    T, k, D, F = cfg.T, cfg.top_k, cfg.d_model, cfg.d_ff
    K, W = args.prefill_steps, 2
    xs = [torch.from_numpy(ld.x(tag).view(np.int16)).to(dev).view(torch.bfloat16) for tag in range(2)]
    bias = torch.from_numpy(ld.bias()).to(dev)
    ws = bm.workspace(L, T, mode)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)

    def step(i):
        x = xs[i % 2]
        bm.route(L, x, ws, bias=bias, ids=ids, weights=wts)
        bm.expert_ffn(L, x, ids, wts, ws, y=y, mode=mode)

    graph_ms, eager_ms, prof = time_steps(bm, torch, step, K, W, False)
    step_ms = eager_ms / K
    routed = 2.0 * T * k * 3 * D * F
    shared = 2.0 * T * 3 * D * F
    # useful FLOP per launch of each expert GEMM
    gemm_flops = {"routed_gateup_gemm_kernel": 2.0 * T * k * 2 * D * F, "routed_down_gemm_kernel": 2.0 * T * k * D * F,
                  "shared_gateup_gemm_kernel": 2.0 * T * 2 * D * F, "shared_down_gemm_kernel": 2.0 * T * D * F}
    if mode == bm.MODE_PREFILL_INT8:  # the same products as int8 MACs (2 ops each)
        gemm_flops = {n.replace("routed_", "routed_i8_").replace("shared_", "shared_i8_"): v
                      for n, v in gemm_flops.items()}
    gemm_ms = sum(prof.get(n, (0.0, 1))[0] for n in gemm_flops) / K
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=cfg.n_experts)
    return {"workload": "prefill chunk T=4096 through one layer (384 experts top-6, Zipf(1.1) router bias "
                        f"lambda={lam}, Q8_0 shared expert)",
            "tokens_per_s": round(T / (step_ms * 1e-3), 1), "ms_per_step": round(step_ms, 4),
            "tflops_step": round((routed + shared) / (step_ms * 1e-3) / 1e12, 1),
            "tflops_grouped_gemm": round((routed + shared) / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
            "numerics": "int8 activations (q8_1 blocks), int8 MFMA" if mode == bm.MODE_PREFILL_INT8 else "bf16",
            "mfma_peak_tflops": 5000.0 if mode == bm.MODE_PREFILL_INT8 else 2500.0,
            "mfma_bf16_peak_tflops": 2500.0,
            "mfma_bf16_measured_tflops": args.measured.get("mfma_bf16_tflops") if hasattr(args, "measured") else None,
            "expert_tokens": {"min": int(counts.min()), "median": float(np.median(counts)), "max": int(counts.max())},
            "kernels": kernel_table(prof, {}, gemm_flops)}


def bench_router_variants(bm, torch, np, synthdata, args, lut, dev) -> dict:
    """moe_route and the moe_route_ex variants (selection-only bias, sqrt-softplus
    scores, hash-routed rows) at T=1 (HIP graph of K calls over 16 router
    matrices) and T=4096 (eager)."""
    cfg = synthdata.CONFIGS["decode"]
    E, k, D = cfg.n_experts, cfg.top_k, cfg.d_model
    ld = synthdata.LayerData(cfg, args.seed, 0)
    base, _ = make_layer(bm, torch, synthdata, cfg, args.seed, 0, lut, dev)
    NI = 16
    gen = torch.Generator(device="cpu").manual_seed(args.seed)
    routers = [(torch.randn((E, D), generator=gen) * 0.02).to(dev) for _ in range(NI)]
    layers = [bm.Layer(D, cfg.d_ff, E, k, base.w_gate, base.w_up, base.w_down, r, base.ws_gate, base.ws_up,
                       base.ws_down) for r in routers]
    sel_b = (torch.randn(E, generator=gen) * (2.0 / E)).to(dev)
    vocab = 129280
    table = torch.stack([torch.randperm(E, generator=gen)[:k] for _ in range(1024)]).repeat(vocab // 1024 + 1, 1)
    table = table[:vocab].to(torch.int32).contiguous().to(dev)
    variants = {
        "softmax": {},
        "softmax_select_bias": {"select_bias": sel_b},
        "sqrt_softplus_select_bias": {"score": bm.SCORE_SQRT_SOFTPLUS, "select_bias": sel_b},
        "hash_rows": {"hash_table": table},
    }
    out = {}
    for T, K, graph in ((1, 200, not args.no_graph), (4096, 10, False)):
        xs = torch.from_numpy(synthdata.activations_bf16(args.seed, 70, T, D).view(np.int16)).to(dev)
        xs = xs.view(torch.bfloat16).view(T, D)
        tok = torch.from_numpy(synthdata.token_ids(args.seed, 71, T).astype(np.int32)).to(dev)
        ws = bm.workspace(layers[0], T)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        for name, kw in variants.items():
            kw = dict(kw)
            if "hash_table" in kw:
                kw["token_ids"] = tok

            def step(i, kw=kw):
                bm.route_ex(layers[i % NI], xs, ws, ids=ids, weights=wts, **kw)

            g_ms, e_ms, _ = time_steps(bm, torch, step, K, 5, graph)
            ms = (g_ms if g_ms is not None else e_ms) / K
            out[f"T{T}_{name}_us"] = round(ms * 1000, 2)
        del ws
    out["timing"] = "T=1: one HIP graph of 200 calls; T=4096: 10 eager calls"
    out["router_bytes_T1"] = E * D * 4
    return out


def engram_inject_bytes(T: int, n_rows: int, W: int) -> dict:
    """Bytes per launch of the two Engram injection kernels: the projection
    reads the KV weight and the rows and writes the float32 keys and value; the
    gate kernel reads those, the two norm weights, and reads and writes the
    residual branches."""
    K = n_rows * 256
    kv = T * 5 * W * 4
    return {"engram_kv_kernel": 5 * W * K * 2 + T * K * 2 + kv,
            "engram_gate_kernel": kv + T * 4 * W * 2 * 2 + 2 * 4 * W * 4 + T * 4 * 4}


def bench_engram_inject(bm, torch, np, synthdata, args, lut, dev) -> dict:
    """engram_inject at the real model's shape (24 rows per token, width 5120)
    for T = 1 and 5 (HIP graph of K calls over 2 KV weights, 630 MB in all) and
    T = 64 (eager)."""
    n_rows, W = synthdata.ENGRAM_INJECT_ROWS, synthdata.ENGRAM_INJECT_WIDTH
    K_in = n_rows * 256
    NI = 2
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    w_kv = [(torch.randn((5 * W, K_in), generator=gen, device=dev) / K_in ** 0.5).to(torch.bfloat16)
            for _ in range(NI)]
    qn, kn = (torch.from_numpy(a).to(dev) for a in synthdata.engram_branch_norms(args.seed, W))
    out = {"shape": f"rows [T][{n_rows}][256] bf16, w_kv [{5 * W}][{K_in}] bf16, residual [T][4][{W}] bf16"}
    for T, K, graph in ((1, 200, not args.no_graph), (5, 200, not args.no_graph), (64, 20, False)):
        rows = torch.randn((T, n_rows, 256), generator=gen, device=dev).to(torch.bfloat16)
        res = torch.randn((T, 4, W), generator=gen, device=dev).to(torch.bfloat16)
        gate = torch.empty((T, 4), dtype=torch.float32, device=dev)
        n = bm.engram_inject_workspace_bytes(T, W)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)

        def step(i):
            bm.engram_inject(rows, w_kv[i % NI], qn, kn, 1e-6, res, gate_out=gate, ws=ws)

        g_ms, e_ms, prof = time_steps(bm, torch, step, K, 5, graph)
        ms = (g_ms if g_ms is not None else e_ms) / K
        alg = engram_inject_bytes(T, n_rows, W)
        out[f"T{T}"] = {"us_per_call": round(ms * 1000, 2), "timing": "hip graph" if g_ms is not None else "eager",
                        "hbm_gbps_call": round(sum(alg.values()) / (ms * 1e-3) / 1e9, 1),
                        "kernels": kernel_table(prof, alg)}
        del ws
    return out


def bench_stack(bm, torch, np, synthdata, args, lut, dev) -> dict:
    """40-layer resident stack: decode T=1 and T=5 (HIP graph) and a prefill
    chunk of T=8192 (eager), each step running every layer (Engram gather at
    layers 1 and 14, then moe_layer_residual: route, experts, and the combine
    fused with the residual step into the next layer's input)."""
    cfg = synthdata.CONFIGS["stack"]
    t0 = time.time()
    layers = [make_layer(bm, torch, synthdata, cfg, args.seed, l, lut, dev)[0] for l in range(cfg.n_layers)]
    tables = {}
    for j, l in enumerate(cfg.engram_layers):
        t = torch.empty(synthdata.ENGRAM_ROWS * 264, dtype=torch.uint8, device=dev)
        bm.fill(t, synthdata.tensor_key(args.seed, synthdata.KIND_ENGRAM, j), bm.FILL_ENGRAM, lut)
        tables[l] = (t.view(synthdata.ENGRAM_ROWS, 264), j)
    torch.cuda.synchronize()
    log(f"[bench] stack: {cfg.n_layers} layers resident ({time.time() - t0:.1f} s)")
    D, F, k = cfg.d_model, cfg.d_ff, cfg.top_k
    out = {"workload": f"{cfg.n_layers}-layer resident stack (384 experts top-6 per layer, Q8_0 shared expert, "
                       f"Engram at layers {list(cfg.engram_layers)}, residual RMS rescale between layers)"}

    def run_phase(T, K, W, mode, graph):
        n = K + W
        xs = torch.from_numpy(synthdata.activations_bf16(args.seed, 60 + T, n * T, D).view(np.int16)).to(dev)
        xs = xs.view(torch.bfloat16).view(n, T, D)
        toks = synthdata.token_ids(args.seed, 70 + T, n * (T + cfg.history))
        rid = []  # per step, per Engram layer j: row ids [T][8] of table j
        for i in range(n):
            r = synthdata.engram_row_ids(args.seed, toks[i * (T + cfg.history):(i + 1) * (T + cfg.history)],
                                         cfg.history)  # [T][2][8]
            rid.append([torch.from_numpy(np.ascontiguousarray(r[:, j, :])).to(dev) for j in range(2)])
        ws = bm.workspace(layers[0], T, mode)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        xb = [torch.empty((T, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        rows = torch.empty((T, 8, 256), dtype=torch.int16, device=dev)

        def step(i):
            x = xs[i]
            for l, L in enumerate(layers):
                if l in tables:
                    t, j = tables[l]
                    bm.engram_gather(t, rid[i][j], out=rows)
                # the layer, its combine fused with the residual step into the next input
                bm.layer(L, x, ws, ids=ids, weights=wts, y=y, mode=mode, x_next=xb[l & 1])
                x = xb[l & 1]

        graph_ms, eager_ms, prof = time_steps(bm, torch, step, K, W, graph)
        step_ms = (graph_ms if graph_ms is not None else eager_ms) / K
        del ws
        return step_ms, eager_ms / K, prof

    # decode phases
    for T, K in ((1, 50), (5, 20)):
        step_ms, eager_ms, prof = run_phase(T, K, 5, bm.MODE_DECODE, not args.no_graph)
        # union per layer (routing of step 0's input through the stack, outside the timed region)
        per_layer = 0.0
        x = torch.from_numpy(synthdata.activations_bf16(args.seed, 60 + T, T, D).view(np.int16)).to(dev)
        x = x.view(torch.bfloat16).view(T, D)
        ws = bm.workspace(layers[0], T)
        U = []
        for L in layers:
            ids, w = bm.route(L, x, ws)
            U.append(len(np.unique(ids.cpu().numpy())))
            y = bm.expert_ffn(L, x, ids, w, ws)
            x = bm.residual_rescale(x, y)
        del ws
        for u in U:
            kb = algorithmic_bytes_layer(u) if T == 1 else algorithmic_bytes(T, u)
            per_layer += sum(kb.values()) + 3 * T * D * 2  # + residual step
        eng = len(cfg.engram_layers) * (T * 8 * (264 + 512) + T * 8 * 8)
        total = per_layer + eng
        out[f"decode_T{T}"] = {"tokens_per_s": round(T / (step_ms * 1e-3), 1), "ms_per_step": round(step_ms, 4),
                               "eager_ms_per_step": round(eager_ms, 4), "union_mean": round(float(np.mean(U)), 2),
                               "algorithmic_bytes_per_step": int(total),
                               "hbm_gbps": round(total / (step_ms * 1e-3) / 1e9, 1)}
        log(f"[bench] stack decode T={T}: {step_ms * 1000:.1f} us/step")
    # prefill phase
    T = cfg.prefill_T
    step_ms, _, prof = run_phase(T, args.stack_prefill_steps, 1, bm.MODE_PREFILL, False)
    flops = cfg.n_layers * (2.0 * T * k * 3 * D * F + 2.0 * T * 3 * D * F)
    out[f"prefill_T{T}"] = {"tokens_per_s": round(T / (step_ms * 1e-3), 1), "ms_per_step": round(step_ms, 3),
                            "tflops": round(flops / (step_ms * 1e-3) / 1e12, 1)}
    log(f"[bench] stack prefill T={T}: {step_ms:.1f} ms/step")
    del layers, tables
    torch.cuda.empty_cache()
    return out


def measure_peaks(bm, torch, dev) -> dict:
    """Achievable HBM read bandwidth (bitmoe_probe_read over 2 GiB) and dense
    bf16 MFMA rate (bitmoe_probe_mfma), best of 5 event-timed runs each."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    n = 2 << 30
    buf = torch.ones(n, dtype=torch.uint8, device=dev)
    best_read = 0.0
    for blocks in (2048, 8192):
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bm.probe_read(buf, n, sink, blocks)
            e1.record()
            e1.synchronize()
            best_read = max(best_read, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    blocks, iters = 2048, 2000
    flops = blocks * 4 * iters * 4 * 32768.0
    best_mfma = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bm.probe_mfma(blocks, iters, sink)
        e1.record()
        e1.synchronize()
        best_mfma = max(best_mfma, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    torch.cuda.empty_cache()
    return {"hbm_read_gbps": round(best_read, 1), "hbm_peak_gbps": HBM_PEAK_GBPS,
            "mfma_bf16_tflops": round(best_mfma, 1), "mfma_bf16_peak_tflops": 2500.0,
            "how": "best of 5 event-timed runs: a 2 GiB streaming read (16-byte loads, 4 in flight per lane, "
                   "2048 and 8192 blocks) and 8192 waves x 2000 rounds of 4 independent 32x32x16 bf16 MFMAs "
                   "on registers"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--instances", type=int, default=16)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-tokens", type=int, default=16)
    ap.add_argument("--cpu-repeats", type=int, default=1)
    ap.add_argument("--verify-steps", type=int, default=200)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip every workload beside the decode line")
    ap.add_argument("--no-stack", action="store_true", help="skip the 40-layer stack workload")
    ap.add_argument("--only", nargs="+",
                    choices=["verify", "int8_decode", "prefill", "router_variants", "engram_inject", "stack"],
                    help="run only these of the workloads beside the decode line")
    ap.add_argument("--stack-prefill-steps", type=int, default=2)
    ap.add_argument("--zipf-lambda", type=float, default=0.3,
                    help="strength of the Zipf(1.1) router bias of the prefill line (a lambda=1 line runs beside it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run 3 plain device-to-device copies of MIB MiB (reference kernel for the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU sharding of this "
              f"path is a design, not a measured configuration.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_moe_amd as bm
    import synthdata

    if not os.path.exists(bm.LIB_PATH):
        from bit_moe_amd import build
        build.build()
    bm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {args.copy_calibration} MiB device-to-device copies")
        del src, dst
    args.measured = measure_peaks(bm, torch, dev)
    log(f"[bench] measured peaks: {args.measured['hbm_read_gbps']} GB/s read, "
        f"{args.measured['mfma_bf16_tflops']} TFLOP/s bf16 MFMA")
    cfg = synthdata.CONFIGS["decode"]
    K, W, NI = args.steps, args.warmup, args.instances
    lut = torch.from_numpy(synthdata.half_normal_lut().view(np.int16).copy()).to(dev)

    # ---- decode workload: inputs resident in HBM before timing
    t0 = time.time()
    layers = [make_layer(bm, torch, synthdata, cfg, args.seed, i, lut, dev)[0] for i in range(NI)]
    n_x = K + W
    xs = torch.from_numpy(synthdata.activations_bf16(args.seed, 1, n_x, cfg.d_model).view(np.int16)).to(dev)
    xs = xs.view(torch.bfloat16).view(n_x, 1, cfg.d_model)
    ws = bm.workspace(layers[0], 1)
    ids = torch.empty((1, cfg.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, cfg.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((1, cfg.d_model), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {NI} decode layer instances resident ({time.time() - t0:.1f} s)")

    def step(i: int) -> None:
        bm.layer(layers[i % NI], xs[i], ws, ids=ids, weights=wts, y=y, mode=bm.MODE_DECODE)

    graph_ms, eager_ms, prof = time_steps(bm, torch, step, K, W, not args.no_graph)
    if graph_ms is not None:
        log(f"[bench] decode graph replay: {graph_ms / K * 1000:.2f} us/step")
    log(f"[bench] decode eager: {eager_ms / K * 1000:.2f} us/step")
    del layers
    torch.cuda.empty_cache()

    T, U = 1, cfg.top_k
    alg = algorithmic_bytes_layer(U)
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    dom_avg_s = prof[dom][0] / prof[dom][1] * 1e-3
    achieved = alg[dom] / dom_avg_s / 1e9
    src = [os.path.join(ROOT, "bit_moe_amd", "csrc", f) for f in DECODE_KERNEL_SOURCES]
    traffic = stored_traffic(src, dom)
    step_ms = (graph_ms if graph_ms is not None else eager_ms) / K
    value = T / (step_ms * 1e-3)
    step_bytes = sum(alg[n] * prof[n][1] for n in prof if n in alg) / K  # bytes of the kernels that ran
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "single-layer MoE decode: T=1, d_model 4096, 384 experts top-6, FFN 2048, "
                               "2-bit super-block experts, Q8_0 shared expert, bf16 activations",
                   "layer_instances": NI, "timing": "hip graph replay" if graph_ms is not None else "eager"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "measured_peak": args.measured["hbm_read_gbps"],
                     "frac_of_measured": round(achieved / args.measured["hbm_read_gbps"], 4)},
        "measured_peaks": args.measured,
        "hbm_gbps_step": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "eager_ms_per_step": round(eager_ms / K, 5),
        "kernels": kernel_table(prof, alg),
    }
    extras = (("verify", bench_verify), ("int8_decode", bench_int8_decode), ("prefill", bench_prefill), ("router_variants", bench_router_variants),
              ("engram_inject", bench_engram_inject), ("stack", bench_stack))
    for name, fn in extras:
        if args.no_extra or (args.only and name not in args.only) or (name == "stack" and args.no_stack):
            continue
        log(f"[bench] {name} workload")
        out[name] = fn(bm, torch, np, synthdata, args, lut, dev)
        torch.cuda.empty_cache()
        if name == "prefill" and args.zipf_lambda != 1.0:
            log("[bench] prefill workload, lambda=1")
            out["prefill_lambda1"] = fn(bm, torch, np, synthdata, args, lut, dev, lam=1.0)
            torch.cuda.empty_cache()
        if name == "prefill":
            log("[bench] prefill workload, int8 numerics")
            out["prefill_int8"] = fn(bm, torch, np, synthdata, args, lut, dev, mode=bm.MODE_PREFILL_INT8)
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_tokens, args.cpu_repeats)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
