"""Python binding of libbitmoe (routed-MoE + Engram hot path on MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libbitmoe.so``; PyTorch supplies device memory and the current stream.  The
library must have been built (``python -m bit_moe_amd.build``); importing the
binding does not build it, and every call fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitmoe.so")

# status codes / enums (include/bitmoe.h)
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, EDEVICE = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
WFMT_NONE, WFMT_Q2SB, WFMT_Q8_0 = 0, 1, 2
MODE_AUTO, MODE_DECODE, MODE_PREFILL, MODE_DECODE_INT8, MODE_PREFILL_INT8 = 0, 1, 2, 3, 4
DEV_BAD_EXPERT, DEV_BAD_ROW, DEV_BAD_TOKEN, DEV_DUP_EXPERT = 1, 2, 4, 8
LAYOUT_CANONICAL = 0
NOALLOC_MAX_T = 8  # tokens per moe_route_noalloc call
SCORE_SOFTMAX, SCORE_SQRT_SOFTPLUS = 0, 1
FILL_RAW, FILL_Q2, FILL_Q8, FILL_ENGRAM = 0, 1, 2, 3

EXPORTS = [
    "bitmoe_workspace_size", "moe_route", "moe_route_ex", "moe_expert_ffn", "engram_gather", "engram_gather_tables", "moe_plan",
    "bitmoe_plan_workspace_size", "moe_dequant", "moe_quantize_q8_1", "bitmoe_fill", "bitmoe_read_status",
    "bitmoe_ws_status", "bitmoe_strerror", "bitmoe_last_error",
    "bitmoe_profile_start", "bitmoe_profile_stop", "bitmoe_profile_get", "bitmoe_probe_read",
    "bitmoe_residual_rescale", "engram_inject", "engram_inject_workspace_size", "moe_route_noalloc",
    "bitmoe_probe_mfma", "moe_layer", "moe_layer_residual",
]


class BitmoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} [{code}]")
        self.code = code


class _LayerC(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("shared_wfmt", ctypes.c_int32),
        ("layout_flags", ctypes.c_int32),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("w_router", ctypes.c_void_p), ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p),
        ("ws_down", ctypes.c_void_p),
    ]


class _RouteOptsC(ctypes.Structure):
    _fields_ = [
        ("score", ctypes.c_int32), ("logit_bias", ctypes.c_void_p), ("select_bias", ctypes.c_void_p),
        ("hash_table", ctypes.c_void_p), ("token_ids", ctypes.c_void_p), ("vocab", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbitmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libbitmoe.so not built at {path}; run `python -m bit_moe_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(_LayerC)
    sig = {
        "bitmoe_workspace_size": [LP, I32, I32, ctypes.POINTER(SZ)],
        "moe_route": [LP, P, I32, I32, P, P, P, P, SZ, P],
        "moe_route_noalloc": [LP, P, I32, I32, P, P, P, P],
        "moe_route_ex": [LP, P, I32, I32, ctypes.POINTER(_RouteOptsC), P, P, P, SZ, P],
        "moe_expert_ffn": [LP, P, I32, I32, P, P, P, I32, I32, P, SZ, P],
        "moe_layer": [LP, P, I32, I32, P, P, P, P, I32, I32, P, SZ, P],
        "moe_layer_residual": [LP, P, I32, P, P, P, P, I32, P, I32, P, SZ, P],
        "engram_gather": [P, I64, P, I64, P, P, P],
        "engram_gather_tables": [P, P, I32, P, I64, I32, P, P, P],
        "moe_plan": [P, I32, I32, I32, P, P, P, P, P, P, P, SZ, P],
        "bitmoe_plan_workspace_size": [I32, I32, I32, ctypes.POINTER(SZ)],
        "moe_dequant": [P, I32, I64, P, I32, P],
        "moe_quantize_q8_1": [P, I32, I64, I32, P, P, P, P],
        "bitmoe_fill": [P, I64, ctypes.c_uint64, I32, P, P],
        "bitmoe_read_status": [P, P, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "bitmoe_probe_read": [P, I64, P, I32, P],
        "bitmoe_probe_mfma": [I32, I32, P, P],
        "bitmoe_residual_rescale": [P, P, I32, I32, I32, P, P],
        "engram_inject_workspace_size": [I32, I32, ctypes.POINTER(SZ)],
        "engram_inject": [P, I32, I32, P, I32, P, P, ctypes.c_float, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.bitmoe_strerror.argtypes = [ctypes.c_int]
    lib.bitmoe_strerror.restype = ctypes.c_char_p
    lib.bitmoe_last_error.argtypes = []
    lib.bitmoe_last_error.restype = ctypes.c_char_p
    lib.bitmoe_ws_status.argtypes = [P]
    lib.bitmoe_ws_status.restype = P
    lib.bitmoe_profile_start.argtypes = []
    lib.bitmoe_profile_start.restype = ctypes.c_int
    lib.bitmoe_profile_stop.argtypes = []
    lib.bitmoe_profile_stop.restype = ctypes.c_int
    lib.bitmoe_profile_get.argtypes = [I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(I64)]
    lib.bitmoe_profile_get.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != OK:
        lib = load()
        raise BitmoeError(rc, f"{lib.bitmoe_strerror(rc).decode()}: {lib.bitmoe_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require(t: torch.Tensor, name: str, dtype=None, device_only=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if device_only and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class Layer:
    """One MoE layer whose weights are device tensors (uint8 blocks)."""

    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    w_router: torch.Tensor
    ws_gate: Optional[torch.Tensor] = None
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None
    layout_flags: int = LAYOUT_CANONICAL

    def c(self) -> _LayerC:
        shared = self.ws_gate is not None
        return _LayerC(self.d_model, self.d_ff, self.n_experts, self.top_k, WFMT_Q2SB,
                       WFMT_Q8_0 if shared else WFMT_NONE, self.layout_flags,
                       self.w_gate.data_ptr(), self.w_up.data_ptr(), self.w_down.data_ptr(),
                       self.w_router.data_ptr(),
                       self.ws_gate.data_ptr() if shared else None,
                       self.ws_up.data_ptr() if shared else None,
                       self.ws_down.data_ptr() if shared else None)


def workspace_size(layer: Layer, T: int, mode: int = MODE_AUTO) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    lc = layer.c()
    _check(lib.bitmoe_workspace_size(ctypes.byref(lc), T, mode, ctypes.byref(n)))
    return n.value


def workspace(layer: Layer, T: int, mode: int = MODE_AUTO, device="cuda") -> torch.Tensor:
    """Zero-filled workspace tensor (its first 256 bytes are the status record)."""
    return torch.zeros(workspace_size(layer, T, mode), dtype=torch.uint8, device=device)


def route(layer: Layer, x: torch.Tensor, ws: torch.Tensor, bias: Optional[torch.Tensor] = None,
          ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None, stream=None):
    lib = load()
    _require(x, "x")
    T = x.shape[0]
    if ids is None:
        ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    _require(ids, "ids", torch.int32)
    _require(weights, "weights", torch.float32)
    if bias is not None:
        _require(bias, "bias", torch.float32)
    lc = layer.c()
    _check(lib.moe_route(ctypes.byref(lc), _ptr(x), _dtype_code(x), T, _ptr(bias), _ptr(ids), _ptr(weights),
                         _ptr(ws), ws.numel(), _stream(stream)))
    return ids, weights


def route_noalloc(layer: Layer, x: torch.Tensor, bias: Optional[torch.Tensor] = None,
                  ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None, stream=None):
    """moe_route_noalloc: moe_route with the library's per-device scratch in
    place of a workspace (T <= NOALLOC_MAX_T)."""
    lib = load()
    _require(x, "x")
    T = x.shape[0]
    if ids is None:
        ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    _require(ids, "ids", torch.int32)
    _require(weights, "weights", torch.float32)
    if bias is not None:
        _require(bias, "bias", torch.float32)
    lc = layer.c()
    _check(lib.moe_route_noalloc(ctypes.byref(lc), _ptr(x), _dtype_code(x), T, _ptr(bias), _ptr(ids),
                                 _ptr(weights), _stream(stream)))
    return ids, weights


def route_ex(layer: Layer, x: torch.Tensor, ws: torch.Tensor, score: int = SCORE_SOFTMAX,
             logit_bias: Optional[torch.Tensor] = None, select_bias: Optional[torch.Tensor] = None,
             hash_table: Optional[torch.Tensor] = None, token_ids: Optional[torch.Tensor] = None,
             ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None, stream=None):
    """moe_route_ex: router variants (selection-only bias, hash-routed rows,
    sqrt-softplus scores).  hash_table [vocab][k] int32 with token_ids [T] int32."""
    lib = load()
    _require(x, "x")
    T = x.shape[0]
    if ids is None:
        ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    _require(ids, "ids", torch.int32)
    _require(weights, "weights", torch.float32)
    for t, nm in ((logit_bias, "logit_bias"), (select_bias, "select_bias")):
        if t is not None:
            _require(t, nm, torch.float32)
    vocab = 0
    if hash_table is not None:
        _require(hash_table, "hash_table", torch.int32)
        vocab = hash_table.shape[0]
    if token_ids is not None:
        _require(token_ids, "token_ids", torch.int32)
    o = _RouteOptsC(score, _ptr(logit_bias), _ptr(select_bias), _ptr(hash_table), _ptr(token_ids), vocab)
    lc = layer.c()
    _check(lib.moe_route_ex(ctypes.byref(lc), _ptr(x), _dtype_code(x), T, ctypes.byref(o), _ptr(ids),
                            _ptr(weights), _ptr(ws), ws.numel(), _stream(stream)))
    return ids, weights


def expert_ffn(layer: Layer, x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor, ws: torch.Tensor,
               y: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16, mode: int = MODE_AUTO, stream=None):
    lib = load()
    _require(x, "x")
    _require(ids, "ids", torch.int32)
    _require(weights, "weights", torch.float32)
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, layer.d_model), dtype=out_dtype, device=x.device)
    _require(y, "y")
    lc = layer.c()
    _check(lib.moe_expert_ffn(ctypes.byref(lc), _ptr(x), _dtype_code(x), T, _ptr(ids), _ptr(weights), _ptr(y),
                              _dtype_code(y), mode, _ptr(ws), ws.numel(), _stream(stream)))
    return y


def layer(layer: Layer, x: torch.Tensor, ws: torch.Tensor, bias: Optional[torch.Tensor] = None,
          ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None,
          y: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16, mode: int = MODE_AUTO, stream=None,
          x_next: Optional[torch.Tensor] = None):
    """moe_layer: moe_route followed by moe_expert_ffn in one call (one token in
    decode mode runs in four launches).  Returns (ids, weights, y).  With
    x_next (bf16 [T][d_model], x bf16): moe_layer_residual, which also writes
    the stack's residual step of x and y into x_next from the combine launch."""
    lib = load()
    _require(x, "x")
    T = x.shape[0]
    if ids is None:
        ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((T, layer.d_model), dtype=out_dtype, device=x.device)
    _require(ids, "ids", torch.int32)
    _require(weights, "weights", torch.float32)
    _require(y, "y")
    if bias is not None:
        _require(bias, "bias", torch.float32)
    lc = layer.c()
    if x_next is not None:
        _require(x, "x", torch.bfloat16)
        _require(x_next, "x_next", torch.bfloat16)
        _check(lib.moe_layer_residual(ctypes.byref(lc), _ptr(x), T, _ptr(bias), _ptr(ids), _ptr(weights), _ptr(y),
                                      _dtype_code(y), _ptr(x_next), mode, _ptr(ws), ws.numel(), _stream(stream)))
        return ids, weights, y
    _check(lib.moe_layer(ctypes.byref(lc), _ptr(x), _dtype_code(x), T, _ptr(bias), _ptr(ids), _ptr(weights),
                         _ptr(y), _dtype_code(y), mode, _ptr(ws), ws.numel(), _stream(stream)))
    return ids, weights, y


def engram_inject_workspace_bytes(T: int, width: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().engram_inject_workspace_size(T, width, ctypes.byref(n)))
    return max(n.value, 1)


def engram_inject(rows: torch.Tensor, w_kv: torch.Tensor, q_norm: torch.Tensor, k_norm: torch.Tensor, eps: float,
                  residual: torch.Tensor, mask: Optional[torch.Tensor] = None, gate_out: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """engram_inject: rows [T][n_rows][256] bf16/int16 bits, w_kv [5W][n_rows*256] bf16,
    q_norm/k_norm [4][W] float32, residual [T][4][W] bf16 updated in place."""
    lib = load()
    T, n_rows = rows.shape[0], rows.shape[1]
    W = residual.shape[2]
    for t, nm in ((rows, "rows"), (w_kv, "w_kv"), (residual, "residual")):
        _require(t, nm)
    _require(q_norm, "q_norm", torch.float32)
    _require(k_norm, "k_norm", torch.float32)
    if mask is not None:
        _require(mask, "mask", torch.uint8)
    if gate_out is not None:
        _require(gate_out, "gate_out", torch.float32)
    if ws is None:
        ws = torch.empty(engram_inject_workspace_bytes(T, W), dtype=torch.uint8, device=residual.device)
    _check(lib.engram_inject(_ptr(rows), T, n_rows, _ptr(w_kv), W, _ptr(q_norm), _ptr(k_norm), float(eps),
                             _ptr(mask), _ptr(residual), _ptr(gate_out), _ptr(ws), ws.numel(), _stream(stream)))
    return residual


def engram_gather(table: torch.Tensor, row_ids: torch.Tensor, out: Optional[torch.Tensor] = None,
                  status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """table [n_rows][264] uint8, row_ids int64 (any shape) -> bf16 bits as int16 [..., 256]."""
    lib = load()
    _require(table, "table", torch.uint8)
    _require(row_ids, "row_ids", torch.int64)
    n = row_ids.numel()
    if out is None:
        out = torch.empty(tuple(row_ids.shape) + (256,), dtype=torch.int16, device=row_ids.device)
    _require(out, "out")
    if status is not None:
        _require(status, "status", torch.int64)
    _check(lib.engram_gather(_ptr(table), table.numel() // 264, _ptr(row_ids), n, _ptr(out), _ptr(status),
                             _stream(stream)))
    return out


def engram_gather_tables(tables, row_ids: torch.Tensor, out: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tables: list of [n_rows][264] uint8 tables; row_ids int64 [n_groups][n_tables][per]
    -> bf16 bits as int16 [n_groups][n_tables][per][256], one launch for every table."""
    lib = load()
    nt = len(tables)
    for j, t in enumerate(tables):
        _require(t, f"tables[{j}]", torch.uint8)
    _require(row_ids, "row_ids", torch.int64)
    if row_ids.dim() != 3 or row_ids.shape[1] != nt:
        raise ValueError(f"row_ids must be [n_groups][{nt}][per], got {tuple(row_ids.shape)}")
    if out is None:
        out = torch.empty(tuple(row_ids.shape) + (256,), dtype=torch.int16, device=row_ids.device)
    _require(out, "out")
    if status is not None:
        _require(status, "status", torch.int64)
    ptrs = (ctypes.c_void_p * nt)(*[t.data_ptr() for t in tables])
    rows = (ctypes.c_int64 * nt)(*[t.numel() // 264 for t in tables])
    _check(lib.engram_gather_tables(ptrs, rows, nt, _ptr(row_ids), row_ids.shape[0], row_ids.shape[2], _ptr(out),
                                    _ptr(status), _stream(stream)))
    return out


def plan(ids: torch.Tensor, n_experts: int, status: Optional[torch.Tensor] = None, stream=None) -> dict:
    lib = load()
    _require(ids, "ids", torch.int32)
    T, k = ids.shape
    dev = ids.device
    n = ctypes.c_size_t(0)
    _check(lib.bitmoe_plan_workspace_size(T, k, n_experts, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    out = dict(counts=torch.empty(n_experts, dtype=torch.int32, device=dev),
               offsets=torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
               perm=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               union=torch.empty(n_experts, dtype=torch.int32, device=dev),
               n_union=torch.empty(1, dtype=torch.int32, device=dev))
    _check(lib.moe_plan(_ptr(ids), T, k, n_experts, _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["perm"]),
                        _ptr(out["union"]), _ptr(out["n_union"]), _ptr(status), _ptr(ws), ws.numel(),
                        _stream(stream)))
    return out


def dequant(blocks: torch.Tensor, wfmt: int, n_weights: int, out_dtype=torch.float32, stream=None):
    lib = load()
    _require(blocks, "blocks", torch.uint8)
    out = torch.empty(n_weights, dtype=out_dtype, device=blocks.device)
    _check(lib.moe_dequant(_ptr(blocks), wfmt, n_weights, _ptr(out), _dtype_code(out), _stream(stream)))
    return out


def quantize_q8_1(x: torch.Tensor, stream=None):
    """The int8 mode's activation quantiser over a [rows][cols] float32 or bf16
    tensor -> (q int8 [rows][cols], d float32 [rows][cols/32], s float32
    [rows][cols/16])."""
    lib = load()
    _require(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows][cols]")
    rows, cols = x.shape
    q = torch.empty(rows, cols, dtype=torch.int8, device=x.device)
    d = torch.empty(rows, max(cols // 32, 1), dtype=torch.float32, device=x.device)
    s = torch.empty(rows, max(cols // 16, 1), dtype=torch.float32, device=x.device)
    _check(lib.moe_quantize_q8_1(_ptr(x), _dtype_code(x), rows, cols, _ptr(q), _ptr(d), _ptr(s), _stream(stream)))
    return q, d, s


def fill(dst: torch.Tensor, key: int, kind: int, lut: Optional[torch.Tensor] = None, stream=None):
    """Fill a uint8 device tensor with the seeded synthetic stream of `key`."""
    lib = load()
    _require(dst, "dst", torch.uint8)
    if lut is not None:
        _require(lut, "lut", torch.int16)
    _check(lib.bitmoe_fill(_ptr(dst), dst.numel(), ctypes.c_uint64(key & ((1 << 64) - 1)), kind, _ptr(lut),
                           _stream(stream)))
    return dst


def read_status(status: torch.Tensor, stream=None):
    """Synchronise and read a status record -> (code flags, smallest offending index or -1)."""
    lib = load()
    code, detail = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = lib.bitmoe_read_status(_ptr(status), _stream(stream), ctypes.byref(code), ctypes.byref(detail))
    if rc not in (OK, EDEVICE):
        _check(rc)
    return code.value, detail.value


def ws_status(ws: torch.Tensor) -> torch.Tensor:
    """The status record at the start of a layer workspace (int64[2] view)."""
    return ws[:16].view(torch.int64)


def profile_start() -> None:
    """Start timing every kernel launch of the library with HIP events."""
    _check(load().bitmoe_profile_start())


def profile_stop() -> dict:
    """Stop timing; returns {kernel name: (total ms, launches)}."""
    lib = load()
    n = lib.bitmoe_profile_stop()
    if n < 0:
        _check(n)
    out = {}
    for i in range(n):
        name, ms, cnt = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
        _check(lib.bitmoe_profile_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)))
        out[name.value.decode()] = (ms.value, cnt.value)
    return out


def probe_read(src: torch.Tensor, n_bytes: int, sink: torch.Tensor, blocks: int, stream=None) -> None:
    """Enqueue the streaming-read probe over the first n_bytes of src."""
    _check(load().bitmoe_probe_read(_ptr(src), n_bytes, _ptr(sink), blocks, _stream(stream)))


def probe_mfma(blocks: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """Enqueue the matrix-core probe: blocks x 4 waves x iters x 4 bf16 32x32x16 MFMAs (32,768 flops each)."""
    _check(load().bitmoe_probe_mfma(blocks, iters, _ptr(sink), _stream(stream)))


def residual_rescale(x: torch.Tensor, y: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Residual step of a layer stack: out = bf16((x + y) / rms(x + y)) per row; x [T][D] bf16, y [T][D]
    float32 or bf16; out may be x."""
    lib = load()
    _require(x, "x", torch.bfloat16)
    _require(y, "y")
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    T, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", torch.bfloat16)
    _check(lib.bitmoe_residual_rescale(_ptr(x), _ptr(y), F32 if y.dtype == torch.float32 else BF16, T, D, _ptr(out),
                                       _stream(stream)))
    return out
