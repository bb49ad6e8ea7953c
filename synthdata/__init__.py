"""Seeded synthetic inputs shared by the oracle side and the device side.

This module holds none of the method's arithmetic: it only draws bytes and
numbers.  Every tensor is a pure function of (master seed, tensor tag), so the
oracle can regenerate any slice of a multi-gigabyte tensor on the host while
the device library fills the whole tensor in HBM from the same definition.

Counter-based byte stream (SplitMix64, Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): for a tensor key K the i-th
64-bit word is mix64(K + (i + 1) * 0x9E3779B97F4A7C15) with

    mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
              z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31

(all mod 2**64).  Byte i of a raw tensor is the low 8 bits of word i.

Formats layered on the raw stream (tensor byte offset b = global index):
* Q2 super-block n (84 B at 84n): bytes 0..79 raw; d = LUT[u16 of raw bytes
  80..81], dmin = LUT[u16 of raw bytes 82..83], stored little endian.
* Q8_0 block n (34 B at 34n): d = LUT[u16 of raw bytes 0..1]; 32 raw int8.
* Engram row r (264 B at 264r): value byte v uses the high 32 bits H of word
  264r + v: c = (H * 254) >> 32, code = c + (c >= 127)  (uniform over the
  254 non-NaN E4M3 codes); scale byte: 110 + ((H * 31) >> 32)  (uniform in
  110..140).
* LUT[u] = fp16(0.01 * Phi^-1(1/2 + (u + 1/2) / 131072)), the half-normal
  |N(0, 0.01)| quantile table (65536 entries, round to nearest even).

Floating-point tensors (router weights, activations, token ids) come from
NumPy's PCG64 seeded with SeedSequence([seed, tag...]) and are uploaded.
"""
from __future__ import annotations

import statistics
from dataclasses import dataclass
from typing import Optional

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
MASK64 = (1 << 64) - 1

VOCAB = 129280
ENGRAM_ROWS = 1 << 22
ROWS_PER_TABLE = 8

# tensor kinds (tags)
KIND_GATE, KIND_UP, KIND_DOWN = 1, 2, 3
KIND_SH_GATE, KIND_SH_UP, KIND_SH_DOWN = 4, 5, 6
KIND_ROUTER, KIND_X, KIND_BIAS = 7, 8, 9
KIND_ENGRAM, KIND_TOKENS, KIND_HASH = 10, 11, 12
KIND_STACK_X = 13

KIND_OF = {"gate": KIND_GATE, "up": KIND_UP, "down": KIND_DOWN}
SHARED_KIND_OF = {"gate": KIND_SH_GATE, "up": KIND_SH_UP, "down": KIND_SH_DOWN}


def mix64_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def tensor_key(seed: int, kind: int, layer: int = 0, index: int = 0) -> int:
    """64-bit key of one tensor (host-side only; the device receives the key)."""
    z = mix64_int(seed + 0x9E3779B97F4A7C15)
    z = mix64_int(z ^ (kind << 48) ^ (layer << 24) ^ index)
    return z


def words(key: int, start: int, count: int) -> np.ndarray:
    """Words start .. start+count-1 of the stream of ``key`` (uint64)."""
    z = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z *= GAMMA
        z += np.uint64(key)
        z ^= z >> np.uint64(30)
        z *= M1
        z ^= z >> np.uint64(27)
        z *= M2
        z ^= z >> np.uint64(31)
    return z


def raw_bytes(key: int, start: int, count: int) -> np.ndarray:
    return (words(key, start, count) & np.uint64(0xFF)).astype(np.uint8)


_LUT: Optional[np.ndarray] = None


def half_normal_lut() -> np.ndarray:
    """uint16 [65536]: fp16 bit patterns of the |N(0, 0.01)| quantiles."""
    global _LUT
    if _LUT is None:
        nd = statistics.NormalDist()
        vals = np.array([0.01 * nd.inv_cdf(0.5 + (u + 0.5) / 131072.0) for u in range(65536)],
                        dtype=np.float64)
        _LUT = vals.astype(np.float16).view(np.uint16)
    return _LUT


def q2_bytes(key: int, first_block: int, n_blocks: int) -> np.ndarray:
    """Q2 super-blocks first_block .. first_block+n_blocks-1, [n][84] uint8."""
    b = raw_bytes(key, 84 * first_block, 84 * n_blocks).reshape(n_blocks, 84)
    lut = half_normal_lut()
    for off in (80, 82):
        u = b[:, off].astype(np.uint32) | (b[:, off + 1].astype(np.uint32) << 8)
        v = lut[u]
        b[:, off] = (v & 0xFF).astype(np.uint8)
        b[:, off + 1] = (v >> 8).astype(np.uint8)
    return b


def q8_0_bytes(key: int, first_block: int, n_blocks: int) -> np.ndarray:
    b = raw_bytes(key, 34 * first_block, 34 * n_blocks).reshape(n_blocks, 34)
    lut = half_normal_lut()
    u = b[:, 0].astype(np.uint32) | (b[:, 1].astype(np.uint32) << 8)
    v = lut[u]
    b[:, 0] = (v & 0xFF).astype(np.uint8)
    b[:, 1] = (v >> 8).astype(np.uint8)
    return b


def engram_rows(key: int, row_ids) -> np.ndarray:
    """Rows ``row_ids`` of an Engram table, [n][264] uint8."""
    ids = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    out = np.empty((ids.size, 264), dtype=np.uint8)
    for r, row in enumerate(ids):
        w = words(key, 264 * int(row), 264)
        H = (w >> np.uint64(32)).astype(np.uint64)
        c = ((H * np.uint64(254)) >> np.uint64(32)).astype(np.int64)[:256]
        out[r, :256] = (c + (c >= 127)).astype(np.uint8)
        out[r, 256:] = (110 + ((H[256:] * np.uint64(31)) >> np.uint64(32))).astype(np.uint8)
    return out


# ---------------------------------------------------------------- PCG64 tensors


def rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits, round to nearest even (finite inputs: their bit
    patterns stay below 0xFF800000, so the sum fits in 32 bits)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_weights(seed: int, layer: int, n_experts: int, d_model: int) -> np.ndarray:
    """float32 [E][d] ~ N(0, 0.02)."""
    g = rng(seed, KIND_ROUTER, layer)
    return (g.standard_normal((n_experts, d_model)) * 0.02).astype(np.float32)


def activations_f32(seed: int, tag: int, T: int, d_model: int) -> np.ndarray:
    g = rng(seed, KIND_X, tag)
    return g.standard_normal((T, d_model)).astype(np.float32)


def activations_bf16(seed: int, tag: int, T: int, d_model: int) -> np.ndarray:
    """BF16 bits [T][d] of N(0, 1) draws."""
    return bf16_bits_from_f32(activations_f32(seed, tag, T, d_model))


def zipf_bias(seed: int, layer: int, n_experts: int, s: float = 1.1, lam: float = 0.3) -> np.ndarray:
    """float32 [E]: lam * ln(pmf_e), pmf_e proportional to r_e**-s over a seeded
    permutation r of 1..E (skews per-expert token counts)."""
    g = rng(seed, KIND_BIAS, layer)
    r = g.permutation(n_experts) + 1
    pmf = r.astype(np.float64) ** (-s)
    pmf /= pmf.sum()
    return (lam * np.log(pmf)).astype(np.float32)


def token_ids(seed: int, tag: int, n: int) -> np.ndarray:
    g = rng(seed, KIND_TOKENS, tag)
    return g.integers(0, VOCAB, size=n, dtype=np.int64)


# ---------------------------------------------------------------- Engram row ids


def engram_row_ids(seed: int, tokens: np.ndarray, first: int, n_tables: int = 2,
                   rows_per_table: int = ROWS_PER_TABLE) -> np.ndarray:
    """Row ids [T][n_tables][rows_per_table] for tokens[first:] of a sequence.

    Seeded 64-bit multiplicative hash of the 1..3 tokens preceding each
    position (head j hashes n_j = 1 + j % 3 tokens); positions before the
    sequence start read the pad id VOCAB; result mod 2**22.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    T = tokens.size - first
    out = np.empty((T, n_tables, rows_per_table), dtype=np.int64)
    base = tensor_key(seed, KIND_HASH)
    for t in range(T):
        p = first + t
        for tb in range(n_tables):
            for j in range(rows_per_table):
                h = mix64_int(base + (rows_per_table * tb + j + 1) * 0x9E3779B97F4A7C15)
                for i in range(1, 1 + (1 + j % 3)):
                    tok = int(tokens[p - i]) if p - i >= 0 else VOCAB
                    h = ((h ^ tok) * 0x9E3779B97F4A7C15) & MASK64
                h ^= h >> 32
                out[t, tb, j] = h % ENGRAM_ROWS
    return out


# Engram injection inputs (the layer's KV weight, branch norm weights, residual
# branches).  The real model's shape: 24 gathered rows per token, width 5120.
ENGRAM_INJECT_ROWS, ENGRAM_INJECT_WIDTH = 24, 5120


def engram_kv_weight(seed: int, n_rows: int, width: int, scale: float = 1.0) -> np.ndarray:
    """BF16 bits [5 width][n_rows 256]: N(0, 1) * scale / sqrt(n_rows 256)."""
    K = n_rows * 256
    g = rng(seed, 80, n_rows, width)
    w = g.standard_normal((5 * width, K), dtype=np.float32) * np.float32(scale / np.sqrt(K))
    return bf16_bits_from_f32(w)


def engram_branch_norms(seed: int, width: int):
    """q_norm, k_norm float32 [4][width]: 1 + 0.1 N(0, 1)."""
    g = rng(seed, 81, width)
    return (1.0 + 0.1 * g.standard_normal((2, 4, width))).astype(np.float32)


def residual_branches(seed: int, T: int, width: int) -> np.ndarray:
    """BF16 bits [T][4][width], N(0, 1)."""
    return bf16_bits_from_f32(rng(seed, 82, T, width).standard_normal((T, 4, width), dtype=np.float32))


# ---------------------------------------------------------------- configurations


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    x_dtype: str  # "f32" | "bf16"
    shared: bool
    zipf_lambda: Optional[float] = None
    engram: bool = False
    history: int = 0  # tokens of history before the batch (Engram hashing)
    n_layers: int = 1  # layers of a resident stack (each with its own seeded tensors)
    engram_layers: tuple = ()  # stack layers that gather Engram rows (one table each)
    prefill_T: int = 0  # stack prefill chunk


CONFIGS = {
    # tiny layer: T=8, d=256, 16 experts top-2, FFN width 128, fp32 activations
    "tiny": Config("tiny", 8, 256, 128, 16, 2, "f32", False),
    # single-layer decode: T=1, d=4096, 384 experts top-6, width 2048, Q8_0 shared
    "decode": Config("decode", 1, 4096, 2048, 384, 6, "bf16", True),
    # batched verify (1 token + 4 drafts) + two Engram tables
    "verify": Config("verify", 5, 4096, 2048, 384, 6, "bf16", True, engram=True, history=3),
    # prefill chunk of 4096 tokens with a Zipf(1.1) router bias
    "prefill": Config("prefill", 4096, 4096, 2048, 384, 6, "bf16", True, zipf_lambda=0.3),
    # 40-layer resident stack: decode T=1 and T=5, prefill 8192; Engram at layers 1 and 14
    "stack": Config("stack", 1, 4096, 2048, 384, 6, "bf16", True, engram=True, history=3, n_layers=40,
                    engram_layers=(1, 14), prefill_T=8192),
}


class LayerData:
    """Host-side generator of one layer's tensors (lazy, per expert)."""

    def __init__(self, cfg: Config, seed: int, layer: int = 0):
        self.cfg = cfg
        self.seed = seed
        self.layer = layer
        d, F = cfg.d_model, cfg.d_ff
        self.blocks_per_expert = d * F // 256
        self.q8_blocks = d * F // 32

    def key(self, kind: str) -> int:
        return tensor_key(self.seed, KIND_OF[kind], self.layer)

    def shared_key(self, kind: str) -> int:
        return tensor_key(self.seed, SHARED_KIND_OF[kind], self.layer)

    def expert_bytes(self, kind: str, e: int) -> np.ndarray:
        n = self.blocks_per_expert
        return q2_bytes(self.key(kind), e * n, n).reshape(-1)

    def all_expert_bytes(self, kind: str) -> np.ndarray:
        n = self.blocks_per_expert * self.cfg.n_experts
        return q2_bytes(self.key(kind), 0, n).reshape(-1)

    def shared_bytes(self, kind: str) -> np.ndarray:
        return q8_0_bytes(self.shared_key(kind), 0, self.q8_blocks).reshape(-1)

    def router(self) -> np.ndarray:
        return router_weights(self.seed, self.layer, self.cfg.n_experts, self.cfg.d_model)

    def bias(self) -> Optional[np.ndarray]:
        if self.cfg.zipf_lambda is None:
            return None
        return zipf_bias(self.seed, self.layer, self.cfg.n_experts, lam=self.cfg.zipf_lambda)

    def x(self, tag: int = 0, T: Optional[int] = None):
        """Activations: float32 array (f32 configs) or BF16 bits (bf16)."""
        T = self.cfg.T if T is None else T
        if self.cfg.x_dtype == "f32":
            return activations_f32(self.seed, tag, T, self.cfg.d_model)
        return activations_bf16(self.seed, tag, T, self.cfg.d_model)

    def x_values(self, tag: int = 0, T: Optional[int] = None) -> np.ndarray:
        x = self.x(tag, T)
        if self.cfg.x_dtype == "f32":
            return x.astype(np.float64)
        return bf16_bits_to_f32(x).astype(np.float64)
