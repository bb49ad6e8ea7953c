"""Number formats of the hot path, written out from their definitions (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Page citations
--------------
* "Feature Request: support DeepSeek V4.1 Flash with bounded SSD expert
  caching", §Feature Description: the routed down matrices use Q2_K, the
  shared expert uses Q8_0; an Engram row is 264 bytes, 256 E4M3 values
  followed by 8 E8M0 scales.  §Possible Implementation: rows are decoded
  straight to BF16 with the same rounding as the model's reference.
* "run the DeepSeek-V4-Flash-Vision tower on CUDA", commit notes: a plain
  q8_0 block takes 34 bytes.

Readings (the pages name the formats but print no byte layout)
--------------------------------------------------------------
Q2 super-block (84 bytes, 256 weights), the GGUF Q2_K layout:
  bytes  0..15  scales[s], s = sub-block 0..15 (16 weights each);
                low nibble = scale sc_s, high nibble = min m_s
  bytes 16..79  2-bit codes; weight i sits in byte 16 + 32*(i//128) + (i%32)
                at bit offset 2*((i%128)//32)
  bytes 80..81  d    (IEEE half, little endian)
  bytes 82..83  dmin (IEEE half, little endian)
  value  w_i = d*sc_s*q_i - dmin*m_s,  s = i//16, q_i in 0..3
Q8_0 block (34 bytes, 32 weights): half d, then 32 int8 q; w = d*q.
E4M3: OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, subnormals).
E8M0: 2**(X-127) for X in 0..254; X = 255 is NaN.
BF16 rounding: round to nearest, ties to even, from the exact value;
  subnormals kept, overflow -> +-inf, sign kept (-0 -> 0x8000), NaN -> NaN.

All values below are exact: every product of the formats above has at most 17
significant bits, so float64 holds them without rounding.
"""
from __future__ import annotations

import math

import numpy as np

Q2_BLOCK_BYTES = 84
Q2_BLOCK_WEIGHTS = 256
Q8_BLOCK_BYTES = 34
Q8_BLOCK_WEIGHTS = 32
ENGRAM_ROW_BYTES = 264
ENGRAM_VALUES = 256
ENGRAM_GROUP = 32  # values per E8M0 scale

# ---------------------------------------------------------------- IEEE half


def half_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- Q2 super-block


def q2_code_location(i: int) -> tuple[int, int]:
    """(byte offset in the block, bit offset) of weight i's 2-bit code."""
    if not 0 <= i < Q2_BLOCK_WEIGHTS:
        raise ValueError(i)
    return 16 + 32 * (i // 128) + (i % 32), 2 * ((i % 128) // 32)


def q2_fields(blocks: np.ndarray):
    """Split [n, 84] uint8 super-blocks into (q[n,256], sc[n,16], m[n,16],
    d[n], dmin[n]) with d and dmin as exact float64.

    The codes follow :func:`q2_code_location`: the 64 code bytes form two
    halves of 32; within a half, bit pair s of byte b is weight 32*s + b.
    """
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, Q2_BLOCK_BYTES)
    n = blocks.shape[0]
    qs = blocks[:, 16:80].reshape(n, 2, 1, 32)                 # [block][half][.][byte]
    shifts = np.array([0, 2, 4, 6], dtype=np.uint8).reshape(1, 1, 4, 1)
    q = ((qs >> shifts) & 3).reshape(n, 256)                   # [block][128*half + 32*s + byte]
    sc = blocks[:, 0:16] & 0x0F
    m = blocks[:, 0:16] >> 4
    d = half_bits_to_f64(blocks[:, 80].astype(np.uint16) | (blocks[:, 81].astype(np.uint16) << 8))
    dmin = half_bits_to_f64(blocks[:, 82].astype(np.uint16) | (blocks[:, 83].astype(np.uint16) << 8))
    return q, sc, m, d, dmin


def q2_dequant(blocks: np.ndarray) -> np.ndarray:
    """Exact weights of [n, 84] super-blocks -> float64 [n*256] in block order.

    w_i = d*sc_s*q_i - dmin*m_s with s = i // 16 (definition above).
    """
    q, sc, m, d, dmin = q2_fields(blocks)
    n = q.shape[0]
    a = d[:, None] * sc                                          # d*sc per sub-block, exact
    b = dmin[:, None] * m                                        # dmin*m per sub-block, exact
    w = q.reshape(n, 16, 16).astype(np.float64) * a[:, :, None] - b[:, :, None]  # sub-block s: weights 16s..16s+15
    return w.reshape(-1)


def q2_matrix(raw: np.ndarray, n_rows: int, n_cols: int) -> np.ndarray:
    """Dequantise a row-major [n_rows][n_cols] Q2 matrix (float64).

    Super-blocks run along the row (the input dimension).  When n_cols < 256
    the super-blocks tile the flat row-major array, so one block spans
    256 / n_cols consecutive rows (reading: the only sensible tiling of a
    256-weight block over rows shorter than the block).
    """
    n = n_rows * n_cols
    if n % Q2_BLOCK_WEIGHTS:
        raise ValueError("matrix size must be a multiple of 256 weights")
    nb = n // Q2_BLOCK_WEIGHTS
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    if raw.size != nb * Q2_BLOCK_BYTES:
        raise ValueError(f"expected {nb * Q2_BLOCK_BYTES} bytes, got {raw.size}")
    return q2_dequant(raw.reshape(nb, Q2_BLOCK_BYTES)).reshape(n_rows, n_cols)


def q2_matrix_bytes(n_rows: int, n_cols: int) -> int:
    return n_rows * n_cols // Q2_BLOCK_WEIGHTS * Q2_BLOCK_BYTES


# ---------------------------------------------------------------- Q8_0


def q8_0_dequant(blocks: np.ndarray) -> np.ndarray:
    """Exact weights of [n, 34] Q8_0 blocks -> float64 [n*32]: w = d*q."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, Q8_BLOCK_BYTES)
    d = half_bits_to_f64(blocks[:, 0].astype(np.uint16) | (blocks[:, 1].astype(np.uint16) << 8))
    q = blocks[:, 2:34].view(np.int8).astype(np.float64)
    return (d[:, None] * q).reshape(-1)


def q8_0_matrix(raw: np.ndarray, n_rows: int, n_cols: int) -> np.ndarray:
    if n_cols % Q8_BLOCK_WEIGHTS:
        raise ValueError("Q8_0 rows must be a multiple of 32 weights")
    nb = n_rows * n_cols // Q8_BLOCK_WEIGHTS
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    if raw.size != nb * Q8_BLOCK_BYTES:
        raise ValueError(f"expected {nb * Q8_BLOCK_BYTES} bytes, got {raw.size}")
    return q8_0_dequant(raw.reshape(nb, Q8_BLOCK_BYTES)).reshape(n_rows, n_cols)


def q8_0_matrix_bytes(n_rows: int, n_cols: int) -> int:
    return n_rows * n_cols // Q8_BLOCK_WEIGHTS * Q8_BLOCK_BYTES


# ---------------------------------------------------------------- E4M3 / E8M0


def e4m3_parts(code: int):
    """OCP E4M3FN code -> (sign, integer mantissa M, exponent E) with
    value = (-1)**sign * M * 2**E, or None for the two NaN codes."""
    code &= 0xFF
    sign = code >> 7
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None
    if e == 0:  # subnormal: 2**-6 * m/8
        return sign, m, -9
    return sign, 8 + m, e - 7 - 3  # 2**(e-7) * (1 + m/8)


def e4m3_to_f64(code: int) -> float:
    p = e4m3_parts(code)
    if p is None:
        return math.nan
    s, mant, ex = p
    v = math.ldexp(mant, ex)
    return -v if s else v


def e8m0_exponent(x: int):
    """E8M0 byte -> unbiased power of two, or None for NaN (0xFF)."""
    x &= 0xFF
    return None if x == 0xFF else x - 127


# ---------------------------------------------------------------- BF16


def bf16_from_parts(sign: int, mant: int, ex: int) -> int:
    """Round (-1)**sign * mant * 2**ex (mant >= 0 integer) to BF16 bits, RNE.

    BF16: 8 exponent bits (bias 127), 7 stored mantissa bits; normal values
    carry 8 significant bits, subnormals are multiples of 2**-133.
    """
    sbit = 0x8000 if sign else 0
    if mant == 0:
        return sbit
    nbits = mant.bit_length()
    top = ex + nbits - 1  # exponent of the leading bit
    if top >= -126:
        q_ex = top - 7  # quantum of the binade: 8 significant bits
    else:
        q_ex = -133  # subnormal quantum
    # value / 2**q_ex, rounded to an integer, ties to even
    shift = q_ex - ex
    if shift <= 0:
        r = mant << (-shift)
    else:
        r = mant >> shift
        rem = mant - (r << shift)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (r & 1)):
            r += 1
    # r * 2**q_ex now exact; encode
    if q_ex == -133:
        # subnormal field; r == 128 is exactly the smallest normal (field 1, mantissa 0)
        return sbit | r
    if r == 256:  # rounding carried into the next binade
        r = 128
        q_ex += 1
    biased = q_ex + 7 + 127
    if biased >= 255:
        return sbit | 0x7F80
    return sbit | (biased << 7) | (r - 128)


def bf16_from_f64(v: float) -> int:
    """Round a float64 value to BF16 bits (RNE) -- exact: the float64 is
    split into its integer significand and exponent first."""
    if math.isnan(v):
        return 0x7FC0
    sign = 1 if math.copysign(1.0, v) < 0 else 0
    if math.isinf(v):
        return (0x8000 if sign else 0) | 0x7F80
    fr, e = math.frexp(abs(v))  # abs(v) = fr * 2**e, 0.5 <= fr < 1
    mant = int(fr * (1 << 53))
    return bf16_from_parts(sign, mant, e - 53)


def bf16_array_from_f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    out = np.fromiter((bf16_from_f64(float(v)) for v in a.reshape(-1)), dtype=np.uint16, count=a.size)
    return out.reshape(a.shape)


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns -> exact float64 values (a BF16 is the top half of a
    binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def engram_decode_value(code: int, scale: int) -> int:
    """BF16 bits of E4M3(code) * 2**(E8M0(scale) - 127), rounded once (RNE)."""
    p = e4m3_parts(code)
    k = e8m0_exponent(scale)
    if p is None or k is None:
        sign = (code >> 7) & 1 if p is None else p[0]
        return (0x8000 if sign else 0) | 0x7FC0
    s, mant, ex = p
    return bf16_from_parts(s, mant, ex + k)


_ENGRAM_TABLE = None


def engram_decode_table() -> np.ndarray:
    """[256 codes][256 scales] -> BF16 bits, every combination evaluated with
    :func:`engram_decode_value`."""
    global _ENGRAM_TABLE
    if _ENGRAM_TABLE is None:
        t = np.empty((256, 256), dtype=np.uint16)
        for c in range(256):
            for x in range(256):
                t[c, x] = engram_decode_value(c, x)
        _ENGRAM_TABLE = t
    return _ENGRAM_TABLE


def is_bf16_nan(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
