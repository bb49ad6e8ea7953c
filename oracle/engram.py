"""Engram row gather and decode (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

"Feature Request: support DeepSeek V4.1 Flash with bounded SSD expert
caching", §Feature Description: a table row is 264 bytes, 256 native E4M3
values plus 8 E8M0 scales; §Possible Implementation: rows are decoded
directly to BF16, rounded the way the model reference rounds.

[Reading: value i uses scale byte 256 + i // 32 (contiguous groups of 32, one
scale per 32 values); the product E4M3(v) * 2**(E8M0(s) - 127) is rounded
once to BF16, ties to even, subnormals kept, overflow to infinity.]
"""
from __future__ import annotations

import numpy as np

from . import formats


def decode_rows(rows: np.ndarray) -> np.ndarray:
    """[n][264] uint8 rows -> [n][256] BF16 bits."""
    rows = np.asarray(rows, dtype=np.uint8).reshape(-1, formats.ENGRAM_ROW_BYTES)
    table = formats.engram_decode_table()
    codes = rows[:, :formats.ENGRAM_VALUES].astype(np.int64)
    group = np.arange(formats.ENGRAM_VALUES) // formats.ENGRAM_GROUP
    scales = rows[:, formats.ENGRAM_VALUES + group].astype(np.int64)
    return table[codes, scales]


def gather(table_rows, n_rows: int, row_ids) -> np.ndarray:
    """Look up ``row_ids`` (any shape) in a table of ``n_rows`` rows and decode.

    ``table_rows(ids) -> [len(ids)][264] uint8`` fetches rows (so a 2**22-row
    table need not be materialised).  Out-of-range ids raise ValueError.
    Returns BF16 bits of shape row_ids.shape + (256,).
    """
    ids = np.asarray(row_ids, dtype=np.int64)
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= n_rows):
        raise ValueError("Engram row id out of range")
    out = decode_rows(table_rows(flat))
    return out.reshape(ids.shape + (formats.ENGRAM_VALUES,))
