"""Independent fp64 reference for the oracle's special cases.

Plain two-pass softmax attention over an explicit range of positions, written
with numpy and without any tiling: softmax(q K^T / sqrt(d)) V.  It reads the
same host arrays as the oracle and widens them with numpy's own conversions
(float16 via numpy, bf16 by bit shifting), so it shares no arithmetic with
the oracle's C code.
"""
from __future__ import annotations

import numpy as np

from art_inputs import bf16_value


def widen(arr) -> np.ndarray:
    arr = np.asarray(arr)
    if arr.dtype == np.float32:
        return arr.astype(np.float64)
    if arr.dtype == np.uint16:
        return bf16_value(arr).astype(np.float64)
    raise TypeError(arr.dtype)


def logical_rows(case, which: str, b: int, g: int, n: int) -> np.ndarray:
    """Rows 0..n-1 of K ('k') or V ('v') for batch b, KV head g, as float64."""
    arr = case.k if which == "k" else case.v
    scale = case.k_scale if which == "k" else case.v_scale
    idx = np.arange(n)
    if case.block_size:
        table = case.block_table[b, g] if case.per_head_tables else case.block_table[b]
        blk = table[idx // case.block_size]
        off = idx % case.block_size
        raw = arr[blk, g, off]
        sc = None if scale is None else scale[blk, g, off]
    else:
        raw = arr[b, g, :n]
        sc = None if scale is None else scale[b, g, :n]
    if raw.dtype == np.int8:
        s = sc.view(np.float16).astype(np.float64)
        return raw.astype(np.float64) * s[:, None]
    if raw.dtype == np.uint8:  # int4 codes, element 2i in the low nibble of byte i
        nib = np.stack([raw & 0x0F, raw >> 4], axis=-1).reshape(raw.shape[0], -1).astype(np.int64)
        codes = np.where(nib >= 8, nib - 16, nib)
        s = sc.view(np.float16).astype(np.float64)
        return codes.astype(np.float64) * s[:, None]
    return widen(raw)


def query(case, b: int, h: int) -> np.ndarray:
    return widen(case.q[b, h])


def attention_weights(case, b: int, h: int, n: int) -> np.ndarray:
    """softmax over positions 0..n-1 of q.k/sqrt(d) (float64)."""
    G = case.Hq // case.Hkv
    K = logical_rows(case, "k", b, h // G, n)
    s = K @ query(case, b, h) / np.sqrt(case.d)
    w = np.exp(s - s.max())
    return w / w.sum()


def attention(case, b: int, h: int, n: int) -> np.ndarray:
    """Full softmax attention output over positions 0..n-1 (float64 [d])."""
    if n == 0:
        return np.zeros(case.d)
    G = case.Hq // case.Hkv
    V = logical_rows(case, "v", b, h // G, n)
    return attention_weights(case, b, h, n) @ V


def attention_at(case, b: int, h: int, positions) -> np.ndarray:
    """Softmax attention over an explicit set of positions (float64 [d])."""
    positions = np.asarray(sorted(positions), dtype=np.int64)
    if positions.size == 0:
        return np.zeros(case.d)
    n = int(positions.max()) + 1
    G = case.Hq // case.Hkv
    K = logical_rows(case, "k", b, h // G, n)[positions]
    V = logical_rows(case, "v", b, h // G, n)[positions]
    s = K @ query(case, b, h) / np.sqrt(case.d)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V
