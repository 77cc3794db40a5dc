"""fp64 CPU oracle for ART-terminated decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``kv_cache_bandwidth_amd``) never imports, links or calls it, and the two share
no code: the C source here (``art_oracle.c``) is compiled with gcc into its own
``liboracle.so``.

The method it follows is described in the header of ``art_oracle.c`` (ART
technical summary on gist.science, sections 2.1-2.4, and the puntofijo.es
article on skipping V dequantisation).  This module is argument marshalling
only: numpy arrays in, numpy arrays out.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "art_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# dtype codes of the oracle's C interface
F32, BF16, I8, I4 = 0, 1, 2, 3

# fields of one trace record (per batch row, query head, tile)
TRACE_FIELDS = ("m", "l", "d_scale", "d_dir", "streak", "kept", "probe_norm", "evaluated")

_lib = None


def build() -> str:
    """Compile art_oracle.c with gcc (no fast-math) into liboracle.so."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", _SRC,
           "-o", _LIB + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    f = lib.art_oracle_decode
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [i32] * 10 + [vp] * 7 + [i32, ctypes.c_double, ctypes.c_double, i32,
                                         ctypes.c_double, vp, vp, vp, i32, i32, i32, vp, i32, i32]
    f.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


@dataclass
class OracleResult:
    out: np.ndarray          # float64 [B, Hq, d]
    tiles_used: np.ndarray   # int32 [B, Hq]
    trace: np.ndarray | None  # float64 [B, Hq, tiles, len(TRACE_FIELDS)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(q, k, v, ctx_lens, *, tile=64, eps_scale=1e-3, eps_dir=1e-4, patience=1,
           v_skip_eps=0.0, block_table=None, block_size=0, k_scale=None, v_scale=None,
           q_dtype=None, kv_dtype=None, trace=False, threads=None, order=0,
           tile_perm=None, per_head_tables=False) -> OracleResult:
    """Run the oracle.

    q: [B, Hq, d] float32, or uint16 bf16 bit patterns.
    k, v: contiguous [B, Hkv, max_ctx, d] when block_size == 0, else paged
          [num_blocks, Hkv, block_size, d]; float32, uint16 (bf16 bits), int8,
          or uint8 holding int4 codes two per byte (last dim d / 2).
    k_scale, v_scale: uint16 fp16 bit patterns shaped like k/v without the last
          dim (int8 caches only).
    block_table: int32 [B, max_blocks_per_seq] (paged only).
    order: 0 ascending tiles, 1 tile 0 then the most recent first, 2 the
          caller's tile_perm (int32 [B, stride]: row b lists its tiles in
          visiting order, tile 0 first).
    per_head_tables: ctx_lens is [B, Hkv], block_table [B, Hkv, mbps] and
          tile_perm [B, Hkv, stride]: every (row, KV head) has its own sequence.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, d = q.shape
    if q_dtype is None:
        q_dtype = F32 if q.dtype == np.float32 else BF16
    if kv_dtype is None:
        kv_dtype = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16,
                    np.dtype(np.int8): I8, np.dtype(np.uint8): I4}[k.dtype]
    if block_size:
        num_blocks, Hkv, bs, _ = k.shape
        assert bs == block_size
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        mbps = block_table.shape[-1]
        max_ctx = 0
    else:
        _, Hkv, max_ctx, _ = k.shape
        num_blocks, mbps = 0, 0
        block_table = None
    seqs = (B, Hkv) if per_head_tables else (B,)
    assert ctx_lens.shape == seqs, (ctx_lens.shape, seqs)
    if block_size:
        assert block_table.shape[:-1] == seqs, (block_table.shape, seqs)
    if kv_dtype in (I8, I4):
        k_scale = np.ascontiguousarray(k_scale, dtype=np.uint16)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.uint16)
    stride = 0
    if order == 2:
        tile_perm = np.ascontiguousarray(tile_perm, dtype=np.int32)
        assert tile_perm.shape[:-1] == ((B, Hkv) if per_head_tables else (B,))
        stride = tile_perm.shape[-1]
    else:
        tile_perm = None
    out = np.zeros((B, Hq, d), np.float64)
    U = np.zeros((B, Hq), np.int32)
    tr = None
    ntr = 0
    if trace:
        ntr = max(1, int(-(-int(ctx_lens.max(initial=0)) // tile)))
        tr = np.full((B, Hq, ntr, len(TRACE_FIELDS)), np.nan)
    rc = lib.art_oracle_decode(B, Hq, Hkv, d, q_dtype, kv_dtype, block_size, mbps, max_ctx,
                               num_blocks, _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale),
                               _ptr(v_scale), _ptr(block_table), _ptr(ctx_lens), tile,
                               float(eps_scale), float(eps_dir), int(patience),
                               float(v_skip_eps), _ptr(out), _ptr(U), _ptr(tr), ntr,
                               threads or default_threads(), int(order), _ptr(tile_perm), stride,
                               int(bool(per_head_tables)))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return OracleResult(out, U, tr)


def widen_f16(bits) -> np.ndarray:
    """The oracle's widening of fp16 bit patterns (uint16 array) to float64."""
    lib = _load()
    f = lib.art_oracle_widen_f16
    f.argtypes, f.restype = [ctypes.c_int], ctypes.c_double
    flat = np.asarray(bits, np.uint16).ravel()
    return np.array([f(int(x)) for x in flat], np.float64).reshape(np.shape(bits))
