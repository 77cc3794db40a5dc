"""ctypes binding of the C ABI in include/art.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libart.so.  PyTorch provides device memory and the stream.  The
library must be built (``python -m kv_cache_bandwidth_amd.build`` or
``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libart.so")

ART_F32, ART_BF16, ART_I8, ART_I4 = 0, 1, 2, 3
ORDER_ASCENDING, ORDER_RECENT, ORDER_LIST = 0, 1, 2

STATUS = {0: "ART_OK", -1: "ART_E_NULL", -2: "ART_E_SHAPE", -3: "ART_E_DTYPE", -4: "ART_E_TILE",
          -5: "ART_E_PARAM", -6: "ART_E_WORKSPACE", -7: "ART_E_HIP"}

EXPORTS = ("art_decode_attention", "art_decode_attention_noalloc", "art_workspace_bytes", "art_validate",
           "art_status_string", "art_last_error", "art_abi_version")


class ArtError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class ArtDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("patience", ctypes.c_int32),
        ("v_skip_eps", ctypes.c_float),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stats", ctypes.c_void_p),
        ("max_workers", ctypes.c_int32),
        ("team_helpers", ctypes.c_int32),
        ("engine", ctypes.c_int32),
        ("tile_order", ctypes.c_int32),
        ("tile_perm_stride", ctypes.c_int32),
        ("tile_perm", ctypes.c_void_p),
        ("per_head_tables", ctypes.c_int32),
        ("workers_per_cu", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


_lib = None


ABI_VERSION = 9  # art_desc layout and entry points this binding marshals (ART_ABI_VERSION in art.h)


def load():
    """Load libart.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m kv_cache_bandwidth_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(ArtDesc)
    vp = ctypes.c_void_p
    lib.art_decode_attention.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_float,
                                         ctypes.c_float, vp, vp, vp]
    lib.art_decode_attention.restype = ctypes.c_int32
    lib.art_decode_attention_noalloc.argtypes = lib.art_decode_attention.argtypes
    lib.art_decode_attention_noalloc.restype = ctypes.c_int32
    lib.art_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.art_workspace_bytes.restype = ctypes.c_size_t
    lib.art_validate.argtypes = [P, ctypes.c_int32, ctypes.c_float, ctypes.c_float]
    lib.art_validate.restype = ctypes.c_int32
    lib.art_status_string.argtypes = [ctypes.c_int32]
    lib.art_status_string.restype = ctypes.c_char_p
    lib.art_last_error.argtypes = []
    lib.art_last_error.restype = ctypes.c_char_p
    lib.art_abi_version.argtypes = []
    lib.art_abi_version.restype = ctypes.c_int32
    if lib.art_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.art_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise ArtError(rc, load().art_last_error().decode())


def make_desc(*, batch, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype, block_size=0,
              max_blocks_per_seq=0, num_blocks=0, max_ctx=0, patience=1, v_skip_eps=0.0,
              k_scale=0, v_scale=0, workspace=0, workspace_bytes=0, stats=0, max_workers=0,
              team_helpers=0, engine=0, tile_order=0, tile_perm_stride=0, tile_perm=0,
              per_head_tables=0, workers_per_cu=0, window=0) -> ArtDesc:
    return ArtDesc(batch, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype, block_size,
                   max_blocks_per_seq, num_blocks, max_ctx, patience, v_skip_eps, k_scale or None,
                   v_scale or None, workspace or None, workspace_bytes, stats or None, max_workers,
                   team_helpers, engine, tile_order, tile_perm_stride, tile_perm or None,
                   int(per_head_tables), workers_per_cu, window)


def workspace_bytes(desc: ArtDesc, tile: int) -> int:
    return int(load().art_workspace_bytes(ctypes.byref(desc), tile))


def validate(desc: ArtDesc, tile: int, eps_scale: float, eps_dir: float) -> int:
    return int(load().art_validate(ctypes.byref(desc), tile, eps_scale, eps_dir))


def _dtype_code(t):
    import torch
    # uint8 caches hold packed int4 codes (two per byte)
    return {torch.float32: ART_F32, torch.bfloat16: ART_BF16, torch.int8: ART_I8, torch.uint8: ART_I4}[t.dtype]


def decode_attention(q, k_cache, v_cache, ctx_lens, *, block_table=None, tile=64, eps_scale=1e-3,
                     eps_dir=1e-4, patience=1, v_skip_eps=0.0, k_scale=None, v_scale=None,
                     out=None, tiles_used=None, workspace=None, stats=None, max_workers=0, team_helpers=0,
                     engine=0, tile_order=0, tile_perm=None, per_head_tables=False,
                     workers_per_cu=0, window=0, stream=None, noalloc=False):
    """ART decode attention on device tensors; returns (out fp32, tiles_used int32).

    q [B, Hq, d] fp32/bf16; k_cache/v_cache paged [num_blocks, Hkv, bs, d] when
    block_table is given, else contiguous [B, Hkv, max_ctx, d]; fp32/bf16/int8
    (int8 needs k_scale/v_scale fp16 shaped like the cache without d); a uint8
    cache holds int4 codes, two per byte (last dim d / 2), with the same scales.
    ctx_lens int32 [B]; block_table int32 [B, max_blocks_per_seq].
    tile_order: ORDER_ASCENDING, ORDER_RECENT or ORDER_LIST (then tile_perm is
    an int32 device tensor [B, stride], row b listing its tiles in visiting order).
    per_head_tables: ctx_lens [B, Hkv], block_table [B, Hkv, mbps] and tile_perm
    [B, Hkv, stride]: every (row, KV head) has its own sequence.
    noalloc: call art_decode_attention_noalloc (the library's static workspace;
    out and tiles_used must then be given, and no workspace): nothing is
    allocated.
    """
    import torch
    lib = load()
    # Every tensor's shape, dtype and placement is checked here, before the
    # library sees a pointer: a mismatch would make the kernels read or write
    # outside the caller's buffers.
    if q.dim() != 3:
        raise ValueError(f"q must be [B, Hq, d], got shape {tuple(q.shape)}")
    B, Hq, d = q.shape
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q must be float32 or bfloat16, got {q.dtype}")
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache must be 4-dimensional, got shape {tuple(k_cache.shape)}")
    if k_cache.dtype not in (torch.float32, torch.bfloat16, torch.int8, torch.uint8):
        raise ValueError(f"k_cache dtype {k_cache.dtype} not supported")
    row = d // 2 if k_cache.dtype == torch.uint8 else d
    if k_cache.shape[-1] != row:
        raise ValueError(f"k_cache rows hold {k_cache.shape[-1]} elements, expected {row} for head_dim {d}")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must have the shape and dtype of k_cache")
    if block_table is not None:
        nb, Hkv, bs, _ = k_cache.shape
        mbps = block_table.shape[-1]
        max_ctx = 0
    else:
        _, Hkv, max_ctx, _ = k_cache.shape
        nb = bs = mbps = 0
        if k_cache.shape[0] != B:
            raise ValueError(f"a contiguous cache leads with the batch {B}, got {k_cache.shape[0]}")
    seqs = (B, Hkv) if per_head_tables else (B,)
    if tuple(ctx_lens.shape) != seqs or (block_table is not None and tuple(block_table.shape[:-1]) != seqs) \
            or (tile_perm is not None and tuple(tile_perm.shape[:-1]) != seqs):
        raise ValueError(f"ctx_lens, block_table and tile_perm must lead with {seqs}")
    scaled = k_cache.dtype in (torch.int8, torch.uint8)
    if scaled:
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t is None or tuple(t.shape) != tuple(k_cache.shape[:-1]):
                raise ValueError(f"{name} must be given, shaped like the cache without its last dim "
                                 f"{tuple(k_cache.shape[:-1])}")
    for name, t, want in (("ctx_lens", ctx_lens, torch.int32), ("block_table", block_table, torch.int32),
                          ("tile_perm", tile_perm, torch.int32), ("k_scale", k_scale, torch.float16),
                          ("v_scale", v_scale, torch.float16), ("stats", stats, torch.int64)):
        if t is not None and t.dtype != want:
            raise ValueError(f"{name} must be {want}, got {t.dtype}")
    if stats is not None and stats.numel() < 4:
        raise ValueError(f"stats must hold at least 4 int64 counters, got {stats.numel()}")
    if out is not None and (tuple(out.shape) != (B, Hq, d) or out.dtype != torch.float32):
        raise ValueError(f"out must be float32 {(B, Hq, d)}, got {out.dtype} {tuple(out.shape)}")
    if tiles_used is not None and (tuple(tiles_used.shape) != (B, Hq) or tiles_used.dtype != torch.int32):
        raise ValueError(f"tiles_used must be int32 {(B, Hq)}, got {tiles_used.dtype} {tuple(tiles_used.shape)}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("ctx_lens", ctx_lens),
                    ("block_table", block_table), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("tile_perm", tile_perm), ("out", out), ("tiles_used", tiles_used), ("stats", stats),
                    ("workspace", workspace)):
        if t is not None and not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    desc = make_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                     q_dtype=_dtype_code(q), kv_dtype=_dtype_code(k_cache), block_size=bs,
                     max_blocks_per_seq=mbps, num_blocks=nb, max_ctx=max_ctx, patience=patience,
                     v_skip_eps=v_skip_eps,
                     k_scale=k_scale.data_ptr() if k_scale is not None else 0,
                     v_scale=v_scale.data_ptr() if v_scale is not None else 0,
                     stats=stats.data_ptr() if stats is not None else 0, max_workers=max_workers,
                     team_helpers=team_helpers, engine=engine, tile_order=tile_order,
                     tile_perm_stride=tile_perm.shape[-1] if tile_perm is not None else 0,
                     tile_perm=tile_perm.data_ptr() if tile_perm is not None else 0,
                     per_head_tables=per_head_tables, workers_per_cu=workers_per_cu, window=window)
    if noalloc:
        if out is None or tiles_used is None or workspace is not None:
            raise ValueError("noalloc needs out and tiles_used and takes no workspace")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        with torch.cuda.device(q.device):  # the entry point runs on the current device
            rc = lib.art_decode_attention_noalloc(ctypes.byref(desc), q.data_ptr(), k_cache.data_ptr(),
                                                  v_cache.data_ptr(),
                                                  block_table.data_ptr() if block_table is not None else None,
                                                  ctx_lens.data_ptr(), tile, eps_scale, eps_dir, out.data_ptr(),
                                                  tiles_used.data_ptr(), stream)
        _check(rc)
        return out, tiles_used
    need = workspace_bytes(desc, tile)
    if need == 0:
        _check(validate(desc, tile, eps_scale, eps_dir))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    desc.workspace = workspace.data_ptr()
    desc.workspace_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if tiles_used is None:
        tiles_used = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.art_decode_attention(ctypes.byref(desc), q.data_ptr(), k_cache.data_ptr(),
                                  v_cache.data_ptr(),
                                  block_table.data_ptr() if block_table is not None else None,
                                  ctx_lens.data_ptr(), tile, eps_scale, eps_dir, out.data_ptr(),
                                  tiles_used.data_ptr(), stream)
    _check(rc)
    return out, tiles_used
