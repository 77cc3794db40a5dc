"""Seeded synthetic inputs for ART decode attention.

This module is the only code shared by the fp64 oracle and the HIP path.  It
holds no attention arithmetic: it draws random caches, rounds them to their
storage types, quantises int8 caches, plants structure (sinks, temperature,
low-logit/large-value rows) and lays caches out contiguously or in pages.

Draw order for every case (numpy PCG64, ``default_rng(seed)``):
  1. Q  [B, Hq, d]                 standard normal (float32 draws)
  2. per (b, kv head) in order: K rows then V rows, [max_ctx, d] each
  3. the structure edits of the case (in the order the case lists them)
  4. the physical block permutation (paged layouts)
Values are drawn in float32 (or float64 where a construction needs it) and
rounded once to the stored type with round-to-nearest-even, so the oracle and
the GPU read identical bytes.

The five named workloads (``WORKLOADS``) are decode-attention configurations
from a single fp32 head up to 128K-token paged caches; ``small`` shrinks batch
and context for oracle-speed tests while keeping every structural feature.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# z-scores used by the temperature construction (upper 5 % and 10 % points of
# the standard normal); beta = z95 + z90 puts ~90 % of the softmax mass on the
# top 5 % of logits when logits ~ N(0, beta^2).
Z95 = 1.6448536269514722
Z90 = 1.2815515655446004
BETA = Z95 + Z90


# ---------------------------------------------------------------- rounding

def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits(x) -> np.ndarray:
    """float -> IEEE binary16 bit patterns (numpy rounds to nearest even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def sink_first_orders(ctx_lens, tile: int, stride: int | None = None, seed: int = 0) -> np.ndarray:
    """Random caller-side tile orders: row b lists its ceil(ctx_lens[b] / tile)
    tiles with tile 0 first and the others shuffled; entries past them are -1."""
    ctx_lens = np.asarray(ctx_lens)
    nts = [-(-int(n) // tile) for n in ctx_lens.ravel()]
    stride = max([1] + nts) if stride is None else stride
    rng = np.random.default_rng(seed)
    perm = np.full((len(nts), stride), -1, np.int32)
    for b, nt in enumerate(nts):
        if nt:
            perm[b, 0] = 0
            perm[b, 1:nt] = 1 + rng.permutation(nt - 1)
    return perm.reshape(ctx_lens.shape + (stride,))


def retained_tables(case: "Case", *, sink_blocks: int, recent_blocks: int, keep_frac: float,
                    seed: int = 0) -> "Case":
    """The same paged cache seen through per-(row, KV head) block tables after a
    block-granular retention policy: every KV head keeps its row's first
    `sink_blocks` and last `recent_blocks` blocks plus a uniformly random
    `keep_frac` share of the blocks between them, drawn per head (0: sinks and
    a recent window only).  The kept blocks are listed in order; a head's
    length counts their tokens (the row's last block may be partial)."""
    assert case.block_size and not case.per_head_tables
    bs = case.block_size
    B, mbps = case.block_table.shape
    rng = np.random.default_rng(seed)
    table = np.zeros((B, case.Hkv, mbps), np.int32)
    lens = np.zeros((B, case.Hkv), np.int32)
    for b in range(B):
        n = int(case.ctx_lens[b])
        nblk = -(-n // bs)
        for g in range(case.Hkv):
            if nblk == 0:
                continue
            head = list(range(min(sink_blocks, nblk)))
            tail = list(range(max(len(head), nblk - recent_blocks), nblk))
            mid = np.arange(len(head), nblk - len(tail))
            kept = head + [int(i) for i in mid[rng.random(mid.size) < keep_frac]] + tail
            table[b, g, :len(kept)] = case.block_table[b, kept]
            last = n - (nblk - 1) * bs if kept[-1] == nblk - 1 else bs
            lens[b, g] = (len(kept) - 1) * bs + last
    return Case(name=case.name + "-retained", B=B, Hq=case.Hq, Hkv=case.Hkv, d=case.d, q=case.q,
                k=case.k, v=case.v, ctx_lens=lens, block_size=bs, block_table=table,
                k_scale=case.k_scale, v_scale=case.v_scale, tile=case.tile,
                eps_scale=case.eps_scale, eps_dir=case.eps_dir, patience=case.patience,
                v_skip_eps=case.v_skip_eps, per_head_tables=True,
                meta=dict(case.meta, kept_blocks=(sink_blocks, recent_blocks, keep_frac)))


def quantize_int8(x):
    """Symmetric per-row int8: scale = fp16(max|x| / 127); code = rint(x/scale).

    Returns (int8 codes shaped like x, uint16 fp16-bit scales shaped x.shape[:-1]).
    Rows of zeros get scale 1 and codes 0.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float16)
    scale = np.where(scale == 0, np.float16(1.0), scale)
    s32 = scale.astype(np.float32)[..., None]
    codes = np.clip(np.rint(x / s32), -127, 127).astype(np.int8)
    return codes, scale.view(np.uint16)


def quantize_int4(x):
    """Symmetric per-row int4: scale = fp16(max|x| / 7); code = rint(x/scale)
    clipped to [-7, 7]; codes packed two per byte, element 2i in the low nibble
    of byte i (two's complement nibbles).

    Returns (uint8 array shaped like x with the last dim halved, uint16 fp16-bit
    scales shaped x.shape[:-1]).  Rows of zeros get scale 1 and codes 0.
    """
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] % 2 == 0
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(7.0)).astype(np.float16)
    scale = np.where(scale == 0, np.float16(1.0), scale)
    s32 = scale.astype(np.float32)[..., None]
    codes = np.clip(np.rint(x / s32), -7, 7).astype(np.int8)
    nib = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8), scale.view(np.uint16)


# ---------------------------------------------------------------- container

@dataclass
class Case:
    """Host arrays of one decode-attention call plus its parameters."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    q: np.ndarray                 # float32 or uint16 (bf16 bits) [B, Hq, d]
    k: np.ndarray                 # cache, see layout
    v: np.ndarray
    ctx_lens: np.ndarray          # int32 [B]
    block_size: int = 0           # 0: contiguous [B, Hkv, max_ctx, d]; else paged [nb, Hkv, bs, d]
    block_table: np.ndarray | None = None  # int32 [B, max_blocks_per_seq]
    k_scale: np.ndarray | None = None      # uint16 fp16 bits (int8 caches)
    v_scale: np.ndarray | None = None
    tile: int = 64
    eps_scale: float = 1e-3
    eps_dir: float = 1e-4
    patience: int = 1
    v_skip_eps: float = 0.0
    per_head_tables: bool = False  # ctx_lens [B, Hkv], block_table [B, Hkv, mbps], tile_perm [B, Hkv, stride]
    order: int = 0                # tile order: 0 ascending, 1 tile 0 then most recent first, 2 tile_perm
    tile_perm: np.ndarray | None = None    # int32 [B, stride]: row b's tiles in visiting order (order 2)
    meta: dict = field(default_factory=dict)

    @property
    def q_dtype(self) -> str:
        return "f32" if self.q.dtype == np.float32 else "bf16"

    @property
    def kv_dtype(self) -> str:
        return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16",
                np.dtype(np.int8): "i8", np.dtype(np.uint8): "i4"}[self.k.dtype]

    @property
    def max_ctx(self) -> int:
        if self.block_size:
            return self.block_table.shape[-1] * self.block_size
        return self.k.shape[2]

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0] if self.block_size else 0

    def kv_bytes_full(self) -> int:
        """Bytes of K+V (+ scales) covering every position 0..ctx_len-1."""
        per = self.k.shape[-1] * self.k.dtype.itemsize * 2 + (4 if self.kv_dtype in ("i8", "i4") else 0)
        return int(self.ctx_lens.astype(np.int64).sum()) * self.Hkv * per


# ---------------------------------------------------------------- builders

def _store(x, kv_dtype):
    if kv_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32), None
    if kv_dtype == "bf16":
        return bf16_bits(x), None
    if kv_dtype == "i8":
        return quantize_int8(x)
    if kv_dtype == "i4":
        return quantize_int4(x)
    raise ValueError(kv_dtype)


def make_case(name, *, B, Hq, Hkv, d, ctx_lens, seed=0, kv_dtype="bf16", q_dtype="bf16",
              block_size=0, num_blocks=None, q_mode="normal", sinks=None,
              planted=None, v_mean=0.0, **params) -> Case:
    """Build one case.

    q_mode: "normal" (N(0,1)) or "temperature" (q = BETA*sqrt(d)*unit(N(0,I))).
    sinks: None or (count, scale_mode) with scale_mode "sqrt_d" (k = 3 sqrt(d) qhat_g
           + N(0,I)) or "literal" (k = 3 qhat_g + N(0,I)); qhat_g = unit(sum of the
           group's unit queries).  Applied at positions 0..count-1 of every KV head.
    planted: None or fraction f: per (b, kv head), round(f*max_ctx) positions drawn
           uniformly without replacement get keys whose logit is exactly -2 sigma_h
           for every query head of the group (sigma_h = ||q_h||/sqrt(d)) and V rows
           scaled by 50.
    v_mean: constant added to every V entry (drift variant).
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32).reshape(B)
    G = Hq // Hkv
    assert Hq % Hkv == 0
    rng = np.random.default_rng(seed)
    max_ctx = int(ctx_lens.max(initial=0))
    unit = block_size or 16  # contiguous rows are padded to a multiple of 16 tokens
    max_ctx = max(-(-max_ctx // unit) * unit, unit)

    # 1. queries
    qf = rng.standard_normal((B, Hq, d), dtype=np.float32)
    if q_mode == "temperature":
        qf = qf / np.linalg.norm(qf, axis=-1, keepdims=True) * np.float32(BETA * np.sqrt(d))
    q = np.ascontiguousarray(qf, np.float32) if q_dtype == "f32" else bf16_bits(qf)
    qv = qf.astype(np.float64) if q_dtype == "f32" else bf16_value(q).astype(np.float64)

    # 2. logical K, V per (b, kv head) -- stored directly in their storage type
    k_log = [[None] * Hkv for _ in range(B)]
    v_log = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        for g in range(Hkv):
            k_log[b][g] = rng.standard_normal((max_ctx, d), dtype=np.float32)
            v_log[b][g] = rng.standard_normal((max_ctx, d), dtype=np.float32)
            if v_mean:
                v_log[b][g] += np.float32(v_mean)

    # 3. structure edits
    meta = {"q_mode": q_mode}
    if sinks is not None:
        count, mode = sinks
        mult = 3.0 * np.sqrt(d) if mode == "sqrt_d" else 3.0
        noise = rng.standard_normal((B, Hkv, count, d), dtype=np.float32)
        for b in range(B):
            for g in range(Hkv):
                qs = qv[b, g * G:(g + 1) * G]
                qs = qs / np.linalg.norm(qs, axis=-1, keepdims=True)
                qhat = qs.sum(0)
                qhat /= np.linalg.norm(qhat)
                k_log[b][g][:count] = (mult * qhat[None, :] + noise[b, g]).astype(np.float32)
        meta["sinks"] = (count, mode)
    if planted is not None:
        npl = int(round(planted * max_ctx))
        pos_all = np.zeros((B, Hkv, npl), np.int64)
        for b in range(B):
            for g in range(Hkv):
                pos = np.sort(rng.choice(min(max_ctx, int(ctx_lens[b]) or max_ctx), size=npl,
                                         replace=False))
                pos_all[b, g] = pos
                Qg = qv[b, g * G:(g + 1) * G]                       # [G, d]
                target = -2.0 * np.linalg.norm(Qg, axis=-1)          # q_h.k = -2||q_h||
                z = rng.standard_normal((npl, d))
                # projection of z onto the orthogonal complement of rowspace(Qg)
                coef = np.linalg.solve(Qg @ Qg.T, Qg @ z.T)          # [G, npl]
                z_perp = z - (Qg.T @ coef).T
                base = Qg.T @ np.linalg.solve(Qg @ Qg.T, target)     # [d]
                k_log[b][g][pos] = (z_perp + base[None, :]).astype(np.float32)
                v_log[b][g][pos] *= np.float32(50.0)
        meta["planted_positions"] = pos_all

    # 4. layout
    k_scale = v_scale = None
    if block_size:
        nb_seq = max_ctx // block_size
        nb = num_blocks if num_blocks is not None else B * nb_seq
        assert nb >= B * nb_seq
        perm = rng.permutation(nb)[:B * nb_seq].astype(np.int32)
        block_table = perm.reshape(B, nb_seq)
        shape = (nb, Hkv, block_size, d // 2 if kv_dtype == "i4" else d)
        k_arr = np.zeros(shape, _storage_np(kv_dtype))
        v_arr = np.zeros(shape, _storage_np(kv_dtype))
        if kv_dtype in ("i8", "i4"):
            k_scale = np.zeros(shape[:-1], np.uint16)
            v_scale = np.zeros(shape[:-1], np.uint16)
        for b in range(B):
            rows = block_table[b]
            for g in range(Hkv):
                for src, dst, sc in ((k_log, k_arr, k_scale), (v_log, v_arr, v_scale)):
                    data, scale = _store(src[b][g], kv_dtype)
                    dst[rows, g] = data.reshape(nb_seq, block_size, shape[-1])
                    if sc is not None:
                        sc[rows, g] = scale.reshape(nb_seq, block_size)
                src = None
            k_log[b] = v_log[b] = None  # free as we go
    else:
        block_table = None
        shape = (B, Hkv, max_ctx, d // 2 if kv_dtype == "i4" else d)
        k_arr = np.zeros(shape, _storage_np(kv_dtype))
        v_arr = np.zeros(shape, _storage_np(kv_dtype))
        if kv_dtype in ("i8", "i4"):
            k_scale = np.zeros(shape[:-1], np.uint16)
            v_scale = np.zeros(shape[:-1], np.uint16)
        for b in range(B):
            for g in range(Hkv):
                for src, dst, sc in ((k_log, k_arr, k_scale), (v_log, v_arr, v_scale)):
                    data, scale = _store(src[b][g], kv_dtype)
                    dst[b, g] = data
                    if sc is not None:
                        sc[b, g] = scale
            k_log[b] = v_log[b] = None
    return Case(name=name, B=B, Hq=Hq, Hkv=Hkv, d=d, q=q, k=k_arr, v=v_arr,
                ctx_lens=ctx_lens, block_size=block_size, block_table=block_table,
                k_scale=k_scale, v_scale=v_scale, meta=meta, **params)


def _storage_np(kv_dtype):
    return {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "i4": np.uint8}[kv_dtype]


# ---------------------------------------------------------------- named workloads

WORKLOADS = {
    1: "single head, d 64, ctx 1024, fp32 contiguous",
    2: "B1 32q/8kv d128 ctx 8192, bf16 contiguous, 4 sink tokens",
    3: "B16 32q/8kv d128 ctx 32768, bf16 paged bs16, temperature (top 5% ~ 90% mass)",
    4: "B4 40q/8kv d128 ctx 131072, bf16 paged bs16, 0.1% planted -2sigma/x50 rows",
    5: "B8 32q/8kv d128 ctx 32768, int8 paged bs16 + fp16 scales, temperature",
}


def config(n: int, seed: int = 0, *, small: bool = False, batch=None, ctx=None,
           sink_mode: str = "sqrt_d", **params) -> Case:
    """Named workload n (1..5).  small=True shrinks batch and context for the
    oracle while keeping every structural feature; batch/ctx override sizes."""
    if n == 1:
        B, Hq, Hkv, d, n_ctx = 1, 1, 1, 64, 1024
        kw = dict(kv_dtype="f32", q_dtype="f32")
    elif n == 2:
        B, Hq, Hkv, d, n_ctx = 1, 32, 8, 128, 8192
        kw = dict(sinks=(4, sink_mode))
    elif n == 3:
        B, Hq, Hkv, d, n_ctx = 16, 32, 8, 128, 32768
        kw = dict(block_size=16, q_mode="temperature")
    elif n == 4:
        B, Hq, Hkv, d, n_ctx = 4, 40, 8, 128, 131072
        kw = dict(block_size=16, planted=0.001)
    elif n == 5:
        B, Hq, Hkv, d, n_ctx = 8, 32, 8, 128, 32768
        kw = dict(block_size=16, q_mode="temperature", kv_dtype="i8")
        params.setdefault("v_skip_eps", 1e-6)
    else:
        raise ValueError(n)
    if small:
        B = min(B, 2)
        n_ctx = min(n_ctx, 2048 if n != 4 else 8192)
    if batch is not None:
        B = batch
    if ctx is not None:
        n_ctx = ctx
    kw.update(params)  # a caller's setting (e.g. kv_dtype) overrides the workload's
    return make_case(f"config{n}{'-small' if small else ''}", B=B, Hq=Hq, Hkv=Hkv, d=d,
                     ctx_lens=[n_ctx] * B, seed=seed, **kw)


def to_device(case):
    """The case's arrays as device tensors (torch, cuda:0): bf16 and fp16 bit
    patterns are reinterpreted, not converted, so the GPU reads the bytes the
    oracle reads.  Plumbing only: no attention arithmetic."""
    import torch
    dev = torch.device("cuda:0")

    def t(a, as_f16=False):
        if a is None:
            return None
        if a.dtype == np.uint16:
            x = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
            x = x.view(torch.float16 if as_f16 else torch.bfloat16)
        else:
            x = torch.from_numpy(np.ascontiguousarray(a))
        return x.to(dev)

    return dict(q=t(case.q), k=t(case.k), v=t(case.v), ctx=t(case.ctx_lens.astype(np.int32)),
                bt=t(case.block_table), ks=t(case.k_scale, as_f16=True),
                vs=t(case.v_scale, as_f16=True),
                perm=t(None if case.tile_perm is None else case.tile_perm.astype(np.int32)))
