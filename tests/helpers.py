"""Small builders shared by the tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np

from art_inputs import Case, bf16_bits


def contiguous_case(q, K, V, ctx_lens=None, *, kv="f32", qd="f32", name="custom", **params):
    """Case from float arrays: q [B,Hq,d], K/V [B,Hkv,n,d] (logical = storage order)."""
    q = np.asarray(q, np.float32)
    K = np.asarray(K, np.float32)
    V = np.asarray(V, np.float32)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    if ctx_lens is None:
        ctx_lens = [K.shape[2]] * B
    conv = (lambda x: x) if kv == "f32" else bf16_bits
    qconv = (lambda x: x) if qd == "f32" else bf16_bits
    return Case(name=name, B=B, Hq=Hq, Hkv=Hkv, d=d, q=qconv(q), k=conv(K), v=conv(V),
                ctx_lens=np.asarray(ctx_lens, np.int32), **params)


def to_paged(case: Case, block_size: int, seed: int, extra_blocks: int = 0) -> Case:
    """Same logical cache as a contiguous case, laid out in randomly permuted pages."""
    assert case.block_size == 0 and not case.per_head_tables
    B, Hkv, n, d = case.k.shape
    nbs = -(-n // block_size)
    nb = B * nbs + extra_blocks
    perm = np.random.default_rng(seed).permutation(nb)[:B * nbs].astype(np.int32)
    table = perm.reshape(B, nbs)

    def pack(arr, tail):
        out = np.zeros((nb, Hkv, block_size) + tail, arr.dtype)
        padded = np.zeros((B, Hkv, nbs * block_size) + tail, arr.dtype)
        padded[:, :, :n] = arr
        for b in range(B):
            out[table[b]] = padded[b].reshape((Hkv, nbs, block_size) + tail).swapaxes(0, 1)
        return out

    return Case(name=case.name + "-paged", B=B, Hq=case.Hq, Hkv=Hkv, d=d, q=case.q,
                k=pack(case.k, (d,)), v=pack(case.v, (d,)), ctx_lens=case.ctx_lens,
                block_size=block_size, block_table=table,
                k_scale=None if case.k_scale is None else pack(case.k_scale, ()),
                v_scale=None if case.v_scale is None else pack(case.v_scale, ()),
                tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                patience=case.patience, v_skip_eps=case.v_skip_eps, order=case.order,
                tile_perm=case.tile_perm, meta=dict(case.meta))


def designed_case(fx, seed=0):
    """Cache whose running output follows the fixture's probe sequence (see golden/README.md)."""
    T, d, nt = fx["tile"], fx["d"], fx["n_tiles"]
    rho = np.asarray(fx["rho"], np.float64)
    th = np.asarray(fx["theta"], np.float64)
    y = np.zeros((nt, d))
    y[:, 0] = rho * np.cos(th)
    y[:, 1] = rho * np.sin(th)
    u = np.zeros((nt, d))
    for t in range(nt):
        u[t] = (t + 1) * y[t] - (t * y[t - 1] if t else 0.0)
    rng = np.random.default_rng(seed)
    u[:, 8:] = rng.uniform(-10, 10, size=(nt, d - 8))  # distractor outside the probe
    V = np.repeat(u, T, axis=0)[None, None]            # [1, 1, nt*T, d]
    K = np.zeros_like(V)
    q = rng.standard_normal((1, 1, d))
    return contiguous_case(q, K, V, tile=T)


def run_oracle(case, **kw):
    import oracle
    args = dict(tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                patience=case.patience, v_skip_eps=case.v_skip_eps,
                block_table=case.block_table, block_size=case.block_size,
                k_scale=case.k_scale, v_scale=case.v_scale, order=case.order,
                tile_perm=case.tile_perm, per_head_tables=case.per_head_tables)
    args.update(kw)
    return oracle.decode(case.q, case.k, case.v, case.ctx_lens, **args)
