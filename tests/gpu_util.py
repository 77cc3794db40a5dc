"""Helpers of the GPU parity tests: move a case to the device, run the HIP
library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

from art_inputs import to_device  # noqa: F401  (re-exported for the tests)
from tests import bruteforce as BF
from tests.helpers import run_oracle

NEAR_REL = 1e-3  # metric within 1e-3 relative of its threshold: the decision may differ


def tol_for(case) -> float:
    return 1e-5 if case.kv_dtype == "f32" else 2e-3


def run_gpu(case, dev=None, **kw):
    import torch
    import kv_cache_bandwidth_amd as art
    dev = dev or to_device(case)
    args = dict(block_table=dev["bt"], tile=case.tile, eps_scale=case.eps_scale,
                eps_dir=case.eps_dir, patience=case.patience, v_skip_eps=case.v_skip_eps,
                k_scale=dev["ks"], v_scale=dev["vs"], tile_order=case.order,
                tile_perm=dev["perm"] if case.order == 2 else None,
                per_head_tables=case.per_head_tables)
    args.update(kw)
    out, used = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], **args)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), used.cpu().numpy()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_parity(case, out, used, *, eps_scale=None, eps_dir=None, patience=None, v_skip_eps=None,
                 rows=None, ora=None):
    """Compare GPU (out, used) with the oracle on batch rows `rows` (default all).

    tiles_used must be equal, except for heads where some evaluated metric lies
    within NEAR_REL of its threshold; those are reported and their output is
    checked against softmax attention over the GPU's own prefix.  Returns a
    dict of statistics."""
    es = case.eps_scale if eps_scale is None else eps_scale
    ed = case.eps_dir if eps_dir is None else eps_dir
    pt = case.patience if patience is None else patience
    vk = case.v_skip_eps if v_skip_eps is None else v_skip_eps
    rows = list(range(case.B)) if rows is None else list(rows)
    sub = _subset(case, rows)
    if ora is None:
        ora = run_oracle(sub, eps_scale=es, eps_dir=ed, patience=pt, v_skip_eps=vk)
    g_out, g_used = out[rows], used[rows]
    tol = tol_for(case)
    mism = np.argwhere(g_used != ora.tiles_used)
    near = []
    if len(mism):
        tr = run_oracle(sub, eps_scale=0.0, eps_dir=0.0, patience=pt, v_skip_eps=vk, trace=True).trace
        for bi, h in mism:
            hi = max(int(g_used[bi, h]), int(ora.tiles_used[bi, h]))
            ds, dd = tr[bi, h, 1:hi, 2], tr[bi, h, 1:hi, 3]
            close = (np.abs(ds - es) <= NEAR_REL * es) | (np.abs(dd - ed) <= NEAR_REL * ed)
            assert close.any(), (f"tiles_used differs away from the thresholds at row {rows[bi]} head {h}: "
                                 f"gpu {g_used[bi, h]} oracle {ora.tiles_used[bi, h]}")
            near.append((rows[bi], int(h), int(g_used[bi, h]), int(ora.tiles_used[bi, h])))
            if g_used[bi, h] > 0:
                # the GPU's own stop: its output must be attention over the
                # positions it visited (with the V-skip rule, when on)
                ref, slack = prefix_reference(sub, bi, int(h), int(g_used[bi, h]), vk, pt)
                assert np.isfinite(g_out[bi, h]).all() and np.abs(g_out[bi, h] - ref).max() <= tol + slack, \
                    f"near-threshold head {rows[bi]},{h}: output differs from attention over its prefix"
    same = g_used == ora.tiles_used
    # every head the oracle finishes must have a finite GPU output (a NaN in
    # one head must not hide behind the others)
    finite = np.isfinite(g_out).all(axis=-1)
    bad = same & (ora.tiles_used >= 0) & ~finite
    assert not bad.any(), f"non-finite GPU output at (row, head) {np.argwhere(bad)[:4].tolist()}"
    err = np.abs(g_out - ora.out).max(axis=-1)
    err = np.where(same, err, 0.0)
    maxerr = float(np.max(err)) if err.size else 0.0
    assert maxerr <= tol, f"max |out - oracle| = {maxerr:.3e} > {tol:.1e}"
    return dict(max_abs=maxerr, near=near, heads=int(same.size), tiles_used=ora.tiles_used)


def prefix_reference(case, b, h, steps, v_skip_eps, patience):
    """Attention of head h of row b over the tiles of its first `steps`
    visiting steps, and the slack beyond the parity tolerance it is compared
    with.  Without the V skip: brute-force softmax over those positions (no
    slack).  With it, in ascending order: the oracle in full mode on the row
    cut after those tiles (the skip rule's running max follows the same
    tiles, so the prefix run is exactly the stopped head's; no slack).  Other
    orders with the V skip: brute force without the skip, with the skip's own
    bound as slack (a left-out row's normalised weight is below v_skip_eps)."""
    pos = visited_positions(case, b, h, steps)
    if v_skip_eps == 0:
        return BF.attention_at(case, b, h, pos), 0.0
    if case.order == 0 and not case.per_head_tables:
        import copy
        c = copy.copy(_subset(case, [b]))
        n = int(c.ctx_lens[0])
        c.ctx_lens = np.array([min(n, steps * case.tile)], np.int32)
        return run_oracle(c, eps_scale=0.0, eps_dir=0.0, patience=patience, v_skip_eps=v_skip_eps).out[0, h], 0.0
    G = case.Hq // case.Hkv
    vmax = float(np.abs(BF.logical_rows(case, "v", b, h // G, max(pos) + 1)[pos]).max()) if pos else 0.0
    return BF.attention_at(case, b, h, pos), len(pos) * v_skip_eps * vmax


def visited_positions(case, b, h, steps):
    """Positions of the tiles head h of row b visits in its first `steps` steps."""
    g = h // (case.Hq // case.Hkv)
    sq = (b, g) if case.per_head_tables else (b,)
    T, n = case.tile, int(case.ctx_lens[sq])
    nt = -(-n // T)
    if case.order == 0:
        seq = list(range(nt))
    elif case.order == 1:
        seq = [0] + list(range(nt - 1, 0, -1))
    else:
        seq = [int(x) for x in case.tile_perm[sq][:nt]]
    return [j for s in seq[:steps] for j in range(s * T, min(n, (s + 1) * T))]


def _subset(case, rows):
    if rows == list(range(case.B)):
        return case
    import copy
    c = copy.copy(case)
    c.B = len(rows)
    c.q = np.ascontiguousarray(case.q[rows])
    c.ctx_lens = np.ascontiguousarray(case.ctx_lens[rows])
    if case.tile_perm is not None:
        c.tile_perm = np.ascontiguousarray(case.tile_perm[rows])
    if case.block_size:
        c.block_table = np.ascontiguousarray(case.block_table[rows])
    else:
        c.k = np.ascontiguousarray(case.k[rows])
        c.v = np.ascontiguousarray(case.v[rows])
        if case.k_scale is not None:
            c.k_scale = np.ascontiguousarray(case.k_scale[rows])
            c.v_scale = np.ascontiguousarray(case.v_scale[rows])
    return c
