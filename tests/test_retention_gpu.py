"""GPU parity with per-(row, KV head) tables: ART on top of a per-head
retention or eviction policy (ART summary, section 2.4: an orthogonal
control layer).  Every engine against the fp64 oracle on the same tables;
same bar as the other parity tests."""
import copy

import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import check_parity, run_gpu, to_device
from tests.helpers import contiguous_case
from tests.test_parity_gpu import _run_and_check

pytestmark = pytest.mark.gpu

ENGINE_TEAM, ENGINE_POOL, ENGINE_ROUND = 1, 2, 6
ORDER_RECENT, ORDER_LIST = 1, 2


def retained(c, keep, seed=0, sink=4, recent=32):
    return A.retained_tables(c, sink_blocks=sink, recent_blocks=recent, keep_frac=keep, seed=seed)


@pytest.mark.parametrize("keep", [0.0, 0.5])
@pytest.mark.parametrize("n", [3, 4, 5])
def test_retained_named_workloads(keep, n):
    c = retained(A.config(n, small=True), keep, seed=n)
    _run_and_check(c, f"config{n} kept {keep} art")
    _run_and_check(c, f"config{n} kept {keep} full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


def test_retained_every_engine():
    c = retained(A.config(3, small=True), 0.5, seed=9)
    _run_and_check(c, "retained team", engine=ENGINE_TEAM)
    _run_and_check(c, "retained pool", engine=ENGINE_POOL)
    _run_and_check(c, "retained round", engine=ENGINE_ROUND)
    _run_and_check(c, "retained work-sharing", max_workers=96)
    _run_and_check(c, "retained helpers", team_helpers=1)


@pytest.mark.parametrize("kv,q,d", [("f32", "f32", 128), ("bf16", "bf16", 64), ("i8", "bf16", 128), ("i4", "bf16", 128),
                                    ("i4", "bf16", 64)])
def test_retained_other_paths(kv, q, d):
    c = A.make_case("kept", B=3, Hq=8, Hkv=2, d=d, ctx_lens=[1500, 700, 333], kv_dtype=kv,
                    q_dtype=q, block_size=16, q_mode="temperature", seed=23,
                    v_skip_eps=1e-6 if kv in ("i8", "i4") else 0.0)
    c = retained(c, 0.5, seed=2, sink=2, recent=16)
    _run_and_check(c, f"{kv}/{q} d{d} retained art")
    _run_and_check(c, f"{kv}/{q} d{d} retained full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


@pytest.mark.parametrize("order", [ORDER_RECENT, ORDER_LIST])
def test_retained_with_tile_orders(order):
    c = retained(A.config(3, small=True), 0.5, seed=4)
    c.order = order
    if order == ORDER_LIST:
        c.tile_perm = A.sink_first_orders(c.ctx_lens, c.tile, stride=-(-c.max_ctx // c.tile), seed=6)
    _run_and_check(c, f"retained order {order} art")
    _run_and_check(c, f"retained order {order} pool", engine=ENGINE_POOL)
    _run_and_check(c, f"retained order {order} full", eps_scale=0.0, eps_dir=0.0)


def test_identical_per_head_tables_equal_shared_tables():
    c = A.config(3, small=True)
    p = copy.copy(c)
    p.per_head_tables = True
    p.ctx_lens = np.repeat(c.ctx_lens[:, None], c.Hkv, axis=1)
    p.block_table = np.repeat(c.block_table[:, None], c.Hkv, axis=1)
    for kw in (dict(), dict(eps_scale=0.0, eps_dir=0.0)):
        o1, u1 = run_gpu(c, **kw)
        o2, u2 = run_gpu(p, **kw)
        assert np.array_equal(u1, u2) and np.array_equal(o1, o2), kw
    # the pool merges per-worker states whose tiles depend on the claims: equal
    # to rounding only
    o1, u1 = run_gpu(c, engine=ENGINE_POOL)
    o2, u2 = run_gpu(p, engine=ENGINE_POOL)
    assert np.array_equal(u1, u2)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5)


def test_contiguous_per_head_lengths():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, 8, 128)) * 2
    K = rng.standard_normal((3, 2, 2048, 128))
    V = rng.standard_normal((3, 2, 2048, 128))
    c = contiguous_case(q, K, V, kv="bf16", qd="bf16", tile=64)
    c.per_head_tables = True
    c.ctx_lens = np.array([[2048, 1000], [1, 0], [777, 1536]], np.int32)
    _run_and_check(c, "contiguous per-head lengths art")
    out, used, _ = _run_and_check(c, "contiguous per-head lengths full", eps_scale=0.0, eps_dir=0.0)
    assert (used[1, 4:] == 0).all() and (out[1, 4:] == 0).all()


def test_invalid_per_head_entries_reported_per_group():
    c = retained(A.config(3, small=True, batch=3), 1.0, seed=5)
    c.ctx_lens[1, 1] = c.block_table.shape[-1] * 16 + 1   # (row 1, KV head 1): longer than its table
    c.block_table[2, 0, 3] = c.num_blocks + 9             # (row 2, KV head 0): bad block in tile 0
    G = c.Hq // c.Hkv
    for kw in (dict(eps_scale=0.0, eps_dir=0.0), dict()):
        out, used = run_gpu(c, **kw)
        assert (used[1, G:2 * G] == -1).all() and np.isnan(out[1, G:2 * G]).all()
        assert (used[2, :G] == -1).all() and np.isnan(out[2, :G]).all()
        assert (used[1, :G] > 0).all() and (used[2, G:2 * G] > 0).all()
    good = copy.deepcopy(c)
    good.ctx_lens[1, 1] = 16
    good.block_table[2, 0, 3] = 0
    out, used = run_gpu(c)
    check_parity(good, out, used, rows=[0])


@pytest.mark.parametrize("tile", [16, 32, 128])
def test_retained_other_tile_sizes(tile):
    c = retained(A.config(3, small=True, batch=2, ctx=1500, tile=tile), 0.5, seed=tile, sink=2, recent=16)
    c.order = ORDER_LIST
    c.tile_perm = A.sink_first_orders(c.ctx_lens, tile, stride=-(-c.max_ctx // tile), seed=3)
    _run_and_check(c, f"retained tile {tile} list art")
    _run_and_check(c, f"retained tile {tile} list full", eps_scale=0.0, eps_dir=0.0)
