"""GPU parity of the tile orders (ART summary, section 2.4: the tile sequence
may be reordered, recency- or importance-first; block 0, the attention sink,
is evaluated first).  Every engine against the fp64 oracle, which applies the
same index remap; same bar as the other parity tests."""
import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import check_parity, log, run_gpu, to_device
from tests.helpers import contiguous_case
from tests.test_parity_gpu import _run_and_check

pytestmark = pytest.mark.gpu

ORDER_RECENT, ORDER_LIST = 1, 2
ENGINE_TEAM, ENGINE_POOL, ENGINE_ROUND = 1, 2, 6


def ordered(c, order, seed=0):
    c.order = order
    c.tile_perm = None
    if order == ORDER_LIST:
        stride = -(-c.max_ctx // c.tile)
        c.tile_perm = A.sink_first_orders(c.ctx_lens, c.tile, stride=stride, seed=seed)
    return c


@pytest.mark.parametrize("order", [ORDER_RECENT, ORDER_LIST])
@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_orders_named_workloads(order, n):
    c = ordered(A.config(n, small=n != 2), order, seed=n)
    _run_and_check(c, f"config{n} order {order} art")
    _run_and_check(c, f"config{n} order {order} full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


@pytest.mark.parametrize("order", [ORDER_RECENT, ORDER_LIST])
def test_orders_every_engine(order):
    c = ordered(A.config(3, small=True), order, seed=11)
    _run_and_check(c, f"config3 order {order} team", engine=ENGINE_TEAM)
    _run_and_check(c, f"config3 order {order} pool", engine=ENGINE_POOL)
    _run_and_check(c, f"config3 order {order} round", engine=ENGINE_ROUND)
    # 128 groups of 128 steps: two rounds
    c8 = ordered(A.config(3, small=True, batch=16, ctx=8192), order, seed=12)
    _run_and_check(c8, f"config3 ctx 8192 order {order} round", engine=ENGINE_ROUND)
    _run_and_check(c, f"config3 order {order} work-sharing", max_workers=96)
    _run_and_check(c, f"config3 order {order} helpers", team_helpers=1)


@pytest.mark.parametrize("order", [ORDER_RECENT, ORDER_LIST])
@pytest.mark.parametrize("kv,q,d", [("f32", "f32", 128), ("bf16", "bf16", 64), ("i8", "bf16", 128), ("i4", "bf16", 128),
                                    ("i4", "bf16", 64)])
def test_orders_other_paths(order, kv, q, d):
    # fp32 caches and head dim 64 run the one-tile-at-a-time kernels; int8 with
    # a V skip runs the team kernel's skip path
    c = A.make_case("orders", B=3, Hq=8, Hkv=2, d=d, ctx_lens=[700, 333, 1000], kv_dtype=kv,
                    q_dtype=q, block_size=16, q_mode="temperature", seed=21,
                    v_skip_eps=1e-6 if kv in ("i8", "i4") else 0.0)
    ordered(c, order, seed=3)
    _run_and_check(c, f"{kv}/{q} d{d} order {order} art")
    _run_and_check(c, f"{kv}/{q} d{d} order {order} full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


def test_orders_ragged_empty_rows():
    c = A.make_case("ragged-orders", B=6, Hq=8, Hkv=2, d=128, ctx_lens=[1000, 1, 0, 63, 64, 65],
                    block_size=16, q_mode="temperature", seed=3)
    for order in (ORDER_RECENT, ORDER_LIST):
        ordered(c, order, seed=5)
        out, used, _ = _run_and_check(c, f"ragged order {order} art")
        assert (used[2] == 0).all() and (out[2] == 0).all()


def test_recent_order_stops_early_where_recent_tokens_dominate():
    # scores high on the last tile only: the ascending order meets it last and
    # runs to the end, sink + most-recent-first meets it second and stops soon
    T, nt, d = 64, 40, 128
    n = T * nt
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 8, d))
    K = np.repeat(rng.standard_normal((1, 1, n, d)) * 0.05, 2, axis=1)
    qm = q[0, :4].mean(0)
    K[0, 0, -T:] += 20.0 * qm / np.linalg.norm(qm)
    qm = q[0, 4:].mean(0)
    K[0, 1, -T:] += 20.0 * qm / np.linalg.norm(qm)
    V = rng.standard_normal((1, 2, n, d))
    c = contiguous_case(q, K, V, kv="bf16", qd="bf16", tile=T, eps_scale=1e-3, eps_dir=1e-4,
                        patience=2)
    _, asc, _ = _run_and_check(c, "dominant recent tile, ascending")
    c.order = ORDER_RECENT
    _, rec, _ = _run_and_check(c, "dominant recent tile, recent first")
    log(f"[orders] tiles_used ascending {asc.tolist()} recent-first {rec.tolist()}")
    assert rec.max() < asc.min()


def test_invalid_list_entries_reported_per_row():
    c = ordered(A.config(3, small=True, batch=3), ORDER_LIST, seed=2)
    c.tile_perm[1, 0] = 1          # row 1: step 0 is not the sink
    c.tile_perm[2, 3] = 10 ** 6    # row 2: a tile that does not exist, at step 3
    out, used = run_gpu(c, eps_scale=0.0, eps_dir=0.0)
    assert (used[1] == -1).all() and np.isnan(out[1]).all()
    assert (used[2] == -1).all() and np.isnan(out[2]).all()
    check_parity(c, out, used, eps_scale=0.0, eps_dir=0.0, rows=[0])
    out, used = run_gpu(c)
    assert (used[1] == -1).all() and np.isnan(out[1]).all()
    # ART mode: a head of row 2 that stops within 3 steps never reads the bad entry
    assert ((used[2] == -1) | ((used[2] >= 1) & (used[2] <= 3))).all()
    check_parity(c, out, used, rows=[0])


def test_list_entries_past_the_stop_are_not_used():
    # constant V rows: the probe never moves, every head stops after step 1
    # (patience 1); the list holds garbage from step 2 on, which the kernels may
    # prefetch but must not let into any result
    T, nt, d = 64, 24, 128
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 8, d))
    K = rng.standard_normal((2, 2, T * nt, d))
    V = np.repeat(rng.standard_normal((2, 2, 1, d)), T * nt, axis=2)
    c = contiguous_case(q, K, V, kv="bf16", qd="bf16", tile=T, eps_scale=1e-3, eps_dir=1e-4)
    ordered(c, ORDER_LIST, seed=8)
    c.tile_perm[:, 2:] = -7
    dev = to_device(c)
    for kw in (dict(), dict(engine=ENGINE_POOL), dict(max_workers=32)):
        out, used = run_gpu(c, dev, **kw)
        assert (used == 2).all(), (kw, used)
        check_parity(c, out, used)


def test_order_does_not_change_full_attention():
    # permutation invariance (section 2.4): full attention in any order agrees
    # to rounding with the ascending order
    c = A.config(3, small=True)
    dev = to_device(c)
    o0, u0 = run_gpu(c, dev, eps_scale=0.0, eps_dir=0.0)
    for order in (ORDER_RECENT, ORDER_LIST):
        ordered(c, order, seed=13)
        dev = to_device(c)
        o, u = run_gpu(c, dev, eps_scale=0.0, eps_dir=0.0)
        assert np.array_equal(u, u0)
        np.testing.assert_allclose(o, o0, rtol=0, atol=2e-5)


@pytest.mark.parametrize("tile", [16, 32, 128])
@pytest.mark.parametrize("order", [ORDER_RECENT, ORDER_LIST])
def test_orders_other_tile_sizes(tile, order):
    # tiles other than 64 tokens run the one-tile-at-a-time matrix-core kernels
    c = ordered(A.config(3, small=True, batch=2, ctx=1000, tile=tile), order, seed=tile)
    _run_and_check(c, f"tile {tile} order {order} art")
    _run_and_check(c, f"tile {tile} order {order} full", eps_scale=0.0, eps_dir=0.0)
