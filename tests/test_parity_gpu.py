"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar: tiles_used equal (except near-threshold heads, reported), outputs within
max-abs 2e-3 for bf16/int8 caches and 1e-5 for fp32 caches.
"""
import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import check_parity, log, run_gpu, to_device
from tests.helpers import contiguous_case, to_paged

pytestmark = pytest.mark.gpu


def _run_and_check(case, label, **kw):
    log(f"[parity] {label}: B={case.B} Hq={case.Hq} Hkv={case.Hkv} d={case.d} "
        f"ctx={case.ctx_lens.tolist()[:4]} kv={case.kv_dtype} T={case.tile} {kw}")
    out, used = run_gpu(case, **kw)
    r = check_parity(case, out, used,
                     **{k: v for k, v in kw.items()
                        if k not in ("max_workers", "team_helpers", "engine", "stats", "workers_per_cu", "window")})
    log(f"[parity] {label}: max_abs={r['max_abs']:.3e} near={r['near']} "
        f"mean tiles_used={np.mean(r['tiles_used']):.1f}")
    return out, used, r


# ---------------------------------------------------------------- named workloads (oracle-sized)

def test_config1_art_and_full():
    c = A.config(1)
    _run_and_check(c, "config1 art")
    _run_and_check(c, "config1 full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("mode", ["sqrt_d", "literal"])
def test_config2(mode):
    c = A.config(2, sink_mode=mode)
    _run_and_check(c, f"config2 {mode} art")
    _run_and_check(c, f"config2 {mode} full", eps_scale=0.0, eps_dir=0.0)


def test_config3_small():
    c = A.config(3, small=True)
    _run_and_check(c, "config3-small art")
    _run_and_check(c, "config3-small full", eps_scale=0.0, eps_dir=0.0)


def test_config4_small():
    c = A.config(4, small=True)
    _run_and_check(c, "config4-small art")
    _run_and_check(c, "config4-small full", eps_scale=0.0, eps_dir=0.0)


def test_config5_small():
    c = A.config(5, small=True)
    _run_and_check(c, "config5-small art+vskip")
    _run_and_check(c, "config5-small full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)
    _run_and_check(c, "config5-small full+vskip", eps_scale=0.0, eps_dir=0.0)


# ---------------------------------------------------------------- shapes, tiles, edge cases

@pytest.mark.parametrize("tile", [16, 32, 128])
def test_tiles(tile):
    c = A.config(3, small=True, batch=2, ctx=1000, tile=tile)
    _run_and_check(c, f"tile {tile} art")
    _run_and_check(c, f"tile {tile} full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("patience", [2, 4])
def test_patience(patience):
    c = A.config(3, small=True, patience=patience)
    _run_and_check(c, f"patience {patience}")


def test_ragged_and_empty_rows():
    c = A.make_case("ragged", B=6, Hq=8, Hkv=2, d=128, ctx_lens=[1000, 1, 0, 63, 64, 65],
                    block_size=16, q_mode="temperature", seed=3)
    out, used, _ = _run_and_check(c, "ragged art")
    assert (used[2] == 0).all() and (out[2] == 0).all()
    assert (used[1] == 1).all()
    _run_and_check(c, "ragged full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("G", [1, 5, 16])
def test_group_sizes(G):
    c = A.make_case(f"G{G}", B=2, Hq=2 * G, Hkv=2, d=128, ctx_lens=[700, 513], block_size=16,
                    q_mode="temperature", seed=G)
    _run_and_check(c, f"G={G} art")
    _run_and_check(c, f"G={G} full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("i8", "bf16")])
def test_head_dim_64(kv, q):
    c = A.make_case("d64", B=2, Hq=4, Hkv=2, d=64, ctx_lens=[600, 333], kv_dtype=kv, q_dtype=q,
                    seed=5, v_skip_eps=1e-6 if kv == "i8" else 0.0)
    _run_and_check(c, f"d64 {kv}/{q} art")
    _run_and_check(c, f"d64 {kv}/{q} full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


def test_fp32_query_bf16_cache_paged():
    c = A.make_case("q32", B=2, Hq=8, Hkv=2, d=128, ctx_lens=[900, 400], q_dtype="f32",
                    block_size=32, seed=8)
    _run_and_check(c, "q fp32, kv bf16, bs 32")


def test_drift_values_stop_early():
    c = A.config(3, small=True, v_mean=3.0)
    _, used, _ = _run_and_check(c, "drift art")
    assert used.max() < 32  # values with a common mean converge quickly


# ---------------------------------------------------------------- invariants

def test_paged_and_contiguous_bit_identical():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 8, 128)) * 2
    K = rng.standard_normal((2, 2, 1024, 128))
    V = rng.standard_normal((2, 2, 1024, 128))
    c = contiguous_case(q, K, V, [1024, 777], kv="bf16", qd="bf16")
    p = to_paged(c, 16, seed=4, extra_blocks=7)
    for kw in (dict(), dict(eps_scale=0.0, eps_dir=0.0)):
        o1, u1 = run_gpu(c, **kw)
        o2, u2 = run_gpu(p, **kw)
        assert np.array_equal(u1, u2) and np.array_equal(o1, o2)
    check_parity(c, o1, u1, eps_scale=0.0, eps_dir=0.0)


def test_deterministic_repeats():
    c = A.config(3, small=True)
    dev = to_device(c)
    for kw in (dict(), dict(eps_scale=0.0, eps_dir=0.0)):
        o0, u0 = run_gpu(c, dev, **kw)
        for _ in range(10):
            o, u = run_gpu(c, dev, **kw)
            assert np.array_equal(u, u0) and np.array_equal(o, o0)


def test_worker_count_does_not_change_results():
    # a worker count selects the work-sharing engine (decider waves + tile
    # workers); its results must not depend on how many workers there are
    c = A.config(3, small=True)
    dev = to_device(c)
    o0, u0 = run_gpu(c, dev, max_workers=64)
    for w in (1, 3, 17, 300):
        o, u = run_gpu(c, dev, max_workers=w)
        assert np.array_equal(u, u0) and np.array_equal(o, o0)


@pytest.mark.parametrize("helpers", [1, 3])
def test_helper_work_groups_do_not_change_results(helpers):
    # helper work-groups on other CUs take some of each group's tiles; the
    # stop decisions come from per-tile records scanned in fixed blocks, so
    # tiles_used is the one without helpers exactly, and the output differs
    # only by the order in which the workers' partial sums are merged.  A
    # launch shape is deterministic: a repeat gives the same bits.
    c = A.config(3, small=True)
    dev = to_device(c)
    o_art, u_art = run_gpu(c, dev)
    for kw in (dict(), dict(eps_scale=1e-30, eps_dir=1e-30)):
        o0, u0 = run_gpu(c, dev, **kw)
        o1, u1 = run_gpu(c, dev, team_helpers=helpers, **kw)
        o1b, u1b = run_gpu(c, dev, team_helpers=helpers, **kw)
        assert np.array_equal(u1, u0)
        assert np.array_equal(u1b, u1) and np.array_equal(o1b, o1)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-5)
    o0, u0 = o_art, u_art
    # and with more groups than the chip can give further CUs: the helpers are dropped
    import dataclasses
    pad = 18
    c2 = dataclasses.replace(
        c, B=c.B + pad,
        q=np.concatenate([c.q, np.zeros((pad,) + c.q.shape[1:], c.q.dtype)]),
        block_table=np.concatenate([c.block_table, np.zeros((pad, c.block_table.shape[1]), c.block_table.dtype)]),
        ctx_lens=np.concatenate([c.ctx_lens, np.zeros(pad, c.ctx_lens.dtype)]))
    o2, u2 = run_gpu(c2, team_helpers=helpers)
    assert np.array_equal(u2[:c.B], u0) and np.array_equal(o2[:c.B], o0)
    assert (u2[c.B:] == 0).all() and (o2[c.B:] == 0).all()


@pytest.mark.parametrize("helpers", [1, 3])
def test_helpers_join_long_groups(helpers):
    # helpers take tiles only from tile 96 on: contexts of 256 tiles, thresholds
    # that never pass (every tile used) and the configuration's own thresholds;
    # tiles_used as without helpers, outputs to rounding, and against the oracle
    c = A.config(3, small=True, ctx=16384)
    dev = to_device(c)
    for kw in (dict(eps_scale=1e-30, eps_dir=1e-30), dict()):
        o0, u0 = run_gpu(c, dev, **kw)
        o1, u1 = run_gpu(c, dev, team_helpers=helpers, **kw)
        assert np.array_equal(u1, u0)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-5)
        r = check_parity(c, o1, u1, **kw)
        log(f"[parity] config3 ctx16384 helpers={helpers} {kw}: max_abs={r['max_abs']:.3e} "
            f"mean tiles_used={np.mean(r['tiles_used']):.1f}")


def test_helper_work_groups_parity():
    c = A.config(2, sink_mode="sqrt_d")
    _run_and_check(c, "config2 art, 3 helper work-groups per group", team_helpers=3)
    c = A.config(4, small=True)
    _run_and_check(c, "config4-small art, 1 helper work-group per group", team_helpers=1)


ENGINE_TEAM, ENGINE_POOL, ENGINE_XCD, ENGINE_PAIR, ENGINE_ROUND = 1, 2, 4, 5, 6


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_pool_engine_parity(n):
    # waves on every CU serve whichever groups have tiles left
    c = A.config(n, small=n != 2)
    _run_and_check(c, f"config{n} pool art", engine=ENGINE_POOL, v_skip_eps=0.0)


def test_pool_engine_matches_team_engine():
    # the same probe records and block scan decide: tiles_used is identical,
    # and the outputs differ only by the order of the partial-sum merges
    c = A.config(3, small=True)
    dev = to_device(c)
    for kw in (dict(), dict(eps_scale=1e-30, eps_dir=1e-30), dict(patience=3)):
        o1, u1 = run_gpu(c, dev, engine=ENGINE_TEAM, **kw)
        o2, u2 = run_gpu(c, dev, engine=ENGINE_POOL, **kw)
        assert np.array_equal(u1, u2)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_xcd_engine_parity(n):
    # every group served by the waves of one XCD, deciders on CUs that load no tiles
    c = A.config(n, small=n != 2)
    _run_and_check(c, f"config{n} xcd art", engine=ENGINE_XCD, v_skip_eps=0.0)


@pytest.mark.parametrize("kw", [dict(), dict(workers_per_cu=1), dict(window=1), dict(window=4),
                                dict(workers_per_cu=2, window=2)])
def test_xcd_engine_knobs(kw):
    # the load window (even a single tile past the decided frontier) and the
    # workers per CU change only the schedule: tiles_used equals the oracle's
    c = A.config(4, small=True)
    _run_and_check(c, f"config4-small xcd art {kw}", engine=ENGINE_XCD, **kw)


def test_xcd_engine_matches_team_engine():
    c = A.config(3, small=True)
    dev = to_device(c)
    for kw in (dict(), dict(eps_scale=1e-30, eps_dir=1e-30), dict(patience=3)):
        o1, u1 = run_gpu(c, dev, engine=ENGINE_TEAM, **kw)
        o2, u2 = run_gpu(c, dev, engine=ENGINE_XCD, **kw)
        assert np.array_equal(u1, u2)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5)


def test_xcd_engine_ragged_empty_and_invalid_rows():
    c = A.config(3, small=True, batch=5)
    c.ctx_lens[1] = 0                                   # empty row
    c.ctx_lens[2] = 1                                   # one token
    c.ctx_lens[3] = 64 * 3 + 17                         # ragged tail
    c.ctx_lens[4] = c.block_table.shape[1] * 16 + 1     # longer than its table
    out, used = run_gpu(c, engine=ENGINE_XCD)
    assert (used[1] == 0).all() and (out[1] == 0).all()
    assert (used[4] == -1).all() and np.isnan(out[4]).all()
    check_parity(c, out, used, rows=[0, 1, 2, 3])


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_pair_engine_parity(n):
    # K and scores on one CU of an XCD, V, folding and decisions on another
    c = A.config(n, small=n != 2)
    _run_and_check(c, f"config{n} pair art", engine=ENGINE_PAIR, v_skip_eps=0.0)


@pytest.mark.parametrize("kv", ["bf16", "i8", "i4"])
def test_pair_engine_matches_team_engine(kv):
    # the same scores (same operands, same instruction) and the same fold:
    # identical stops, outputs equal to rounding
    c = A.config(3, small=True, kv_dtype=kv)
    dev = to_device(c)
    for kw in (dict(), dict(eps_scale=1e-30, eps_dir=1e-30), dict(patience=3)):
        o1, u1 = run_gpu(c, dev, engine=ENGINE_TEAM, **kw)
        o2, u2 = run_gpu(c, dev, engine=ENGINE_PAIR, **kw)
        assert np.array_equal(u1, u2), kw
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-6)


def test_pair_engine_ragged_empty_and_invalid_rows():
    c = A.config(3, small=True, batch=8)
    c.ctx_lens[1] = 0                                   # empty row
    c.ctx_lens[2] = 1                                   # one token
    c.ctx_lens[3] = 64 * 3 + 17                         # ragged tail
    c.ctx_lens[4] = c.block_table.shape[1] * 16 + 1     # longer than its table
    c.block_table[5, 7] = -3                            # an invalid block id inside the row
    out, used = run_gpu(c, engine=ENGINE_PAIR)
    assert (used[1] == 0).all() and (out[1] == 0).all()
    assert (used[4] == -1).all() and np.isnan(out[4]).all()
    check_parity(c, out, used, rows=[0, 1, 2, 3, 6, 7])
    assert (used[5] == -1).all() or (used[5] > 0).all()  # stops before the bad block, else reports it


def test_pair_engine_full_size():
    # the 32K workload at full size (128 groups on 256 CUs), every row
    c = A.config(3)
    out, used = run_gpu(c, engine=ENGINE_PAIR)
    r = check_parity(c, out, used)
    log(f"[parity] config3 full size pair: max_abs={r['max_abs']:.3e} near={r['near']}")


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_round_engine_parity(n):
    # the steps in rounds over every CU; the last wave of a group decides them
    c = A.config(n, small=n != 2)
    _run_and_check(c, f"config{n} round art", engine=ENGINE_ROUND, v_skip_eps=0.0)


@pytest.mark.parametrize("kv", ["bf16", "i8", "i4"])
def test_round_engine_matches_team_engine(kv):
    # the same tile partials and the same block scan: identical stops; the
    # outputs merge the same partials in another order (rounding only)
    # 128 groups of 128 steps: two rounds, steps [0, 64) and [64, 128)
    c = A.config(3, small=True, batch=16, ctx=8192, kv_dtype=kv)
    dev = to_device(c)
    for kw in (dict(), dict(eps_scale=1e-30, eps_dir=1e-30), dict(patience=3), dict(eps_scale=1e-2, eps_dir=1e-3)):
        o1, u1 = run_gpu(c, dev, engine=ENGINE_TEAM, **kw)
        o2, u2 = run_gpu(c, dev, engine=ENGINE_ROUND, **kw)
        assert np.array_equal(u1, u2), kw
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5)


def test_round_engine_ragged_empty_and_invalid_rows():
    c = A.config(3, small=True, batch=8, ctx=8192)
    c.ctx_lens[1] = 0                                   # empty row
    c.ctx_lens[2] = 1                                   # one token
    c.ctx_lens[3] = 64 * 3 + 17                         # ragged tail
    c.ctx_lens[4] = c.block_table.shape[1] * 16 + 1     # longer than its table
    c.block_table[5, 7] = -3                            # an invalid block id inside the row
    c.ctx_lens[6] = 64 * 100 + 5                        # a ragged tail in the second round (steps 96..127)
    out, used = run_gpu(c, engine=ENGINE_ROUND)
    assert (used[1] == 0).all() and (out[1] == 0).all()
    assert (used[4] == -1).all() and np.isnan(out[4]).all()
    check_parity(c, out, used, rows=[0, 1, 2, 3, 6, 7])
    assert (used[5] == -1).all() or (used[5] > 0).all()  # stops before the bad block, else reports it


def _round_bounds(nt_max, ng):
    # the rounds' first steps as the library plans them: about 3 steps per wave
    # of 2048 in the first rounds (64 to 256 steps), then as many steps as
    # came before, at most 512
    first = min(max((3 * 2048 // ng + 15) // 16 * 16, 64), 256)
    a = [0]
    while a[-1] < nt_max:
        c = min(max((a[-1] + 15) // 16 * 16, first), 512)
        a.append(min(a[-1] + c, nt_max))
    return a


def test_round_engine_repeated_calls_and_statistics():
    # successive calls (each with its own epoch) give the same result; the
    # tiles loaded are at least those the stops need and at most what the
    # rounds that hold each group's stop cover
    import torch
    c = A.config(3, small=True, ctx=8192)
    dev = to_device(c)
    first = None
    for _ in range(3):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        out, used = run_gpu(c, dev, engine=ENGINE_ROUND, stats=stats)
        if first is None:
            first = (out, used)
            check_parity(c, out, used)
        else:
            assert np.array_equal(used, first[1])
            assert np.array_equal(out, first[0])  # deterministic
        per_group = used.reshape(c.B, c.Hkv, -1).max(axis=2)
        nt = -(-c.ctx_lens // c.tile)
        bounds = _round_bounds(int(nt.max()), c.B * c.Hkv)
        cover = np.array([[min(next(b for b in bounds if b >= u), nt[i]) for u in row]
                          for i, row in enumerate(per_group)])
        loaded = int(stats[0].item())
        assert per_group.sum() <= loaded <= cover.sum(), (per_group.sum(), loaded, cover.sum())


@pytest.mark.parametrize("n", [3, 4, 5])
def test_round_engine_full_size(n):
    # every row of the full-size workload against the oracle
    c = A.config(n)
    out, used = run_gpu(c, engine=ENGINE_ROUND, v_skip_eps=0.0)
    r = check_parity(c, out, used, v_skip_eps=0.0)
    log(f"[parity] config{n} full size round: max_abs={r['max_abs']:.3e} near={r['near']}")


def test_pool_engine_ragged_empty_and_invalid_rows():
    c = A.config(3, small=True, batch=5)
    c.ctx_lens[1] = 0                                   # empty row
    c.ctx_lens[2] = 1                                   # one token
    c.ctx_lens[3] = 64 * 3 + 17                         # ragged tail
    c.ctx_lens[4] = c.block_table.shape[1] * 16 + 1     # longer than its table
    out, used = run_gpu(c, engine=ENGINE_POOL)
    assert (used[1] == 0).all() and (out[1] == 0).all()
    assert (used[4] == -1).all() and np.isnan(out[4]).all()
    check_parity(c, out, used, rows=[0, 1, 2, 3])


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_work_sharing_engine(n):
    # the engine used for few groups, forced here on the named workloads
    c = A.config(n, small=n != 2)
    _run_and_check(c, f"config{n} work-sharing art", max_workers=96)


def test_invalid_block_and_length_reported_per_row():
    c = A.config(3, small=True, batch=3)
    c.block_table[1, 5] = c.num_blocks + 3          # row 1: bad block inside tile 1
    c.ctx_lens[2] = c.block_table.shape[1] * 16 + 1  # row 2: longer than its table
    out, used = run_gpu(c, eps_scale=0.0, eps_dir=0.0)
    assert (used[1] == -1).all() and np.isnan(out[1]).all()
    assert (used[2] == -1).all() and np.isnan(out[2]).all()
    c.block_table[1, 5] = 0  # the oracle rejects bad ids outright: check row 0 alone
    check_parity(c, out, used, eps_scale=0.0, eps_dir=0.0, rows=[0])
    c.block_table[1, 5] = c.num_blocks + 3
    out, used = run_gpu(c)
    # ART mode: a head of row 1 that stops before tile 1 never reads the bad block
    assert (used[2] == -1).all()
    assert ((used[1] == -1) | (used[1] == 1)).all()
    assert np.isfinite(out[0]).all() and (used[0] > 0).all()


# ---------------------------------------------------------------- full-size workloads (every row)

@pytest.mark.parametrize("mode", ["art", "full"])
@pytest.mark.parametrize("n", [3, 4, 5])
def test_full_size_every_row(n, mode):
    # the headline sizes in the launch configuration bench.py times (library
    # defaults), every row against the oracle
    log(f"[parity] generating config {n} at full size ({mode})")
    c = A.config(n)
    dev = to_device(c)
    kw = dict() if mode == "art" else dict(eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)
    out, used = run_gpu(c, dev, **kw)
    r = check_parity(c, out, used, **kw)
    log(f"[parity] config{n} full size {mode}: max_abs={r['max_abs']:.3e} near={r['near']} "
        f"mean tiles_used={np.mean(r['tiles_used']):.1f}")
    assert (used <= -(-c.ctx_lens[:, None] // c.tile)).all() and (used >= 1).all()


# ---------------------------------------------------------------- zero probe and fp16 subnormal scales

@pytest.mark.parametrize("shape", ["fp32 d64 T16", "bf16 d128 T64"])
@pytest.mark.parametrize("engine", [0, ENGINE_TEAM, ENGINE_POOL, ENGINE_XCD, ENGINE_PAIR, ENGINE_ROUND])
def test_zero_norm_probe_in_art_mode(shape, engine):
    # the designed case of the oracle pin (probe exactly 0 through tile k - 1,
    # thresholds no finite metric reaches): a metric against a zero probe is
    # +inf on the GPU too, so every head stops at tile k + 1 + patience.
    # fp32 runs the one-tile-at-a-time kernels, bf16 the streamed tile.
    from tests.test_oracle import zero_probe_case
    fp32 = shape.startswith("fp32")
    for k, patience in ((3, 1), (2, 2)):
        c = zero_probe_case(k, patience, nt=12, T=16 if fp32 else 64, d=64 if fp32 else 128)
        if not fp32:
            c = contiguous_case(c.q, c.k, c.v, tile=c.tile, eps_scale=c.eps_scale, eps_dir=c.eps_dir,
                                patience=patience, kv="bf16", qd="bf16")
        out, used, _ = _run_and_check(c, f"zero probe k={k} p={patience} {shape} engine {engine}",
                                      engine=engine)
        assert (used == k + 1 + patience).all(), used


@pytest.mark.parametrize("engine", [0, ENGINE_TEAM, ENGINE_POOL, ENGINE_XCD, ENGINE_PAIR, ENGINE_ROUND])
def test_int8_subnormal_scales(engine):
    # fp16 scales below 2^-14 (subnormal) widen exactly on both sides
    c = A.config(5, small=True, seed=6)
    rng = np.random.default_rng(6)
    c.k_scale = rng.integers(0x200, 0x400, size=c.k_scale.shape).astype(np.uint16)
    c.v_scale = rng.integers(1, 0x400, size=c.v_scale.shape).astype(np.uint16)
    # scores this small give near-uniform weights: thresholds that stop
    c.eps_scale, c.eps_dir = 1e-2, 1e-3
    _run_and_check(c, f"config5-small subnormal scales art engine {engine}", engine=engine, v_skip_eps=0.0)
    _run_and_check(c, "config5-small subnormal scales full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


# ---------------------------------------------------------------- V skip on bf16 caches

@pytest.mark.parametrize("n", [3, 4])
def test_vskip_bf16_cache(n):
    # the V-skip predicate does not depend on the cache format: bf16 caches
    # take the same skip path as int8 ones (team kernel, work-sharing engine,
    # one-tile-at-a-time kernel for fp32 queries)
    import torch
    c = A.config(n, small=True, v_skip_eps=1e-4)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    _run_and_check(c, f"config{n} bf16 art+vskip", stats=stats)
    assert int(stats[3].item()) > 0  # some (head, row) pairs were skipped
    _run_and_check(c, f"config{n} bf16 full+vskip", eps_scale=0.0, eps_dir=0.0)
    _run_and_check(c, f"config{n} bf16 art+vskip work-sharing", max_workers=96)
    _run_and_check(c, f"config{n} bf16 art+vskip patience 3", patience=3)


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("i8", "bf16"), ("i4", "bf16"), ("bf16", "f32")])
def test_vskip_predicate_limits(kv, q):
    # exp(s - M) >= eps at its limits, on the streamed tile (bf16/int8/int4
    # caches), the work-sharing engine and the one-tile-at-a-time kernel (fp32
    # queries): eps > 1 leaves every V row out (out = 0, every weight still in
    # l); eps = 1 keeps only the rows that reach the running max; a tiny eps
    # keeps every row
    c = A.make_case("vskip limits", B=3, Hq=8, Hkv=2, d=128, ctx_lens=[1500, 700, 333], kv_dtype=kv,
                    q_dtype=q, block_size=16, q_mode="temperature", seed=31)
    full = dict(eps_scale=0.0, eps_dir=0.0)
    for kw in (dict(), dict(max_workers=96)):
        out, _, _ = _run_and_check(c, f"{kv}/{q} eps_v 1.0001 {kw}", v_skip_eps=1.0001, **full, **kw)
        assert (out == 0).all()
        # in ART mode too: every V row left out makes every probe 0, and a
        # zero probe never passes (reading 14): no head stops
        out, used, _ = _run_and_check(c, f"{kv}/{q} eps_v 1.0001 art {kw}", v_skip_eps=1.0001,
                                      eps_scale=1e30, eps_dir=1e30, **kw)
        assert (out == 0).all()
        assert (used == -(-c.ctx_lens[:, None] // c.tile)).all()
        _run_and_check(c, f"{kv}/{q} eps_v 1 {kw}", v_skip_eps=1.0, **full, **kw)
        _run_and_check(c, f"{kv}/{q} eps_v 1e-30 art {kw}", v_skip_eps=1e-30, **kw)
        _run_and_check(c, f"{kv}/{q} eps_v 1e-30 full {kw}", v_skip_eps=1e-30, **full, **kw)


def _host_skipped_pairs(c, eps):
    """(head, row) pairs with s - M_t < ln eps over every tile, ascending order,
    M_t the running max through tile t (float64), and how many of them lie
    within 1e-3 of the threshold (their decision may go either way in fp32)."""
    from tests import bruteforce as BF
    G = c.Hq // c.Hkv
    ln = np.log(eps)
    count = near = 0
    for b in range(c.B):
        n = int(c.ctx_lens[b])
        for h in range(c.Hq):
            K = BF.logical_rows(c, "k", b, h // G, n)
            sc = K @ BF.query(c, b, h) / np.sqrt(c.d)
            for t0 in range(0, n, c.tile):
                M = sc[:t0 + c.tile].max()
                x = sc[t0:t0 + c.tile] - M - ln
                count += int((x < 0).sum())
                near += int((np.abs(x) < 1e-3).sum())
    return count, near


def _host_vskip_rows(c, eps):
    """V rows some query head of their KV head keeps (s - M_t >= ln eps for
    at least one head, ascending order, float64), the rows whose keep
    decision lies within 1e-3 of the threshold, and all rows."""
    from tests import bruteforce as BF
    G = c.Hq // c.Hkv
    ln = np.log(eps)
    kept = near = total = 0
    for b in range(c.B):
        n = int(c.ctx_lens[b])
        for g in range(c.Hkv):
            K = BF.logical_rows(c, "k", b, g, n)
            best = np.full(n, -np.inf)
            for h in range(g * G, (g + 1) * G):
                sc = K @ BF.query(c, b, h) / np.sqrt(c.d)
                M = np.maximum.accumulate(np.array([sc[:t0 + c.tile].max() for t0 in range(0, n, c.tile)]))
                x = sc - np.repeat(M, c.tile)[:n] - ln
                best = np.maximum(best, x)
            kept += int((best >= 0).sum())
            near += int((np.abs(best) < 1e-3).sum())
            total += n
    return kept, near, total


@pytest.mark.parametrize("n", [3, 5])
def test_vskip_pair_count(n):
    # stats[3], the (head, row) pairs left out of P.V (counted by the default
    # engine): exact in full mode, where every tile is consumed once; stats[1],
    # the V rows loaded: on a bf16 cache only those some head of the group
    # keeps, so at eps_v = 1e-4 below the rows of the tiles read; on an int8
    # cache every row (the skip leaves out their arithmetic only)
    import torch
    c = A.config(n, small=True, v_skip_eps=1e-4)
    want, near = _host_skipped_pairs(c, 1e-4)
    assert want > 0
    rows_kept, rows_near, rows_all = _host_vskip_rows(c, 1e-4)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    _run_and_check(c, f"config{n} full+vskip count", eps_scale=0.0, eps_dir=0.0, stats=stats)
    got = int(stats[3].item())
    log(f"[parity] config{n} skipped pairs: gpu {got} host {want} (near threshold {near})")
    assert abs(got - want) <= near, (got, want, near)
    got_rows = int(stats[1].item())
    log(f"[parity] config{n} V rows loaded: gpu {got_rows} host {rows_kept} of {rows_all} (near {rows_near})")
    if c.kv_dtype == "bf16":
        assert abs(got_rows - rows_kept) <= rows_near, (got_rows, rows_kept, rows_near)
        assert got_rows < rows_all
    else:
        assert got_rows == rows_all, (got_rows, rows_all)


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("i8", "bf16"), ("i4", "bf16"), ("f32", "f32")])
def test_load_statistics(kv, q):
    # stats[0] K tiles loaded, stats[1] V rows loaded: in full mode every tile
    # of every (row, KV head) is loaded once; stats[2] is left unchanged
    import torch
    c = A.make_case("load stats", B=3, Hq=8, Hkv=2, d=128, ctx_lens=[1500, 700, 333], kv_dtype=kv,
                    q_dtype=q, block_size=16, q_mode="temperature", seed=37)
    all_tiles = c.Hkv * int((-(-c.ctx_lens // c.tile)).sum())
    all_rows = c.Hkv * int(c.ctx_lens.sum())
    for kw in (dict(), dict(max_workers=96)):
        stats = torch.full((4,), 0, dtype=torch.int64, device="cuda")
        stats[2] = 7
        run_gpu(c, eps_scale=0.0, eps_dir=0.0, stats=stats, **kw)
        st = stats.cpu().numpy()
        assert st[0] == all_tiles and st[1] == all_rows and st[2] == 7 and st[3] == 0, (kw, st)


@pytest.mark.parametrize("n", [2, 3])
def test_load_statistics_art(n):
    # ART mode: at least the tiles the stop rule needs (the max of tiles_used
    # over a group's heads), at most every tile; V rows within the same bounds
    # (workloads whose heads stop early, at full size)
    import torch
    c = A.config(n)
    G = c.Hq // c.Hkv
    nt = -(-c.ctx_lens // c.tile)
    all_tiles = c.Hkv * int(nt.sum())
    for kw in (dict(), dict(engine=2), dict(max_workers=96)):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        _, used = run_gpu(c, stats=stats, **kw)
        st = stats.cpu().numpy()
        used_g = used.reshape(c.B, c.Hkv, G).max(axis=-1)
        needed = int(used_g.sum())
        rows_needed = int(np.minimum(used_g * c.tile, c.ctx_lens[:, None]).sum())
        log(f"[stats] config{n} ART {kw}: loaded {st[0]} needed {needed} of {all_tiles}, rows {st[1]}")
        assert needed < all_tiles  # the heads stop early here
        assert needed <= st[0] <= all_tiles and rows_needed <= st[1] <= c.Hkv * int(c.ctx_lens.sum()), (kw, st)
        assert st[2] == 0 and st[3] == 0


# ---------------------------------------------------------------- int4 caches

@pytest.mark.parametrize("d,paged", [(128, True), (64, True), (128, False)])
def test_int4_cache(d, paged):
    # int4 codes two per byte with fp16 scales: the one-tile-at-a-time kernels
    c = A.make_case("i4", B=3, Hq=8, Hkv=2, d=d, ctx_lens=[1500, 700, 0], kv_dtype="i4",
                    block_size=16 if paged else 0, q_mode="temperature", seed=31)
    _run_and_check(c, f"int4 d{d} paged={paged} art")
    _run_and_check(c, f"int4 d{d} paged={paged} art+vskip", v_skip_eps=1e-4)
    _run_and_check(c, f"int4 d{d} paged={paged} full", eps_scale=0.0, eps_dir=0.0)
    _run_and_check(c, f"int4 d{d} paged={paged} full+vskip", eps_scale=0.0, eps_dir=0.0, v_skip_eps=1e-4)


def test_int4_config5_small():
    # the streamed 64-token tile (codes widened to bf16 for the matrix cores)
    c = A.config(5, small=True, kv_dtype="i4")
    _run_and_check(c, "config5-small int4 art+vskip")
    _run_and_check(c, "config5-small int4 art", v_skip_eps=0.0)
    _run_and_check(c, "config5-small int4 art pool", engine=ENGINE_POOL, v_skip_eps=0.0)
    _run_and_check(c, "config5-small int4 art work-sharing", max_workers=96, v_skip_eps=0.0)
    _run_and_check(c, "config5-small int4 full", eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)


@pytest.mark.parametrize("G", [1, 5, 8])
def test_int4_group_sizes(G):
    c = A.make_case(f"i4-G{G}", B=2, Hq=2 * G, Hkv=2, d=128, ctx_lens=[1700, 513], kv_dtype="i4",
                    block_size=16, q_mode="temperature", seed=40 + G)
    _run_and_check(c, f"int4 G={G} art")
    _run_and_check(c, f"int4 G={G} art+vskip", v_skip_eps=1e-4)
    _run_and_check(c, f"int4 G={G} full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("variant", ["recent_first", "random_list", "retained", "int4"])
def test_full_size_sampled_rows_variants(variant):
    # the 32K workload at full size with a tile order, per-head retained tables
    # or (workload 5) an int4 cache, in the launch configuration bench.py times;
    # the oracle checks the first and last rows
    log(f"[parity] generating full-size case for {variant}")
    if variant == "int4":
        c = A.config(5, kv_dtype="i4")
    else:
        c = A.config(3)
        if variant == "recent_first":
            c.order = 1
        elif variant == "random_list":
            c.order = 2
            c.tile_perm = A.sink_first_orders(c.ctx_lens, c.tile, stride=-(-c.max_ctx // c.tile), seed=1)
        else:
            c = A.retained_tables(c, sink_blocks=4, recent_blocks=512, keep_frac=0.25, seed=1)
    dev = to_device(c)
    rows = [0, c.B - 1]
    out, used = run_gpu(c, dev)
    r = check_parity(c, out, used, rows=rows)
    log(f"[parity] {variant} full size: max_abs={r['max_abs']:.3e} near={r['near']} "
        f"mean tiles_used (sampled)={np.mean(r['tiles_used']):.1f}")
    assert (used >= 1).all()


# ---------------------------------------------------------------- query-head split (G = 6, 8, 12, 16)

@pytest.mark.parametrize("G", [5, 6, 7, 8, 10, 12, 13, 16])
def test_query_head_split(G):
    # in ART mode a KV head's G query heads run as groups of at most 4 heads
    # on the 4-head tile (the last group smaller when G does not divide);
    # per-head results must not change
    c = A.make_case(f"split-G{G}", B=3, Hq=2 * G, Hkv=2, d=128, ctx_lens=[1700, 513, 0], block_size=16,
                    q_mode="temperature", seed=50 + G)
    _run_and_check(c, f"G={G} art")
    _run_and_check(c, f"G={G} art pool", engine=ENGINE_POOL)
    _run_and_check(c, f"G={G} art work-sharing", max_workers=64)
    _run_and_check(c, f"G={G} art+vskip", v_skip_eps=1e-4)
    _run_and_check(c, f"G={G} full", eps_scale=0.0, eps_dir=0.0)


@pytest.mark.parametrize("kv", ["i8", "i4"])
def test_query_head_split_quantised_contiguous(kv):
    c = A.make_case(f"split-{kv}", B=2, Hq=16, Hkv=2, d=128, ctx_lens=[2000, 777], kv_dtype=kv,
                    block_size=0, q_mode="temperature", seed=61)
    _run_and_check(c, f"G=8 {kv} contiguous art")
    c.order, c.tile_perm = 1, None
    _run_and_check(c, f"G=8 {kv} contiguous art recent-first")


def test_query_head_split_uneven_edge_rows():
    # G = 5 (groups of 3 and 2): empty, one-token and invalid rows write only
    # their own heads
    c = A.make_case("split-edge", B=4, Hq=10, Hkv=2, d=128, ctx_lens=[900, 0, 1, 333], block_size=16,
                    q_mode="temperature", seed=63)
    c.ctx_lens[3] = c.block_table.shape[1] * 16 + 1   # longer than its table
    out, used = run_gpu(c)
    assert (used[1] == 0).all() and (out[1] == 0).all()
    assert (used[3] == -1).all() and np.isnan(out[3]).all()
    check_parity(c, out, used, rows=[0, 1, 2])
    out, used = run_gpu(c, engine=ENGINE_POOL)
    assert (used[3] == -1).all() and np.isnan(out[3]).all()
    check_parity(c, out, used, rows=[0, 1, 2])


def test_query_head_split_per_head_tables_and_lists():
    c = A.make_case("split-ph", B=2, Hq=16, Hkv=2, d=128, ctx_lens=[3000, 1500], block_size=16,
                    q_mode="temperature", seed=62)
    c = A.retained_tables(c, sink_blocks=2, recent_blocks=64, keep_frac=0.5, seed=4)
    c.order = 2
    c.tile_perm = A.sink_first_orders(c.ctx_lens, c.tile, stride=-(-c.max_ctx // c.tile), seed=5)
    _run_and_check(c, "G=8 per-head tables, caller's list, art")
    _run_and_check(c, "G=8 per-head tables, caller's list, pool", engine=ENGINE_POOL)
