"""Seeded combinations of the library's options against the fp64 oracle:
cache dtype, head dim, query heads per KV head (with the query-head split),
tile size, tile order, per-head tables, V skip, patience and engine.  Each
case is drawn from its own seed, so a failure names a reproducible case."""
import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import log
from tests.test_parity_gpu import _run_and_check

pytestmark = pytest.mark.gpu

N_CASES = 96


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    kv = str(rng.choice(["bf16", "bf16", "i8", "i4", "f32"]))
    d = int(rng.choice([128, 128, 64]))
    G = int(rng.choice([1, 2, 4, 5, 6, 8, 12]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.integers(1, 4))
    tile = int(rng.choice([64, 64, 32, 16, 128]))
    ctx = [int(x) for x in rng.integers(0, 2500, size=B)]
    ctx[0] = max(ctx[0], 300)
    c = A.make_case(f"combo{seed}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, ctx_lens=ctx, kv_dtype=kv,
                    q_dtype="f32" if kv == "f32" else "bf16", block_size=int(rng.choice([16, 32, 0])),
                    q_mode="temperature", seed=seed, tile=tile, patience=int(rng.choice([1, 1, 2])),
                    v_skip_eps=float(rng.choice([0.0, 0.0, 1e-4])))
    if c.block_size and rng.random() < 0.4:
        c = A.retained_tables(c, sink_blocks=1, recent_blocks=int(rng.integers(4, 40)),
                              keep_frac=float(rng.random()), seed=seed)
    c.order = int(rng.choice([0, 1, 2]))
    if c.order == 2:
        c.tile_perm = A.sink_first_orders(c.ctx_lens, c.tile, stride=-(-c.max_ctx // c.tile), seed=seed)
    engine = int(rng.choice([0, 0, 1, 2]))
    return c, engine


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_combination(seed):
    c, engine = draw(seed)
    log(f"[combo {seed}] kv={c.kv_dtype} d={c.d} G={c.Hq // c.Hkv} Hkv={c.Hkv} B={c.B} T={c.tile} "
        f"bs={c.block_size} per_head={c.per_head_tables} order={c.order} vskip={c.v_skip_eps} "
        f"patience={c.patience} engine={engine}")
    _run_and_check(c, f"combo {seed} art", engine=engine)
    _run_and_check(c, f"combo {seed} full", eps_scale=0.0, eps_dir=0.0, engine=engine)
