"""Pins of the fp64 oracle against facts that do not come from the oracle.

Every check below ties the oracle to something else: textbook softmax
attention (tests/bruteforce.py), closed forms of hand-designed inputs,
invariants of the method, or designed probe sequences under tests/golden/.
Method passages: gist.science ART summary sections 2.1-2.4; puntofijo.es
article on skipping V dequantisation.
"""
import glob
import json
import os

import numpy as np
import pytest

import art_inputs as A
from tests import bruteforce as BF
from tests.helpers import contiguous_case, designed_case, run_oracle, to_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(B=2, Hq=4, Hkv=2, d=16, n=100, seed=0, kv="f32", qd="f32", **params):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    return contiguous_case(q, K, V, kv=kv, qd=qd, **params)


def ntiles(n, T):
    return -(-n // T)


# ---------------------------------------------------------------- P1: full mode = softmax attention

@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 300])
@pytest.mark.parametrize("d", [4, 8, 64])
@pytest.mark.parametrize("T", [1, 3, 16, 64])
def test_full_mode_equals_bruteforce(n, d, T):
    c = rand_case(B=1, Hq=2, Hkv=1, d=d, n=n, seed=n * 7 + d + T, tile=T, eps_scale=0.0, eps_dir=0.0)
    r = run_oracle(c)
    assert (r.tiles_used == ntiles(n, T)).all()
    for h in range(2):
        ref = BF.attention(c, 0, h, n)
        assert np.allclose(r.out[0, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_full_mode_gqa_ragged_bruteforce(kv):
    c = rand_case(B=3, Hq=6, Hkv=2, d=32, n=200, seed=3, kv=kv, qd=kv, tile=16,
                  eps_scale=0.0, eps_dir=0.0)
    c.ctx_lens[:] = [200, 17, 129]
    r = run_oracle(c)
    for b in range(3):
        n = int(c.ctx_lens[b])
        assert (r.tiles_used[b] == ntiles(n, 16)).all()
        for h in range(6):
            assert np.allclose(r.out[b, h], BF.attention(c, b, h, n), rtol=1e-12, atol=1e-13)


def test_single_tile_is_plain_attention_and_zero_context():
    c = rand_case(B=2, Hq=2, Hkv=1, d=16, n=40, seed=11, tile=64)
    c.ctx_lens[:] = [40, 0]
    r = run_oracle(c)
    assert (r.tiles_used[0] == 1).all()  # one tile: never a comparison
    assert np.allclose(r.out[0, 1], BF.attention(c, 0, 1, 40), rtol=1e-12, atol=1e-13)
    assert (r.tiles_used[1] == 0).all() and (r.out[1] == 0).all()


# ---------------------------------------------------------------- P2: prefix identity

@pytest.mark.parametrize("seed", range(6))
def test_stop_equals_attention_over_used_prefix(seed):
    # loose thresholds so random data stops at various tiles
    c = rand_case(B=2, Hq=4, Hkv=2, d=16, n=400, seed=100 + seed, tile=8,
                  eps_scale=0.05, eps_dir=0.02, patience=1 + seed % 3)
    c.ctx_lens[:] = [400, 397 - 13 * seed]
    r = run_oracle(c)
    stopped = 0
    for b in range(2):
        n = int(c.ctx_lens[b])
        for h in range(4):
            U = int(r.tiles_used[b, h])
            stopped += U < ntiles(n, 8)
            ref = BF.attention(c, b, h, min(U * 8, n))
            assert np.allclose(r.out[b, h], ref, rtol=1e-12, atol=1e-13)
    assert stopped > 0  # the case must exercise termination


# ---------------------------------------------------------------- P3: convexity (weights via one-hot V)

def test_full_mode_weights_are_softmax_and_convex():
    n = d = 48
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, d)) * 2
    K = rng.standard_normal((1, 1, n, d))
    V = np.eye(n)[None, None]  # row j = e_j, so out = the weight vector
    c = contiguous_case(q, K, V, tile=16, eps_scale=0.0, eps_dir=0.0)
    w = run_oracle(c).out[0, 0]
    assert (w >= 0).all() and abs(w.sum() - 1) < 1e-13
    assert np.allclose(w, BF.attention_weights(c, 0, 0, n), rtol=1e-12, atol=1e-15)


def test_outputs_lie_in_value_bounds():
    c = A.config(2, small=True, seed=4)
    r = run_oracle(c)
    G = c.Hq // c.Hkv
    for h in range(c.Hq):
        U = int(r.tiles_used[0, h])
        V = BF.logical_rows(c, "v", 0, h // G, min(U * c.tile, int(c.ctx_lens[0])))
        assert (r.out[0, h] >= V.min(0) - 1e-12).all() and (r.out[0, h] <= V.max(0) + 1e-12).all()


# ---------------------------------------------------------------- P4: bounds on tiles_used

@pytest.mark.parametrize("patience", [1, 2, 4])
def test_tiles_used_bounds(patience):
    c = rand_case(B=3, Hq=4, Hkv=4, d=8, n=300, seed=patience, tile=8,
                  eps_scale=0.2, eps_dir=0.1, patience=patience)
    c.ctx_lens[:] = [300, 9, 1]
    r = run_oracle(c)
    for b in range(3):
        nt = ntiles(int(c.ctx_lens[b]), 8)
        assert (r.tiles_used[b] >= min(patience + 1, nt)).all()
        assert (r.tiles_used[b] <= nt).all()


# ---------------------------------------------------------------- P5: constant V closed form

@pytest.mark.parametrize("patience", [1, 3])
def test_constant_values(patience):
    rng = np.random.default_rng(9)
    d, n = 16, 256
    c_vec = rng.uniform(0.5, 2.0, size=d)
    q = rng.standard_normal((1, 2, d))
    K = rng.standard_normal((1, 1, n, d))
    V = np.broadcast_to(c_vec, (1, 1, n, d))
    c = contiguous_case(q, K, V, tile=16, eps_scale=1e-9, eps_dir=1e-9, patience=patience)
    r = run_oracle(c)
    cv = c.v[0, 0, 0].astype(np.float64)
    assert (r.tiles_used == patience + 1).all()
    assert np.allclose(r.out[0], cv, rtol=1e-14, atol=0)
    full = run_oracle(c, eps_scale=0.0, eps_dir=0.0)
    assert (full.tiles_used == n // 16).all()  # 0 is never strictly below 0


# ---------------------------------------------------------------- reading 14: a zero probe never passes

def zero_probe_case(k, patience, nt=10, T=4, d=16, seed=11):
    """Keys all equal (uniform weights); the V rows of tiles 0..k-1 are zero in
    the probe dims 0..7 and those of later tiles equal a constant c there, so
    the probe is exactly 0 through tile k - 1 and (t - k + 1) / (t + 1) * c
    after.  Dims beyond 8 are random (outside the probe)."""
    rng = np.random.default_rng(seed)
    c_vec = rng.uniform(0.5, 2.0, size=8)
    V = np.zeros((1, 1, nt * T, d))
    V[0, 0, k * T:, :8] = c_vec
    V[0, 0, :, 8:] = rng.uniform(-3, 3, size=(nt * T, d - 8))
    K = np.zeros((1, 1, nt * T, d))
    q = rng.standard_normal((1, 2, d))
    # thresholds no finite metric reaches: every tile passes unless a norm is 0
    return contiguous_case(q, K, V, tile=T, eps_scale=1e30, eps_dir=1e30, patience=patience)


@pytest.mark.parametrize("k,patience", [(0, 1), (1, 1), (3, 1), (3, 2), (6, 3)])
def test_zero_norm_probe_never_passes(k, patience):
    # Closed form: a metric against a probe of norm 0 is +inf (reading 14), so
    # no tile passes while the probe or the previous one is 0: tiles k and
    # later are the first whose probe is nonzero, the first comparison of two
    # nonzero probes is at tile k + 1 (tile 1 when k = 0), and the stop comes
    # `patience` passing tiles later
    c = zero_probe_case(k, patience)
    r = run_oracle(c, trace=True)
    first = max(k + 1, 1)
    assert (r.tiles_used == first + patience).all(), (r.tiles_used, first + patience)
    ds = r.trace[0, 0, 1:first, 2]
    assert np.isinf(ds).all()  # every comparison before: a zero norm on either side


def test_widen_f16_every_pattern():
    # the oracle's fp16 widening (normal, subnormal, zero, inf, nan, both
    # signs) against numpy's IEEE binary16 conversion, for all 65536 patterns
    import oracle
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_int8_with_subnormal_scales_equals_dequantised_fp32():
    # fp16 scales below 2^-14 take the subnormal branch of the widening; the
    # int8 oracle must still equal the fp64 oracle on the dequantised cache
    # (code * scale is exact in fp32: an 8-bit code times a 10-bit fraction)
    c = A.config(5, small=True, seed=3, batch=1, ctx=256)
    rng = np.random.default_rng(4)
    c.k_scale = rng.integers(1, 0x400, size=c.k_scale.shape).astype(np.uint16)
    c.v_scale = rng.integers(1, 0x400, size=c.v_scale.shape).astype(np.uint16)
    deq = lambda codes, sc: (codes.astype(np.float32) * sc.view(np.float16).astype(np.float32)[..., None])
    f = A.Case(name="deq", B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, q=c.q,
               k=deq(c.k, c.k_scale), v=deq(c.v, c.v_scale), ctx_lens=c.ctx_lens,
               block_size=c.block_size, block_table=c.block_table, tile=c.tile)
    for kw in (dict(v_skip_eps=0.0), dict(eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)):
        a = run_oracle(c, **kw)
        b = run_oracle(f, **kw)
        assert np.array_equal(a.out, b.out) and np.array_equal(a.tiles_used, b.tiles_used)


# ---------------------------------------------------------------- P6: designed probe sequences

FIXTURES = sorted(glob.glob(os.path.join(GOLDEN, "*.json")))


@pytest.mark.parametrize("path", FIXTURES, ids=[os.path.basename(p) for p in FIXTURES])
def test_designed_sequences(path):
    fx = json.load(open(path))
    c = designed_case(fx)
    rho = np.asarray(fx["rho"])
    th = np.asarray(fx["theta"])
    exp_scale = np.abs(np.diff(rho)) / rho[:-1]
    exp_dir = 1 - np.cos(np.diff(th))
    for run in fx["runs"]:
        r = run_oracle(c, eps_scale=run["eps_scale"], eps_dir=run["eps_dir"],
                       patience=run["patience"], trace=True)
        U = int(r.tiles_used[0, 0])
        assert U == run["tiles_used"], run["why"]
        tr = r.trace[0, 0]
        # every evaluated comparison matches the closed form of the design
        for t in range(1, U):
            assert abs(tr[t, 2] - exp_scale[t - 1]) < 2e-7, (t, tr[t, 2], exp_scale[t - 1])
            assert abs(tr[t, 3] - exp_dir[t - 1]) < 2e-7, (t, tr[t, 3], exp_dir[t - 1])
        assert np.isnan(tr[0, 2]) and np.isnan(tr[0, 3])  # no comparison at tile 0
        if U < fx["n_tiles"]:
            assert np.isnan(tr[U, 7])  # tiles after the stop are never visited


def test_probe_ignores_dims_beyond_eight():
    fx = json.load(open(os.path.join(GOLDEN, "and_rule.json")))
    r1 = run_oracle(designed_case(fx, seed=0))
    r2 = run_oracle(designed_case(fx, seed=1))  # different distractor in dims 8..15
    assert (r1.tiles_used == r2.tiles_used).all()


# ---------------------------------------------------------------- P7: paged layout

@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_paged_permutation_invariance(kv):
    c = rand_case(B=2, Hq=4, Hkv=2, d=16, n=160, seed=21, kv=kv, qd=kv, tile=16,
                  eps_scale=0.05, eps_dir=0.02)
    c.ctx_lens[:] = [160, 77]
    base = run_oracle(c)
    for s in (1, 2):
        p = to_paged(c, 16, seed=s, extra_blocks=5)
        r = run_oracle(p)
        assert np.array_equal(r.out, base.out) and np.array_equal(r.tiles_used, base.tiles_used)


def test_bad_block_id_rejected():
    c = to_paged(rand_case(B=1, Hq=1, Hkv=1, d=8, n=32, seed=1, tile=16), 16, seed=0)
    c.block_table[0, 1] = c.k.shape[0]  # one past the last block
    with pytest.raises(ValueError):
        run_oracle(c)


# ---------------------------------------------------------------- P8: GQA = replicated cache

def test_gqa_equals_replicated_cache():
    c = rand_case(B=2, Hq=8, Hkv=2, d=16, n=200, seed=31, tile=16, eps_scale=0.05, eps_dir=0.02)
    rep = contiguous_case(c.q, np.repeat(c.k, 4, axis=1), np.repeat(c.v, 4, axis=1),
                          c.ctx_lens, tile=16, eps_scale=0.05, eps_dir=0.02)
    a, b = run_oracle(c), run_oracle(rep)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.tiles_used, b.tiles_used)


# ---------------------------------------------------------------- P9: int8 = dequantised fp32

def test_int8_equals_dequantised_fp32():
    c = A.config(5, small=True, seed=2, batch=1, ctx=512)
    deq = lambda codes, sc: (codes.astype(np.float32) * sc.view(np.float16).astype(np.float32)[..., None])
    f = A.Case(name="deq", B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, q=c.q,
               k=deq(c.k, c.k_scale), v=deq(c.v, c.v_scale), ctx_lens=c.ctx_lens,
               block_size=c.block_size, block_table=c.block_table, tile=c.tile)
    for kw in (dict(v_skip_eps=0.0), dict(v_skip_eps=1e-6),
               dict(eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)):
        a = run_oracle(c, **kw)
        b = run_oracle(f, **kw)
        assert np.array_equal(a.out, b.out) and np.array_equal(a.tiles_used, b.tiles_used)


def int4_reference_decode(packed, sc):
    """The int4 codec decoded by hand: byte i holds element 2i in bits 0-3 and
    element 2i+1 in bits 4-7, each a two's complement 4-bit code."""
    out = np.zeros(packed.shape[:-1] + (2 * packed.shape[-1],), np.float32)
    for e in range(out.shape[-1]):
        byte = packed[..., e // 2].astype(np.int32)
        nib = (byte >> (4 * (e % 2))) & 15
        out[..., e] = np.where(nib > 7, nib - 16, nib)
    return out * sc.view(np.float16).astype(np.float32)[..., None]


def test_int4_codec_round_trip():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 3, 64)).astype(np.float32)
    x[0, 0] = 0.0
    packed, sc = A.quantize_int4(x)
    assert packed.shape == (5, 3, 32) and packed.dtype == np.uint8
    y = int4_reference_decode(packed, sc)
    step = sc.view(np.float16).astype(np.float32)[..., None]
    assert (np.abs(y - x) <= 0.5 * step + 1e-6).all()   # rounding to the nearest code
    assert (y[0, 0] == 0).all()
    # codes span -7..7 and the largest magnitude of each row maps to +-7
    codes = np.rint(y / step)
    assert codes.min() >= -7 and codes.max() <= 7
    assert (np.abs(codes).max(axis=-1)[1:] == 7).all()


def test_int4_equals_dequantised_fp32():
    c = A.config(5, small=True, seed=3, batch=1, ctx=512, kv_dtype="i4")
    assert c.kv_dtype == "i4" and c.k.shape[-1] == c.d // 2
    f = A.Case(name="deq", B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, q=c.q,
               k=int4_reference_decode(c.k, c.k_scale), v=int4_reference_decode(c.v, c.v_scale),
               ctx_lens=c.ctx_lens, block_size=c.block_size, block_table=c.block_table, tile=c.tile)
    for kw in (dict(v_skip_eps=0.0), dict(v_skip_eps=1e-4),
               dict(eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)):
        a = run_oracle(c, **kw)
        b = run_oracle(f, **kw)
        assert np.array_equal(a.out, b.out) and np.array_equal(a.tiles_used, b.tiles_used)
    # and full mode is plain attention over the decoded cache
    r = run_oracle(c, eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)
    n = int(c.ctx_lens[0])
    for h in (0, c.Hq - 1):
        assert np.allclose(r.out[0, h], BF.attention(c, 0, h, n), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P10: V skip

def test_vskip_limits():
    c = rand_case(B=1, Hq=2, Hkv=1, d=16, n=200, seed=41, tile=16)
    base = run_oracle(c)
    zero = run_oracle(c, v_skip_eps=0.0)
    assert np.array_equal(base.out, zero.out)
    none_kept = run_oracle(c, v_skip_eps=1.0001, eps_scale=0.0, eps_dir=0.0)
    assert (none_kept.out == 0).all()  # every exp(s - M) <= 1 < eps


def test_vskip_one_hot_weights():
    # with V = identity rows the output is the weight vector: skipped rows give
    # exactly 0, kept rows keep their full softmax weight (skipped mass stays in l)
    n = d = 64
    rng = np.random.default_rng(42)
    q = rng.standard_normal((1, 1, d)) * 4
    K = rng.standard_normal((1, 1, n, d))
    c = contiguous_case(q, K, np.eye(n)[None, None], tile=8, eps_scale=0.0, eps_dir=0.0)
    eps = 1e-3
    w_skip = run_oracle(c, v_skip_eps=eps).out[0, 0]
    w = BF.attention_weights(c, 0, 0, n)
    zeroed = w_skip == 0
    assert zeroed.any() and (~zeroed).any()
    assert np.allclose(w_skip[~zeroed], w[~zeroed], rtol=1e-12, atol=1e-16)
    assert (w[zeroed] < eps).all()  # a final weight never exceeds exp(s - M_t)
    # the decision uses the running max: the first tile's top score is never skipped
    s0 = K[0, 0, :8] @ q[0, 0] / np.sqrt(d)
    assert not zeroed[int(np.argmax(s0))]


def test_vskip_error_bound():
    c = A.config(3, small=True, seed=6, batch=1, ctx=1024)
    full = run_oracle(c, eps_scale=0.0, eps_dir=0.0)
    eps = 1e-3
    sk = run_oracle(c, eps_scale=0.0, eps_dir=0.0, v_skip_eps=eps, trace=True)
    G = c.Hq // c.Hkv
    for h in range(c.Hq):
        V = BF.logical_rows(c, "v", 0, h // G, 1024)
        n_skipped = int(1024 - np.nansum(sk.trace[0, h, :, 5]))
        bound = n_skipped * eps * np.linalg.norm(V, axis=1).max()
        assert np.linalg.norm(sk.out[0, h] - full.out[0, h]) <= bound + 1e-12


# ---------------------------------------------------------------- P11: output awareness

def test_low_weight_large_value_row_delays_the_stop():
    """A row with a low attention weight but a large value moves the output,
    so the stop rule does not fire at its tile (ART summary, section 1 and 2.2:
    low-weight tokens can matter through their values; the criterion watches
    the output, not the scores)."""
    rng = np.random.default_rng(77)
    d, T, n = 32, 16, 16 * 8
    q = rng.standard_normal((1, 1, d))
    K = rng.standard_normal((1, 1, n, d))
    V = np.ones((1, 1, n, d))
    c0 = contiguous_case(q, K, V, tile=T, eps_scale=1e-3, eps_dir=1e-4)
    assert run_oracle(c0).tiles_used[0, 0] == 2  # constant V: stable at t=1
    # plant a row in tile 1 whose logit is -2 sigma and whose value is x50 and rotated
    qv = c0.q[0, 0].astype(np.float64)
    sigma = np.linalg.norm(qv) / np.sqrt(d)
    j = T + 5
    kp = -2 * sigma * np.sqrt(d) * qv / (qv @ qv)
    K2 = K.copy(); K2[0, 0, j] = kp
    V2 = V.copy(); V2[0, 0, j] = 0.0; V2[0, 0, j, 1] = 50.0
    c1 = contiguous_case(q, K2, V2, tile=T, eps_scale=1e-3, eps_dir=1e-4)
    r1 = run_oracle(c1, trace=True)
    w = BF.attention_weights(c1, 0, 0, 2 * T)
    assert w[j] < 1.0 / (2 * T)                      # key-only view: below-average weight
    assert r1.trace[0, 0, 1, 2] >= 1e-3 or r1.trace[0, 0, 1, 3] >= 1e-4
    assert r1.tiles_used[0, 0] > 2                   # the stop moved past the planted tile


def test_vskip_uses_running_max_through_the_tile():
    """Designed scores: tile 0 holds the overall maximum, tile 1's best row sits
    20 below it, tile 2 holds a row 20 above tile 0's max.  With the running max
    through the current tile, tile 1's best row is skipped (exp(-20) < eps) even
    though it tops its own tile, and tile 0's best row is kept even though a
    later tile exceeds it by 20."""
    d, T = 8, 4
    q = np.zeros((1, 1, d)); q[0, 0, 0] = np.sqrt(d)    # score = k[0]
    K = np.zeros((1, 1, 3 * T, d))
    K[0, 0, :, 0] = [5, 0, 0, 0,    -15, -30, -30, -30,    25, 0, 0, 0]
    n = 3 * T
    V = np.zeros((1, 1, n, n)); V[0, 0] = np.eye(n)
    K = np.concatenate([K, np.zeros((1, 1, n, n - d))], axis=-1)
    q = np.concatenate([q, np.zeros((1, 1, n - d))], axis=-1)
    c = contiguous_case(q, K, V, tile=T, eps_scale=0.0, eps_dir=0.0)
    w = run_oracle(c, v_skip_eps=1e-6).out[0, 0]
    assert w[4] == 0.0          # top of tile 1, but exp(-15 - 5) < 1e-6
    assert w[0] > 0.0           # top of tile 0 when it was read
    assert w[8] > 0.0


# ---------------------------------------------------------------- P-order: tile orders (section 2.4)
#
# Section 2.4 of the ART summary lets the tile sequence be reordered
# (recency-first, importance-first) with no approximation error, block 0 (the
# attention sink) being evaluated first.  A tile order is an index remap: ART
# over a cache in order pi must equal ART in ascending order over the cache
# whose tile s physically holds tile pi(s).

def visiting_order(order, nt, perm_row=None):
    if order == 0:
        return list(range(nt))
    if order == 1:
        return [0] + list(range(nt - 1, 0, -1))
    return [int(x) for x in perm_row[:nt]]


def permuted_tiles(case, orders):
    """Contiguous case whose row b holds, as tile s, the tile orders[b][s] of `case`."""
    import copy
    T = case.tile
    c = copy.copy(case)
    c.k = case.k.copy()
    c.v = case.v.copy()
    for b, seq in enumerate(orders):
        for s, src in enumerate(seq):
            c.k[b, :, s * T:(s + 1) * T] = case.k[b, :, src * T:(src + 1) * T]
            c.v[b, :, s * T:(s + 1) * T] = case.v[b, :, src * T:(src + 1) * T]
    c.order, c.tile_perm = 0, None
    return c


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_order_full_mode_is_plain_attention(order, kv):
    c = rand_case(B=3, Hq=6, Hkv=2, d=32, n=200, seed=41 + order, kv=kv, qd=kv, tile=16,
                  eps_scale=0.0, eps_dir=0.0)
    c.ctx_lens[:] = [200, 17, 129]
    c.order = order
    c.tile_perm = A.sink_first_orders(c.ctx_lens, 16, seed=5) if order == 2 else None
    r = run_oracle(c)
    for b in range(3):
        n = int(c.ctx_lens[b])
        assert (r.tiles_used[b] == ntiles(n, 16)).all()
        for h in range(6):
            assert np.allclose(r.out[b, h], BF.attention(c, b, h, n), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("seed", range(4))
def test_order_equals_physically_permuted_cache(order, seed):
    T = 8
    c = rand_case(B=3, Hq=4, Hkv=2, d=16, n=320, seed=200 + seed, tile=T,
                  eps_scale=0.05, eps_dir=0.02, patience=1 + seed % 2)
    c.ctx_lens[:] = [320, 160 - 8 * seed, 24]
    c.order = order
    c.tile_perm = A.sink_first_orders(c.ctx_lens, T, stride=50, seed=seed) if order == 2 else None
    seqs = [visiting_order(order, ntiles(int(n), T), None if c.tile_perm is None else c.tile_perm[b])
            for b, n in enumerate(c.ctx_lens)]
    r = run_oracle(c, trace=True)
    ref = run_oracle(permuted_tiles(c, seqs), trace=True)
    assert np.array_equal(r.tiles_used, ref.tiles_used)
    assert np.array_equal(r.out, ref.out)
    assert np.array_equal(np.isnan(r.trace), np.isnan(ref.trace))
    assert np.array_equal(np.nan_to_num(r.trace), np.nan_to_num(ref.trace))
    U = r.tiles_used[0]
    assert (U < ntiles(320, T)).any() and (U > 2).any()  # stops, and not all at once
    # the order changes the outcome (else this would not test the remap)
    asc = run_oracle(c, order=0, tile_perm=None)
    assert not np.array_equal(asc.tiles_used, r.tiles_used)


@pytest.mark.parametrize("seed", range(4))
def test_recent_first_ragged_tile_and_stop(seed):
    # the partial last tile is visited second; the output of a stopped head is
    # attention over the tiles it visited
    T = 8
    c = rand_case(B=2, Hq=4, Hkv=2, d=16, n=300, seed=300 + seed, tile=T,
                  eps_scale=0.05, eps_dir=0.02, patience=1 + seed % 2)
    c.ctx_lens[:] = [300, 211 - 9 * seed]
    c.order = 1
    r = run_oracle(c)
    stopped = 0
    for b in range(2):
        n = int(c.ctx_lens[b])
        nt = ntiles(n, T)
        seq = visiting_order(1, nt)
        for h in range(4):
            U = int(r.tiles_used[b, h])
            stopped += U < nt
            pos = [j for s in seq[:U] for j in range(s * T, min(n, (s + 1) * T))]
            assert np.allclose(r.out[b, h], BF.attention_at(c, b, h, pos), rtol=1e-12, atol=1e-13)
    assert stopped > 0


def test_recent_first_stops_early_where_recent_tokens_dominate():
    # scores high on the last tile only: ascending order meets the dominant
    # tile last and runs to the end; sink + recency-first meets it second and
    # stops right after, with an output close to full attention
    T, nt, d = 16, 40, 32
    n = T * nt
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, d))
    K = rng.standard_normal((1, 1, n, d)) * 0.05
    K[0, 0, -T:] += 9.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    V = rng.standard_normal((1, 1, n, d))
    c = contiguous_case(q, K, V, tile=T, eps_scale=1e-3, eps_dir=1e-4, patience=2)
    asc = run_oracle(c)
    c.order = 1
    rec = run_oracle(c)
    full = BF.attention(c, 0, 0, n)
    assert int(asc.tiles_used[0, 0]) == nt
    assert int(rec.tiles_used[0, 0]) <= 5
    assert np.abs(rec.out[0, 0] - full).max() < 1e-2


def test_invalid_tile_orders_rejected():
    T = 16
    c = rand_case(B=2, Hq=2, Hkv=1, d=16, n=160, seed=17, tile=T, eps_scale=0.0, eps_dir=0.0)
    c.order = 2
    good = A.sink_first_orders(c.ctx_lens, T, seed=1)
    c.tile_perm = good
    run_oracle(c)
    for b, s, val in [(0, 0, 3), (1, 4, 0), (1, 9, 10), (0, 2, -1)]:
        bad = good.copy()
        bad[b, s] = val
        c.tile_perm = bad
        with pytest.raises(ValueError):
            run_oracle(c)
    c.tile_perm = good[:, :5]  # shorter than a row's tiles
    with pytest.raises(ValueError):
        run_oracle(c)


def test_order_entries_past_the_stop_are_not_read():
    # constant V: the probe is the same after every tile, so every head stops
    # after tile 1 (patience 1) and later entries are never visited
    T, nt, d = 16, 10, 16
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, d))
    K = rng.standard_normal((1, 1, T * nt, d))
    V = np.repeat(rng.standard_normal((1, 1, 1, d)), T * nt, axis=2)
    c = contiguous_case(q, K, V, tile=T, eps_scale=1e-3, eps_dir=1e-4, patience=1)
    c.order = 2
    perm = A.sink_first_orders(c.ctx_lens, T, seed=2)
    perm[0, 2:] = 99
    c.tile_perm = perm
    r = run_oracle(c)
    assert (r.tiles_used == 2).all()
    perm[0, 1] = 99
    with pytest.raises(ValueError):
        run_oracle(c)


# ---------------------------------------------------------------- per-head tables (composition with retention)
#
# ART runs unchanged on top of a per-head retention or eviction policy (ART
# summary, section 2.4: an orthogonal control layer).  With per-head tables
# every (row, KV head) is its own sequence; the pins tie that to calls with
# shared tables and to plain attention over the positions a policy kept.

def paged_case(B=3, Hq=8, Hkv=2, d=16, n=640, seed=0, T=16, **params):
    c = rand_case(B=B, Hq=Hq, Hkv=Hkv, d=d, n=n, seed=seed, tile=T, **params)
    return to_paged(c, 16, seed=seed + 1, extra_blocks=5)


def per_head_slice(c, g):
    """The KV head g of a per-head case as a call of its own with shared tables."""
    import copy
    G = c.Hq // c.Hkv
    s = copy.copy(c)
    s.Hq, s.Hkv = G, 1
    s.q = np.ascontiguousarray(c.q[:, g * G:(g + 1) * G])
    s.k = np.ascontiguousarray(c.k[:, g:g + 1])
    s.v = np.ascontiguousarray(c.v[:, g:g + 1])
    s.ctx_lens = np.ascontiguousarray(c.ctx_lens[:, g])
    s.block_table = np.ascontiguousarray(c.block_table[:, g])
    s.tile_perm = None if c.tile_perm is None else np.ascontiguousarray(c.tile_perm[:, g])
    s.per_head_tables = False
    return s


@pytest.mark.parametrize("order", [0, 1, 2])
def test_per_head_identical_tables_equal_shared_tables(order):
    c = paged_case(seed=31, eps_scale=0.05, eps_dir=0.02)
    c.ctx_lens[:] = [640, 401, 77]
    c.order = order
    c.tile_perm = A.sink_first_orders(c.ctx_lens, 16, stride=40, seed=2) if order == 2 else None
    ref = run_oracle(c)
    import copy
    p = copy.copy(c)
    p.per_head_tables = True
    p.ctx_lens = np.repeat(c.ctx_lens[:, None], c.Hkv, axis=1)
    p.block_table = np.repeat(c.block_table[:, None], c.Hkv, axis=1)
    p.tile_perm = None if order != 2 else np.repeat(c.tile_perm[:, None], c.Hkv, axis=1)
    r = run_oracle(p)
    assert np.array_equal(r.tiles_used, ref.tiles_used) and np.array_equal(r.out, ref.out)


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("keep", [0.0, 0.5])
def test_per_head_tables_equal_separate_calls(order, keep):
    c = paged_case(B=3, Hq=8, Hkv=2, n=960, seed=40, eps_scale=0.05, eps_dir=0.02)
    c.ctx_lens[:] = [960, 611, 203]
    p = A.retained_tables(c, sink_blocks=2, recent_blocks=24, keep_frac=keep, seed=7)
    assert (p.ctx_lens[:, 0] != p.ctx_lens[:, 1]).any() or keep == 0.0
    p.order = order
    p.tile_perm = A.sink_first_orders(p.ctx_lens, 16, stride=60, seed=4) if order == 2 else None
    r = run_oracle(p)
    G = c.Hq // c.Hkv
    for g in range(c.Hkv):
        s = run_oracle(per_head_slice(p, g))
        assert np.array_equal(r.tiles_used[:, g * G:(g + 1) * G], s.tiles_used)
        assert np.array_equal(r.out[:, g * G:(g + 1) * G], s.out)
    assert (r.tiles_used < -(-p.ctx_lens.repeat(G, axis=1) // 16)).any()  # some heads stop


def test_retained_full_mode_is_attention_over_kept_positions():
    c = paged_case(B=2, Hq=4, Hkv=2, n=700, seed=50, eps_scale=0.0, eps_dir=0.0)
    c.ctx_lens[:] = [700, 333]
    p = A.retained_tables(c, sink_blocks=1, recent_blocks=5, keep_frac=0.4, seed=3)
    r = run_oracle(p)
    G = c.Hq // c.Hkv
    for b in range(2):
        n = int(c.ctx_lens[b])
        for g in range(2):
            k = -(-int(p.ctx_lens[b, g]) // 16)
            blocks = [int(np.flatnonzero(c.block_table[b] == blk)[0]) for blk in p.block_table[b, g, :k]]
            pos = [j for i in blocks for j in range(16 * i, min(n, 16 * (i + 1)))]
            assert len(pos) == p.ctx_lens[b, g]
            for h in range(g * G, (g + 1) * G):
                assert r.tiles_used[b, h] == -(-len(pos) // 16)
                assert np.allclose(r.out[b, h], BF.attention_at(c, b, h, pos), rtol=1e-12, atol=1e-13)


def test_per_head_lengths_checked():
    c = paged_case(B=2, Hq=4, Hkv=2, n=320, seed=60)
    p = A.retained_tables(c, sink_blocks=1, recent_blocks=4, keep_frac=1.0, seed=1)
    p.ctx_lens[1, 1] = p.block_table.shape[-1] * 16 + 1
    with pytest.raises(ValueError):
        run_oracle(p)
