"""Checks of the seeded input generator (no attention arithmetic under test)."""
import numpy as np
import pytest
import torch

import art_inputs as A
from tests import bruteforce as BF


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.bf16_bits(x), ref)
    assert np.array_equal(A.bf16_value(A.bf16_bits(x)), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_int8_quantiser_roundtrip():
    x = np.random.default_rng(1).standard_normal((64, 128)).astype(np.float32)
    codes, sc = A.quantize_int8(x)
    s = sc.view(np.float16).astype(np.float32)
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
    err = np.abs(codes * s[:, None] - x)
    assert (err <= s[:, None] / 2 + 1e-6 + np.abs(x) * 1e-3).all()


def test_seed_reproducible_and_distinct():
    a = A.config(3, small=True, seed=0)
    b = A.config(3, small=True, seed=0)
    c = A.config(3, small=True, seed=1)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.block_table, b.block_table)
    assert not np.array_equal(a.k, c.k)


def test_paged_layout_is_a_permutation():
    c = A.config(3, small=True)
    t = c.block_table.ravel()
    assert len(np.unique(t)) == t.size and t.min() >= 0 and t.max() < c.num_blocks


def test_temperature_concentrates_mass():
    # logits ~ N(0, beta^2) with beta = z95 + z90: the top 5 % of keys hold ~90 %
    c = A.config(3, small=True, ctx=2048)
    masses = []
    for h in range(0, c.Hq, 7):
        w = BF.attention_weights(c, 0, h, 2048)
        masses.append(np.sort(w)[::-1][: 2048 // 20].sum())
    assert 0.8 < np.mean(masses) < 0.97


@pytest.mark.parametrize("mode,lo,hi", [("sqrt_d", 0.99, 1.0), ("literal", 0.0, 0.05)])
def test_sink_mass(mode, lo, hi):
    c = A.config(2, small=True, sink_mode=mode)
    mass = [BF.attention_weights(c, 0, h, 2048)[:4].sum() for h in range(c.Hq)]
    assert lo <= np.min(mass) and np.max(mass) <= hi


def test_planted_rows_have_logit_minus_two_sigma():
    c = A.config(4, small=True)
    G = c.Hq // c.Hkv
    pos = c.meta["planted_positions"]
    assert pos.shape[-1] == round(0.001 * 8192)
    for b in range(c.B):
        for g in range(c.Hkv):
            K = BF.logical_rows(c, "k", b, g, 8192)
            V = BF.logical_rows(c, "v", b, g, 8192)
            for h in range(g * G, (g + 1) * G):
                qv = BF.query(c, b, h)
                sig = np.linalg.norm(qv) / np.sqrt(c.d)
                s = K[pos[b, g]] @ qv / np.sqrt(c.d)
                assert np.allclose(s, -2 * sig, atol=0.05 * sig)   # exact before bf16 rounding
            assert np.linalg.norm(V[pos[b, g]], axis=1).mean() > 20 * np.linalg.norm(V, axis=1).mean() / 2
