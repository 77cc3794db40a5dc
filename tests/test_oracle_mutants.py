"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle/art_oracle.c with one plausible mistake
planted by a textual substitution (a dropped term, a wrong index, a flipped
comparison, a different reading of the method).  The mutant is compiled with
gcc into a temporary library, swapped in for the real one, and the pins of
tests/test_oracle.py are run against it: at least one must fail.  Mistakes are
planted only in the oracle, only on the CPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "art_oracle.c")

MUTANTS = {
    "norm_of_difference": ("ds = fabs(xn - prev_norm) / prev_norm;",
                           "{ double s2 = 0; for (int i = 0; i < P; ++i) s2 += (x[i]-prev[i])*(x[i]-prev[i]); ds = sqrt(s2) / prev_norm; }"),
    "no_rescale_of_l": ("l *= alpha;", ";"),
    "no_rescale_of_acc": ("for (int i = 0; i < d; ++i) acc[i] *= alpha;", ";"),
    "gqa_modulo_mapping": ("g = h / G;", "g = h % J->Hkv;"),
    "non_strict_threshold": ("if (ds < J->eps_scale && dd < J->eps_dir) ++streak;",
                             "if (ds <= J->eps_scale && dd <= J->eps_dir) ++streak;"),
    "or_instead_of_and": ("if (ds < J->eps_scale && dd < J->eps_dir) ++streak;",
                          "if (ds < J->eps_scale || dd < J->eps_dir) ++streak;"),
    "streak_not_reset": ("else streak = 0;", "else {}"),
    "probe_dims_shifted": ("for (int i = 0; i < P; ++i) x[i] = acc[i] / l;",
                           "for (int i = 0; i < P; ++i) x[i] = acc[i + 1] / l;"),
    "unnormalised_probe": ("for (int i = 0; i < P; ++i) x[i] = acc[i] / l;",
                           "for (int i = 0; i < P; ++i) x[i] = acc[i];"),
    "check_from_tile_0": ("if (t >= 1) {\n            if (xn == 0.0 || prev_norm == 0.0) {",
                          "if (t >= 0) {\n            if (t == 0) { ds = 0.0; dd = 0.0; } else if (xn == 0.0 || prev_norm == 0.0) {"),
    "stop_excludes_tile": ("if (stop) { U = t + 1; break; }", "if (stop) { U = t; break; }"),
    "no_sqrt_d_scaling": ("s[j - j0] = dot / sqrt_d;", "s[j - j0] = dot;"),
    "skipped_weight_not_in_l": ("            l += p;\n            if (J->v_skip_eps > 0.0 && p < J->v_skip_eps) continue;",
                                "            if (J->v_skip_eps > 0.0 && p < J->v_skip_eps) continue;\n            l += p;"),
    "vskip_tile_local_max": ("if (J->v_skip_eps > 0.0 && p < J->v_skip_eps) continue;",
                             "if (J->v_skip_eps > 0.0 && exp(s[j - j0] - tmax) < J->v_skip_eps) continue;"),
    "paged_offset_wrong": ("return ((long)blk * J->Hkv + g) * J->block_size + (j % J->block_size);",
                           "return ((long)blk * J->Hkv + g) * J->block_size + (j / J->block_size) % J->block_size;"),
    "last_tile_not_masked": ("const int j0 = pt * T, j1 = (j0 + T < n) ? j0 + T : n;",
                             "const int j0 = pt * T, j1 = (j0 + T < n) ? j0 + T : ((nt * T <= J->max_ctx) ? nt * T : n);"),
    "order_ignored": ("if (J->order == 0) return t;", "return t;"),
    "recent_order_shifted": ("return t == 0 ? 0 : nt - t;", "return t == 0 ? 0 : nt - 1 - t + (t == nt - 1);"),
    "recent_order_oldest_first": ("return t == 0 ? 0 : nt - t;", "return t;"),
    "perm_row_ignored": ("J->perm[sq * J->perm_stride + t]", "J->perm[t]"),
    "perm_sink_not_forced": ("if (t == 0) return e == 0 ? 0 : -1;", "if (t == 0) return (e >= 0 && e < nt) ? e : -1;"),
    "positions_from_step": ("const int j0 = pt * T, j1", "const int j0 = t * T, j1"),
    "int4_nibbles_swapped": ("int nib = (i % 2 == 0) ? (p[i / 2] & 0x0f) : (p[i / 2] >> 4);",
                             "int nib = (i % 2 == 1) ? (p[i / 2] & 0x0f) : (p[i / 2] >> 4);"),
    "int4_unsigned_codes": ("int code = nib >= 8 ? nib - 16 : nib;", "int code = nib;"),
    "per_head_sequence_ignored": ("return J->per_head ? (long)b * J->Hkv + g : b;", "return b;"),
    "per_head_table_row_shared": ("J->block_table[seq_of(J, b, g) * J->max_blocks_per_seq",
                                  "J->block_table[(long)b * J->max_blocks_per_seq"),
    "per_head_list_row_shared": ("const int pt = visit_tile(J, sq, nt, t);", "const int pt = visit_tile(J, b, nt, t);"),
    "int8_scale_ignored": ("double s = widen_f16(scale[row]);", "double s = 1.0;"),
    "direction_not_clamped_half": ("dd = 1.0 - dot / (xn * prev_norm);", "dd = 0.5 * (1.0 - dot / (xn * prev_norm));"),
    "zero_norm_probe_passes": ("                ds = INFINITY;\n                dd = INFINITY;",
                               "                ds = 0.0;\n                dd = 0.0;"),
    "f16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "f16_inf_as_max": ("v = m ? NAN : INFINITY;", "v = m ? NAN : 65504.0;"),
    "f16_sign_dropped": ("return sign ? -v : v;", "return v;"),
}

# pins to run against every mutant (name -> callable with fixed arguments)
PINS = [
    lambda: [P.test_full_mode_equals_bruteforce(n, d, T) for n in (5, 65, 300) for d in (4, 64) for T in (1, 16)],
    lambda: [P.test_full_mode_gqa_ragged_bruteforce(kv) for kv in ("f32", "bf16")],
    P.test_single_tile_is_plain_attention_and_zero_context,
    lambda: [P.test_stop_equals_attention_over_used_prefix(s) for s in range(6)],
    P.test_full_mode_weights_are_softmax_and_convex,
    lambda: [P.test_tiles_used_bounds(p) for p in (1, 2, 4)],
    lambda: [P.test_constant_values(p) for p in (1, 3)],
    lambda: [P.test_designed_sequences(f) for f in P.FIXTURES],
    P.test_probe_ignores_dims_beyond_eight,
    lambda: [P.test_paged_permutation_invariance(kv) for kv in ("f32", "bf16")],
    P.test_gqa_equals_replicated_cache,
    P.test_int8_equals_dequantised_fp32,
    P.test_vskip_limits,
    P.test_vskip_one_hot_weights,
    P.test_vskip_error_bound,
    P.test_vskip_uses_running_max_through_the_tile,
    P.test_low_weight_large_value_row_delays_the_stop,
    lambda: [P.test_order_full_mode_is_plain_attention(o, "f32") for o in (1, 2)],
    lambda: [P.test_order_equals_physically_permuted_cache(o, s) for o in (1, 2) for s in range(2)],
    lambda: [P.test_recent_first_ragged_tile_and_stop(s) for s in range(2)],
    P.test_recent_first_stops_early_where_recent_tokens_dominate,
    P.test_invalid_tile_orders_rejected,
    P.test_order_entries_past_the_stop_are_not_read,
    lambda: [P.test_per_head_tables_equal_separate_calls(o, k) for o in (0, 2) for k in (0.0, 0.5)],
    P.test_retained_full_mode_is_attention_over_kept_positions,
    P.test_int4_equals_dequantised_fp32,
    lambda: [P.test_zero_norm_probe_never_passes(k, p) for k, p in ((0, 1), (3, 1), (3, 2))],
    P.test_widen_f16_every_pattern,
    P.test_int8_with_subnormal_scales_equals_dequantised_fp32,
]


def _build_mutant(tmp, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    path = os.path.join(tmp, "mut.c")
    open(path, "w").write(src.replace(old, new))
    lib = os.path.join(tmp, "libmut.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", path, "-o", lib, "-lm", "-lpthread"],
                   check=True, capture_output=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    import ctypes
    old, new = MUTANTS[name]
    tmp = tempfile.mkdtemp()
    try:
        lib = ctypes.CDLL(_build_mutant(tmp, old, new))
        real = oracle._load()
        f = lib.art_oracle_decode
        f.argtypes, f.restype = real.art_oracle_decode.argtypes, real.art_oracle_decode.restype
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = []
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, pytest.fail.Exception):
                caught.append(getattr(pin, "__name__", "lambda"))
        assert caught, f"no pin detects mutant {name}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
