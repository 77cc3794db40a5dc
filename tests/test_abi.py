"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/art.h, and rejects bad arguments on the host."""
import ctypes
import math
import os
import re

import pytest

import kv_cache_bandwidth_amd as art
from kv_cache_bandwidth_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "art.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(art_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = art.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.art_abi_version() == 9


def desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype=B.ART_BF16,
                kv_dtype=B.ART_BF16, block_size=16, max_blocks_per_seq=4, num_blocks=8,
                patience=1)
    base.update(kw)
    return B.make_desc(**base)


def ok_desc(**kw):
    d = desc(**kw)
    need = B.workspace_bytes(d, kw.get("tile", 64))
    assert need > 0
    d.workspace = 1 << 20  # any aligned address: validation never dereferences it
    d.workspace_bytes = need
    return d


def test_valid_desc_passes():
    assert B.validate(ok_desc(), 64, 1e-3, 1e-4) == 0
    assert B.validate(ok_desc(block_size=0, max_ctx=64), 64, 0.0, 0.0) == 0
    assert B.validate(ok_desc(tile_order=1), 64, 1e-3, 1e-4) == 0
    assert B.validate(ok_desc(per_head_tables=1), 64, 1e-3, 1e-4) == 0
    # a caller's order: one entry per tile a row can hold (8 blocks of 16 -> 2 tiles of 64)
    assert B.validate(ok_desc(max_blocks_per_seq=8, tile_order=2, tile_perm=1 << 20, tile_perm_stride=2),
                      64, 1e-3, 1e-4) == 0
    assert B.validate(desc(max_blocks_per_seq=8, tile_order=2, tile_perm=1 << 20, tile_perm_stride=1),
                      64, 1e-3, 1e-4) == -2


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2),
    (dict(num_q_heads=0), -2),
    (dict(num_q_heads=7), -2),                 # not a multiple of num_kv_heads
    (dict(num_q_heads=34, num_kv_heads=2), -2),  # 17 heads per KV head
    (dict(head_dim=96), -2),
    (dict(q_dtype=B.ART_I8), -3),
    (dict(kv_dtype=7), -3),
    (dict(kv_dtype=B.ART_I8), -1),             # int8 without scales
    (dict(kv_dtype=B.ART_I4), -1),             # int4 without scales
    (dict(block_size=8), -2),
    (dict(block_size=24), -2),
    (dict(max_blocks_per_seq=0), -2),
    (dict(num_blocks=0), -2),
    (dict(block_size=0, max_ctx=100), -2),     # contiguous stride not a multiple of 16
    (dict(patience=0), -5),
    (dict(v_skip_eps=-1.0), -5),
    (dict(v_skip_eps=float("nan")), -5),
    (dict(max_workers=-3), -5),
    (dict(team_helpers=-1), -5),
    (dict(team_helpers=4), -5),
    (dict(engine=-1), -5),
    (dict(engine=7), -5),
    (dict(workers_per_cu=-1), -5),
    (dict(window=-1), -5),
    (dict(window=113), -5),
    (dict(tile_order=-1), -5),
    (dict(tile_order=3), -5),
    (dict(tile_order=2), -1),                  # a caller's order without tile_perm
    (dict(per_head_tables=2), -5),
    (dict(tile_order=2, tile_perm=1 << 20, tile_perm_stride=0), -2),  # 4 blocks of 16 = 1 tile
])
def test_bad_desc_rejected(kw, code):
    assert B.validate(desc(**kw), 64, 1e-3, 1e-4) == code
    assert B.workspace_bytes(desc(**kw), 64) == 0
    assert art.load().art_last_error().decode() != ""


@pytest.mark.parametrize("tile", [0, 8, 48, 256])
def test_bad_tile_rejected(tile):
    assert B.validate(ok_desc(), tile, 1e-3, 1e-4) == -4


@pytest.mark.parametrize("eps", [(-1e-3, 1e-4), (1e-3, float("nan")), (math.inf, 1e-4)])
def test_bad_thresholds_rejected(eps):
    assert B.validate(ok_desc(), 64, *eps) == -5


def test_workspace_checks():
    d = ok_desc()
    d.workspace = None
    assert B.validate(d, 64, 1e-3, 1e-4) == -6
    d = ok_desc()
    d.workspace = (1 << 20) + 16
    assert B.validate(d, 64, 1e-3, 1e-4) == -6
    d = ok_desc()
    d.workspace_bytes -= 1
    assert B.validate(d, 64, 1e-3, 1e-4) == -6


def test_null_desc_and_status_strings():
    lib = art.load()
    assert lib.art_validate(None, 64, 1e-3, 1e-4) == -1
    assert lib.art_workspace_bytes(None, 64) == 0
    for code in range(-7, 1):
        assert lib.art_status_string(code)
    assert b"unknown" in lib.art_status_string(-99)


def test_decode_rejects_before_touching_device():
    # invalid arguments return an error without launching anything
    lib = art.load()
    d = desc(patience=0)
    rc = lib.art_decode_attention(ctypes.byref(d), None, None, None, None, None, 64, 1e-3, 1e-4,
                                  None, None, None)
    assert rc == -5
    d = ok_desc()
    rc = lib.art_decode_attention(ctypes.byref(d), None, None, None, None, None, 64, 1e-3, 1e-4,
                                  None, None, None)
    assert rc == -1  # q/k/v/ctx_lens/out/tiles_used missing


def test_noalloc_refuses_on_the_host():
    # art_decode_attention_noalloc checks the call and its workspace size
    # before it looks up its static array on the device
    lib = art.load()
    limit = int(re.search(r"#define ART_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
                .expand(r"\1")) << 20
    assert limit == 96 << 20
    assert lib.art_decode_attention_noalloc(None, None, None, None, None, None, 64, 1e-3, 1e-4,
                                            None, None, None) == -1
    d = desc(patience=0)
    assert lib.art_decode_attention_noalloc(ctypes.byref(d), None, None, None, None, None, 64, 1e-3, 1e-4,
                                            None, None, None) == -5
    # 64 rows of 64K tokens: more workspace than the array holds, whatever desc.workspace says
    d = desc(batch=64, num_q_heads=32, num_kv_heads=8, max_blocks_per_seq=4096, num_blocks=1)
    assert B.workspace_bytes(d, 64) > limit
    d.workspace, d.workspace_bytes = 1 << 20, 1 << 40
    assert lib.art_decode_attention_noalloc(ctypes.byref(d), None, None, None, None, None, 64, 1e-3, 1e-4,
                                            None, None, None) == -6
    assert b"static scratch holds 100663296" in lib.art_last_error()


def test_plain_c_client(tmp_path):
    # the header is valid C11 and the library serves a C program directly
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(art.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c_abi_check.c"), "-o", exe, "-L", lib_dir, "-l:libart.so",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def _cpu_args(**over):
    """Host tensors of a small paged bf16 call (never launched: every case
    below is rejected before the library sees a pointer)."""
    import torch
    B, Hq, Hkv, d, nb, bs = 2, 8, 2, 128, 8, 16
    a = dict(q=torch.zeros(B, Hq, d, dtype=torch.bfloat16),
             k_cache=torch.zeros(nb, Hkv, bs, d, dtype=torch.bfloat16),
             v_cache=torch.zeros(nb, Hkv, bs, d, dtype=torch.bfloat16),
             ctx_lens=torch.zeros(B, dtype=torch.int32),
             block_table=torch.zeros(B, 4, dtype=torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(q="q2d"), "q must be"),
    (dict(k_cache="bad_last_dim"), "k_cache rows"),
    (dict(v_cache="other_shape"), "v_cache must have"),
    (dict(v_cache="other_dtype"), "v_cache must have"),
    (dict(k_cache="int8_no_scales", v_cache="int8_no_scales"), "k_scale must be given"),
    (dict(k_cache="int8", v_cache="int8", k_scale="bad_scale", v_scale="good_scale"), "k_scale must be given"),
    (dict(k_cache="int8", v_cache="int8", k_scale="f32_scale", v_scale="good_scale"), "k_scale must be"),
    (dict(out="bad_out"), "out must be"),
    (dict(tiles_used="bad_used"), "tiles_used must be"),
    (dict(stats="short_stats"), "stats must hold"),
    (dict(stats="int32_stats"), "stats must be"),
    (dict(ctx_lens="int64_lens"), "ctx_lens must be"),
    (dict(block_table="short_table_rows"), "must lead with"),
    (dict(), "contiguous device tensor"),  # well formed, but host tensors
])
def test_binding_rejects_mismatched_tensors(over, match):
    import torch
    nb, Hkv, bs, d = 8, 2, 16, 128
    make = {
        "q2d": torch.zeros(2, 128, dtype=torch.bfloat16),
        "bad_last_dim": torch.zeros(nb, Hkv, bs, 64, dtype=torch.bfloat16),
        "other_shape": torch.zeros(nb, Hkv, bs + 16, d, dtype=torch.bfloat16),
        "other_dtype": torch.zeros(nb, Hkv, bs, d, dtype=torch.float32),
        "int8_no_scales": torch.zeros(nb, Hkv, bs, d, dtype=torch.int8),
        "int8": torch.zeros(nb, Hkv, bs, d, dtype=torch.int8),
        "bad_scale": torch.zeros(nb, Hkv, bs + 1, dtype=torch.float16),
        "good_scale": torch.zeros(nb, Hkv, bs, dtype=torch.float16),
        "f32_scale": torch.zeros(nb, Hkv, bs, dtype=torch.float32),
        "bad_out": torch.zeros(2, 8, 64, dtype=torch.float32),
        "bad_used": torch.zeros(2, 8, dtype=torch.int64),
        "short_stats": torch.zeros(3, dtype=torch.int64),
        "int32_stats": torch.zeros(4, dtype=torch.int32),
        "int64_lens": torch.zeros(2, dtype=torch.int64),
        "short_table_rows": torch.zeros(3, 4, dtype=torch.int32),
    }
    kw = {k: make[v] for k, v in over.items()}
    args = _cpu_args(**{k: kw[k] for k in ("q", "k_cache", "v_cache", "ctx_lens", "block_table") if k in kw})
    rest = {k: v for k, v in kw.items() if k not in args}
    with pytest.raises(ValueError, match=match):
        art.decode_attention(args["q"], args["k_cache"], args["v_cache"], args["ctx_lens"],
                             block_table=args["block_table"], **rest)


def _round_region_bytes(ng, nt_max, g, d=128):
    # the round engine's workspace regions: every step's running state (a
    # partial slot of 48 + G*d floats) and probe record (12 floats per head),
    # the groups' decision states (22 words per lane per head block) and
    # control words (2 + 32 per group), each 256-byte aligned
    def a256(x):
        return (x + 255) // 256 * 256
    slot = 48 + g * d
    hb = (g + 3) // 4
    return (a256(ng * nt_max * slot * 4) + a256(ng * nt_max * g * 12 * 4) + a256(ng * hb * 22 * 64 * 4)
            + a256(ng * 34 * 8))


@pytest.mark.parametrize("batch", [8, 16])
def test_round_engine_workspace_layout(batch):
    # engine ROUND lays out exactly the round regions on top of the team
    # engine's workspace; engine AUTO only where it takes the rounds (at most
    # 64 groups of 256-1024 tiles, at most 4 query heads per group); no
    # round regions with the V skip or off the 64-token streamed tile
    ctx, bs = 32768, 16

    def ws(engine, v_skip=0.0, tile=64, kv=2):
        d = B.make_desc(batch=batch, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype=1, kv_dtype=kv,
                        block_size=bs, max_blocks_per_seq=ctx // bs, num_blocks=batch * ctx // bs,
                        k_scale=1, v_scale=1, engine=engine, v_skip_eps=v_skip)
        return B.workspace_bytes(d, tile)

    ng, nt = batch * 8, ctx // 64
    team, rnd, auto = ws(1), ws(6), ws(0)
    assert team > 0
    assert rnd - team == _round_region_bytes(ng, nt, 4)
    assert auto == (rnd if ng <= 64 else team)
    assert ws(6, v_skip=1e-6) == ws(1, v_skip=1e-6)    # the V skip runs on the team engine
    assert ws(6, tile=32) == ws(1, tile=32)            # only the streamed 64-token tile
    assert ws(6, kv=1) - ws(1, kv=1) == _round_region_bytes(ng, nt, 4)  # bf16 alike
