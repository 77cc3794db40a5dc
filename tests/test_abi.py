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
    assert lib.art_abi_version() == 7


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
    (dict(engine=5), -5),
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
