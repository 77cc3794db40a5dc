"""art_decode_attention_noalloc (the library's static workspace) against
art_decode_attention with a caller workspace, both through the C ABI: two
or more calls in a row on one device, each later call smaller than the one
before it, so that every call after the first finds the previous call's
words in the array.  Bar: tiles_used equal, outputs within the parity
tolerance of the cache format (max-abs 2e-3 bf16/int8, 1e-5 fp32), every
output the call finishes finite; the noalloc outputs also meet the oracle."""
import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import check_parity, log, to_device, tol_for

pytestmark = pytest.mark.gpu

ENGINES = {"auto": {}, "team": dict(engine=1), "pool": dict(engine=2), "shared": dict(engine=3),
           "xcd": dict(engine=4)}


def _call(case, dev, noalloc, **kw):
    import torch
    import kv_cache_bandwidth_amd as art
    # outputs start as garbage the call must overwrite
    out = torch.full((case.B, case.Hq, case.d), float("nan"), dtype=torch.float32, device="cuda")
    used = torch.full((case.B, case.Hq), -9, dtype=torch.int32, device="cuda")
    args = dict(block_table=dev["bt"], tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                patience=case.patience, v_skip_eps=case.v_skip_eps, k_scale=dev["ks"], v_scale=dev["vs"],
                tile_order=case.order, tile_perm=dev["perm"] if case.order == 2 else None,
                per_head_tables=case.per_head_tables)
    args.update(kw)
    art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], out=out, tiles_used=used,
                         noalloc=noalloc, **args)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), used.cpu().numpy()


def _compare(case, label, dev=None, oracle=True, **kw):
    dev = dev or to_device(case)
    log(f"[noalloc] {label}: B={case.B} Hq={case.Hq} Hkv={case.Hkv} d={case.d} kv={case.kv_dtype} "
        f"ctx={case.ctx_lens.tolist()[:4]} {kw}")
    o_ws, u_ws = _call(case, dev, False, **kw)
    o_na, u_na = _call(case, dev, True, **kw)
    assert (u_na == u_ws).all(), f"{label}: tiles_used differ on {int((u_na != u_ws).sum())} heads"
    done = u_ws >= 0
    assert np.isfinite(o_na[done]).all(), f"{label}: non-finite noalloc output on a finished head"
    diff = float(np.abs(o_na - o_ws)[done].max()) if done.any() else 0.0
    assert diff <= tol_for(case), f"{label}: max |noalloc - workspace| = {diff:.3e}"
    if oracle:
        es = {k: kw[k] for k in ("eps_scale", "eps_dir", "v_skip_eps") if k in kw}
        check_parity(case, o_na, u_na, **es)
    log(f"[noalloc] {label}: ok, max diff {diff:.2e}, mean tiles_used {u_na.mean():.1f}")


_BIG = {}


def _big():
    if not _BIG:
        c = A.config(3, seed=0)
        _BIG["case"], _BIG["dev"] = c, to_device(c)
    return _BIG["case"], _BIG["dev"]


@pytest.mark.parametrize("engine", list(ENGINES))
def test_noalloc_matches_workspace_call(engine):
    kw = ENGINES[engine]
    # the first call at the headline size (a workspace of ~75 MB, most of the
    # array), then smaller ones of other shapes and modes
    big, dev = _big()
    _compare(big, f"{engine} config3 full size", dev=dev, oracle=False, **kw)
    _compare(A.config(3, small=True, seed=1), f"{engine} config3 small", **kw)
    _compare(A.config(5, small=True, seed=2), f"{engine} config5 small (int8, V skip)", **kw)
    _compare(A.config(2, seed=3), f"{engine} config2 full mode", eps_scale=0.0, eps_dir=0.0, **kw)
    _compare(A.config(1, seed=4), f"{engine} config1", **kw)


def test_noalloc_round_engine():
    # the round engine keeps every step's records: calls whose records fit the
    # static array run it, larger ones are refused (engine ROUND) or served by
    # the team engine (engine AUTO, see test_noalloc_matches_workspace_call)
    _compare(A.config(3, small=True, ctx=8192, seed=5), "round config3 ctx 8192", engine=6)
    _compare(A.config(3, small=True, seed=6), "round config3 small", engine=6)
    _compare(A.config(4, small=True, seed=7), "round config4 small", engine=6)


def test_noalloc_empty_batch_and_zero_lengths():
    import torch
    c = A.config(3, small=True, seed=5)
    c.ctx_lens[:] = 0
    _compare(c, "zero-length rows")
    import kv_cache_bandwidth_amd as art
    dev = to_device(c)
    # batch 0: nothing to do, nothing launched
    q0 = dev["q"][:0]
    out = torch.empty((0, c.Hq, c.d), dtype=torch.float32, device="cuda")
    used = torch.empty((0, c.Hq), dtype=torch.int32, device="cuda")
    art.decode_attention(q0, dev["k"], dev["v"], dev["ctx"][:0], block_table=dev["bt"][:0], tile=c.tile,
                         out=out, tiles_used=used, noalloc=True)
    torch.cuda.synchronize()


def test_noalloc_rejects_a_call_larger_than_its_scratch():
    import torch
    import kv_cache_bandwidth_amd as art
    from kv_cache_bandwidth_amd import _binding as B
    # 64 rows of 64K tokens (every block id 0 of a one-block pool): the
    # call's workspace exceeds the static array
    c = A.config(3, small=True, seed=6)
    dev = to_device(c)
    k = torch.zeros((1, c.Hkv, 16, c.d), dtype=dev["k"].dtype, device="cuda")
    bt = torch.zeros((64, 4096), dtype=torch.int32, device="cuda")
    ctx = torch.full((64,), 65536, dtype=torch.int32, device="cuda")
    q = torch.zeros((64, c.Hq, c.d), dtype=dev["q"].dtype, device="cuda")
    out = torch.empty((64, c.Hq, c.d), dtype=torch.float32, device="cuda")
    used = torch.empty((64, c.Hq), dtype=torch.int32, device="cuda")
    with pytest.raises(B.ArtError) as e:
        art.decode_attention(q, k, k, ctx, block_table=bt, tile=64, out=out, tiles_used=used, noalloc=True)
    assert e.value.status == -6 and "static scratch" in e.value.detail
    # the array still serves a call that fits
    _compare(A.config(2, small=True, seed=7), "after a refused call")
