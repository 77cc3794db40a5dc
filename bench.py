#!/usr/bin/env python3
"""Benchmark of ART-terminated decode attention on one MI355X.

A step is one art_decode_attention call (ART mode, thresholds 1e-3 / 1e-4,
patience 1) over the whole batch of the 32K-context Llama-3-8B-shaped workload
(batch 16, 32 query / 8 KV heads, head dim 128, bf16 paged KV cache with
16-token blocks under a seeded random block permutation, temperature giving the
top 5 % of keys ~90 % of the softmax mass), inputs resident in HBM.

Each timed step is bracketed by HIP events on the launch stream; between
steps (outside the events) a 1 GiB buffer is written so the 256 MB Infinity
Cache and the L2s hold none of the cache.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 3] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
# HBM bytes per launch of the dominant kernel, from hardware counters, by workload
TRAFFIC_FILES = {3: "traffic_art_team_kernel_ctx32k.txt", 5: "traffic_art_team_kernel_vskip_int8_ctx32k.txt"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def recorded_traffic(path, kernel_src):
    """HBM bytes per launch recorded from hardware counters (FETCH_SIZE and
    WRITE_SIZE, each scaled by its reading for a plain copy of known size), or
    None when the kernel source has changed since they were taken."""
    import hashlib
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        with open(kernel_src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("kernel_source_sha256") != sha:
            return None
        fetch = float(kv["fetch_kib_per_launch"]) / float(kv["fetch_copy_factor"])
        write = float(kv["write_kib_per_launch"]) / float(kv["write_copy_factor"])
        return int(round((fetch + write) * 1024))
    except (OSError, KeyError, ValueError):
        return None


def alg_bytes(case, used_g, kv_rows_loaded=None):
    """Bytes the method must move for one step (see the measurement notes):
    K and V rows of the tiles each group reads (V only where loaded when rows
    are skipped), their int8 scales, the block-table entries of those tiles,
    the queries, the outputs and tiles_used."""
    rows = np.minimum(used_g.astype(np.int64) * case.tile, case.ctx_lens[:, None].astype(np.int64))
    k_rows = int(rows.sum())
    # under the V skip the V rows loaded, capped at those of the needed tiles
    # (rows of tiles loaded past a stop are not the method's)
    v_rows = k_rows if kv_rows_loaded is None else min(int(kv_rows_loaded), k_rows)
    # bytes of one cache row (an int4 row holds d / 2 bytes) and its fp16 scale
    per_row = case.k.shape[-1] * case.k.dtype.itemsize + (2 if case.kv_dtype in ("i8", "i4") else 0)
    kv = (k_rows + v_rows) * per_row
    table = 0
    if case.block_size:
        table = int(np.ceil(rows / case.block_size).sum()) * 4
    q = case.q.nbytes
    out = case.B * case.Hq * case.d * 4 + case.B * case.Hq * 4
    return kv + table + q + out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-full", action="store_true", help="skip the full-attention comparison")
    ap.add_argument("--flush-mb", type=int, default=1024)
    ap.add_argument("--no-others", action="store_true",
                    help="skip the context timings of the other workloads (2, 4, 5)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (a known-size "
                         "reference for hardware byte counters) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the threshold / patience sweep (stops, error against full "
                         "attention, premature stops, time) on workloads 3, 4 and 3 with drifting "
                         "values, print one JSON line and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode-attention path is single-GPU "
              "(sharding across GPUs is a design note, not built). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    if args.sweep:
        print(json.dumps(threshold_sweep(args)), flush=True)
        return
    import art_inputs as A
    import kv_cache_bandwidth_amd as art
    from art_inputs import to_device

    log(f"generating workload config {args.config} (seed {args.seed})")
    t0 = time.time()
    case = A.config(args.config, seed=args.seed)
    log(f"generated in {time.time() - t0:.1f}s: {A.WORKLOADS[args.config]}")
    dev = to_device(case)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    flush_buf = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device="cuda")
    G = case.Hq // case.Hkv

    def call(eps_scale, eps_dir, v_skip, stats=None, ws=None, out=None, used=None):
        return art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], block_table=dev["bt"],
                                    tile=case.tile, eps_scale=eps_scale, eps_dir=eps_dir,
                                    patience=case.patience, v_skip_eps=v_skip, k_scale=dev["ks"],
                                    v_scale=dev["vs"], stats=stats, workspace=ws, out=out,
                                    tiles_used=used)

    def timed(eps_scale, eps_dir, v_skip, steps, warmup):
        out, used = call(eps_scale, eps_dir, v_skip)
        ws = torch.empty(art.workspace_bytes(_desc(eps_scale), case.tile), dtype=torch.uint8,
                         device="cuda")
        for _ in range(warmup):
            flush_buf.fill_(1)
            call(eps_scale, eps_dir, v_skip, ws=ws, out=out, used=used)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t_wall = time.perf_counter()
        for e0, e1 in evs:
            flush_buf.fill_(1)
            e0.record(stream)
            call(eps_scale, eps_dir, v_skip, ws=ws, out=out, used=used)
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        return ms, wall, out, used

    def _desc(eps):
        # sizes only: the scale pointers just have to be non-null (nothing is read)
        scaled = case.kv_dtype in ("i8", "i4")
        return art.make_desc(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                             head_dim=case.d, q_dtype=1 if case.q_dtype == "bf16" else 0,
                             kv_dtype={"f32": 0, "bf16": 1, "i8": 2, "i4": 3}[case.kv_dtype],
                             k_scale=1 if scaled else 0, v_scale=1 if scaled else 0,
                             block_size=case.block_size,
                             max_blocks_per_seq=case.block_table.shape[1] if case.block_size else 0,
                             num_blocks=case.num_blocks,
                             max_ctx=0 if case.block_size else case.max_ctx,
                             patience=case.patience)

    es, ed, vk = case.eps_scale, case.eps_dir, case.v_skip_eps
    # counters of one ART call: tiles loaded (speculative ones included), V rows loaded
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    out, used = call(es, ed, vk, stats=stats)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    used_np = used.cpu().numpy()
    log(f"ART call: mean tiles_used {used_np.mean():.1f}, tiles loaded {int(st[0])}")

    log(f"timing ART mode: {args.warmup} warmup + {args.steps} steps")
    ms, wall, out, used = timed(es, ed, vk, args.steps, args.warmup)
    used_np = used.cpu().numpy()
    used_g = used_np.reshape(case.B, case.Hkv, G).max(axis=-1)
    nt = -(-case.ctx_lens // case.tile)
    mean_ms = statistics.mean(ms)
    med_ms = statistics.median(ms)
    b_alg = alg_bytes(case, used_g, kv_rows_loaded=int(st[1]) if vk > 0 else None)
    achieved = b_alg / (mean_ms * 1e-3) / 1e9
    head_skip = 1.0 - used_np.sum() / (nt[:, None] * case.Hq).sum()
    kv_read = np.minimum(used_g * case.tile, case.ctx_lens[:, None]).sum()
    byte_skip = 1.0 - kv_read / (case.ctx_lens.astype(np.int64).sum() * case.Hkv)
    tiles_needed = int(np.ceil(np.minimum(used_g * case.tile, case.ctx_lens[:, None]) / case.tile).sum())
    res = {
        "metric": "decode-attn us/step (ART, 32K ctx) + achieved HBM GB/s, roofline %, % KV tiles skipped",
        "value": round(mean_ms * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.kv_dtype,
        "data": "synthetic",
        "config": {"workload": A.WORKLOADS[args.config], "batch": case.B, "q_heads": case.Hq,
                   "kv_heads": case.Hkv, "head_dim": case.d, "ctx": int(case.ctx_lens[0]),
                   "tile": case.tile, "eps_scale": es, "eps_dir": ed, "patience": case.patience,
                   "v_skip_eps": vk},
        "us_per_step_median": round(med_ms * 1e3, 2),
        "us_per_step_p10_p90": [round(float(np.percentile(ms, 10)) * 1e3, 2),
                                round(float(np.percentile(ms, 90)) * 1e3, 2)],
        "kv_tiles_skipped_head_level": round(float(head_skip), 4),
        "kv_bytes_skipped": round(float(byte_skip), 4),
        "tiles_loaded": int(st[0]),
        "tiles_needed": tiles_needed,
        "speculative_tiles": int(st[0]) - tiles_needed,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(
                         os.path.join(ROOT, "profiles", TRAFFIC_FILES[args.config]),
                         os.path.join(ROOT, "kv_cache_bandwidth_amd", "csrc", "art_kernels.hip"))
                     if args.config in TRAFFIC_FILES else None,
                     "alg_bytes_per_step": int(b_alg)},
        "wall_s_timed_region": round(wall, 4),
    }

    if not args.no_full:
        log("timing full attention (thresholds 0)")
        ms_f, _, out_f, used_f = timed(0.0, 0.0, 0.0, args.steps, args.warmup)
        mf = statistics.mean(ms_f)
        b_full = alg_bytes(case, np.broadcast_to(nt[:, None], used_g.shape))
        res["full_attention"] = {"us_per_step": round(mf * 1e3, 2),
                                 "achieved_GBs": round(b_full / (mf * 1e-3) / 1e9, 1),
                                 "frac": round(b_full / (mf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        res["speedup_vs_full"] = round(mf / mean_ms, 3)
        # detector overhead: the ART path with thresholds that never pass
        ms_n, _, _, _ = timed(1e-30, 1e-30, 0.0, max(5, args.steps // 2), 2)
        res["never_firing_art_us_per_step"] = round(statistics.mean(ms_n) * 1e3, 2)

    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        log(f"CPU oracle baseline on {threads} threads")
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            r = oracle.decode(case.q, case.k, case.v, case.ctx_lens, tile=case.tile, eps_scale=es,
                              eps_dir=ed, patience=case.patience, v_skip_eps=vk,
                              block_table=case.block_table, block_size=case.block_size,
                              k_scale=case.k_scale, v_scale=case.v_scale, threads=threads)
            times.append(time.perf_counter() - t0)
        cpu_us = statistics.median(times) * 1e6
        res["cpu_baseline"] = {"value": round(cpu_us, 1), "unit": "us/step", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole step ({case.B} rows x {case.Hq} heads), fp64, "
                                         f"median of 3 on {platform.processor() or platform.machine()}"}
        res["parity_vs_oracle"] = {
            "tiles_used_equal": int((used.cpu().numpy() == r.tiles_used).sum()),
            "heads": int(r.tiles_used.size),
            "max_abs_out": float(np.abs(out.cpu().numpy().astype(np.float64) - r.out).max())}
    if not args.no_others:
        res["tile_orders"] = tile_orders(case, dev, flush_buf)
        res["per_head_retention"] = per_head_retention(case, flush_buf)
        res["vskip_bf16"] = vskip_bf16(case, dev, flush_buf)
        res["other_workloads"] = other_workloads(args, flush_buf)
    print(json.dumps(res), flush=True)


def _median_call(dev, a, flush_buf, steps):
    import torch
    import kv_cache_bandwidth_amd as art
    stream = torch.cuda.current_stream()
    out, used = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], **a)
    ms = []
    for _ in range(steps + 2):
        flush_buf.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], out=out, tiles_used=used, **a)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return statistics.median(ms[2:]) * 1e3, used.cpu().numpy()


def per_head_retention(case, flush_buf, steps=7):
    """Context, not the metric: ART on top of per-head block tables -- each KV
    head keeps its row's first 4 blocks, the last 512 (8K tokens) and a random
    quarter of the blocks between, drawn per head -- against full attention
    over the same retained tables (median us per call)."""
    import art_inputs as A
    from art_inputs import to_device
    log("context timing: per-head retention tables")
    kept = A.retained_tables(case, sink_blocks=4, recent_blocks=512, keep_frac=0.25, seed=1)
    dev = to_device(kept)
    a = dict(block_table=dev["bt"], tile=kept.tile, eps_scale=kept.eps_scale, eps_dir=kept.eps_dir,
             patience=kept.patience, v_skip_eps=kept.v_skip_eps, k_scale=dev["ks"], v_scale=dev["vs"],
             per_head_tables=True)
    t_art, used = _median_call(dev, a, flush_buf, steps)
    t_full, _ = _median_call(dev, dict(a, eps_scale=0.0, eps_dir=0.0), flush_buf, steps)
    G = kept.Hq // kept.Hkv
    nt = -(-kept.ctx_lens // kept.tile)
    return {"policy": "per KV head: first 4 + last 512 blocks of 16, a random 25% of the rest",
            "kept_tokens_share": round(float(kept.ctx_lens.sum() / (case.ctx_lens.sum() * case.Hkv)), 4),
            "art_us": round(t_art, 1), "full_us": round(t_full, 1),
            "kv_tiles_skipped_head_level": round(float(1.0 - used.sum() / (np.repeat(nt, G, axis=1)).sum()), 4)}


SWEEP_SCALE = (1e-4, 1e-3, 1e-2)
SWEEP_DIR = (1e-5, 1e-4, 1e-3)
SWEEP_PATIENCE = (1, 2, 4)


def threshold_sweep(args, steps=5):
    """The stop rule against its parameters (ART summary, sections 2.2-2.3):
    for every (eps_scale, eps_dir, patience) of the grid, on workload 3, on
    workload 4 (rows of large value at low weight) and on workload 3 with
    values drifting around a common mean: the share of (head, tile) pairs
    skipped, the error of each head's output against full attention (relative
    L2), the share of stopped heads whose error exceeds 1e-2 and 1e-3
    (premature stops), and the median time per call."""
    import torch
    import art_inputs as A
    import kv_cache_bandwidth_amd as art
    from art_inputs import to_device
    flush_buf = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device="cuda")
    res = {"grid": {"eps_scale": SWEEP_SCALE, "eps_dir": SWEEP_DIR, "patience": SWEEP_PATIENCE},
           "workloads": {}}
    for name, case in (("workload3", lambda: A.config(3, seed=args.seed)),
                       ("workload4", lambda: A.config(4, seed=args.seed)),
                       ("workload3_drift", lambda: A.config(3, seed=args.seed, v_mean=3.0))):
        log(f"sweep: generating {name}")
        case = case()
        dev = to_device(case)
        base = dict(block_table=dev["bt"], tile=case.tile, v_skip_eps=0.0, k_scale=dev["ks"],
                    v_scale=dev["vs"])
        full, _ = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], eps_scale=0.0,
                                       eps_dir=0.0, **base)
        full = full.double()
        fn = full.norm(dim=-1)
        nt = torch.from_numpy(-(-case.ctx_lens // case.tile)).cuda()[:, None]
        rows = []
        for es in SWEEP_SCALE:
            for ed in SWEEP_DIR:
                for p in SWEEP_PATIENCE:
                    a = dict(base, eps_scale=es, eps_dir=ed, patience=p)
                    out, used = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], **a)
                    err = (out.double() - full).norm(dim=-1) / fn
                    stopped = used < nt
                    ns = int(stopped.sum())
                    t, _ = _median_call(dev, a, flush_buf, steps)
                    rows.append({"eps_scale": es, "eps_dir": ed, "patience": p,
                                 "skipped": round(1.0 - float(used.sum()) / float((nt * case.Hq).sum()), 4),
                                 "err_max": float(err.max()), "err_mean": float(err.mean()),
                                 "premature_1e-2": round(float((stopped & (err > 1e-2)).sum()) / max(1, ns), 4),
                                 "premature_1e-3": round(float((stopped & (err > 1e-3)).sum()) / max(1, ns), 4),
                                 "us": round(t, 1)})
        res["workloads"][name] = {"workload": A.WORKLOADS[3 if "3" in name else 4]
                                  + (", values N(3, 1)" if "drift" in name else ""), "rows": rows}
        del dev
    return res


def vskip_bf16(case, dev, flush_buf, steps=7):
    """Context, not the metric: the V skip on this bf16 workload (same
    thresholds), median us per call and the share of (query head, V row)
    pairs of the tiles read that were skipped."""
    import torch
    res = {}
    for eps in (1e-6, 1e-4):
        log(f"context timing: V skip {eps:g} on bf16")
        a = dict(block_table=dev["bt"], tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                 patience=case.patience, v_skip_eps=eps, k_scale=dev["ks"], v_scale=dev["vs"])
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        import kv_cache_bandwidth_amd as art
        art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], stats=stats, **a)
        torch.cuda.synchronize()
        st = stats.cpu().numpy()
        t, _ = _median_call(dev, a, flush_buf, steps)
        G = case.Hq // case.Hkv
        res[f"eps_{eps:g}"] = {"art_us": round(t, 1),
                               "pairs_skipped_share": round(float(st[3]) / max(1.0, float(st[0]) * case.tile * G), 4)}
    return res


def tile_orders(case, dev, flush_buf, steps=7):
    """Context, not the metric: the same workload and thresholds with the tiles
    visited sink first then most recent first, and in a random sink-first list
    (median us per call, head-level share of tiles skipped)."""
    import torch
    import art_inputs as A
    import kv_cache_bandwidth_amd as art
    stream = torch.cuda.current_stream()
    stride = -(-case.max_ctx // case.tile)
    perm = torch.from_numpy(A.sink_first_orders(case.ctx_lens, case.tile, stride=stride, seed=1)).cuda()
    nt = -(-case.ctx_lens // case.tile)
    res = {}
    for name, kw in (("recent_first", dict(tile_order=art.ORDER_RECENT)),
                     ("random_list", dict(tile_order=art.ORDER_LIST, tile_perm=perm))):
        log(f"context timing: tile order {name}")
        a = dict(block_table=dev["bt"], tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                 patience=case.patience, v_skip_eps=case.v_skip_eps, k_scale=dev["ks"], v_scale=dev["vs"],
                 **kw)
        out, used = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], **a)
        ms = []
        for _ in range(steps + 2):
            flush_buf.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], out=out, tiles_used=used, **a)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        u = used.cpu().numpy()
        res[name] = {"art_us": round(statistics.median(ms[2:]) * 1e3, 1),
                     "kv_tiles_skipped_head_level": round(float(1.0 - u.sum() / (nt[:, None] * case.Hq).sum()), 4)}
    return res


def other_workloads(args, flush_buf, steps=7):
    """Context, not the metric: ART (library default engine, each workload's
    own thresholds and V-skip setting) and full attention on workloads 2, 4
    and 5 at full size, and workload 5 with an int4 cache, median µs per
    call, same timing method."""
    import torch
    import art_inputs as A
    import kv_cache_bandwidth_amd as art
    from art_inputs import to_device
    stream = torch.cuda.current_stream()
    res = {}
    for n in (2, 4, 5, "5i4"):
        if n == args.config:
            continue
        log(f"context timing: workload {n}")
        case = A.config(5, seed=args.seed, kv_dtype="i4") if n == "5i4" else A.config(n, seed=args.seed)
        dev = to_device(case)

        rows_loaded, tiles_loaded = {}, {}

        def med(**kw):
            a = dict(block_table=dev["bt"], tile=case.tile, eps_scale=case.eps_scale, eps_dir=case.eps_dir,
                     patience=case.patience, v_skip_eps=case.v_skip_eps, k_scale=dev["ks"], v_scale=dev["vs"])
            a.update(kw)
            # one counting call first: V rows loaded, for the algorithmic bytes under the V skip
            stats = torch.zeros(4, dtype=torch.int64, device="cuda")
            out, used = art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], stats=stats, **a)
            torch.cuda.synchronize()
            rows_loaded[a["v_skip_eps"]] = int(stats[1])
            tiles_loaded[a["v_skip_eps"]] = int(stats[0])
            ms = []
            for _ in range(steps + 2):
                flush_buf.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                art.decode_attention(dev["q"], dev["k"], dev["v"], dev["ctx"], out=out, tiles_used=used, **a)
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            return statistics.median(ms[2:]) * 1e3, used.cpu().numpy()

        def roof(us, used_heads, vskip):
            # algorithmic bytes of the call (its own tiles_used; with the V skip
            # the V rows it loaded) over its median time, against HBM peak
            G = case.Hq // case.Hkv
            used_g = used_heads.reshape(case.B, case.Hkv, G).max(axis=-1)
            b = alg_bytes(case, used_g, kv_rows_loaded=rows_loaded[vskip] if vskip > 0 else None)
            gbs = b / (us * 1e-6) / 1e9
            return {"alg_bytes": int(b), "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}

        t_art, used = med()
        t_full, used_full = med(eps_scale=0.0, eps_dir=0.0, v_skip_eps=0.0)
        nt = -(-case.ctx_lens // case.tile)
        name = A.WORKLOADS[5].replace("int8", "int4 (two codes per byte)") if n == "5i4" else A.WORKLOADS[n]
        entry = {"workload": name, "art_us": round(t_art, 1), "full_us": round(t_full, 1),
                 "kv_tiles_skipped_head_level": round(float(1.0 - used.sum() / (nt[:, None] * case.Hq).sum()), 4),
                 "art_roofline": roof(t_art, used, case.v_skip_eps),
                 "full_roofline": roof(t_full, used_full, 0.0)}
        # detector overhead (thresholds that never pass, no V skip) and ART
        # without the V skip on each engine (the default engine picks one of them)
        entry["never_firing_art_us"] = round(med(eps_scale=1e-30, eps_dir=1e-30, v_skip_eps=0.0)[0], 1)
        entry["art_no_vskip_us_by_engine"] = {
            name: round(med(v_skip_eps=0.0, engine=e)[0], 1)
            for name, e in (("team", 1), ("pool", 2), ("round", 6))}
        if case.v_skip_eps > 0:
            t_nv, used_nv = med(v_skip_eps=0.0)
            entry["art_no_vskip_us"] = round(t_nv, 1)
            entry["art_no_vskip_roofline"] = roof(t_nv, used_nv, 0.0)
            # V rows loaded over the rows of the K tiles loaded, in the V-skip call
            entry["v_rows_loaded_share"] = round(
                rows_loaded[case.v_skip_eps] / max(1, tiles_loaded[case.v_skip_eps] * case.tile), 4)
        res[f"workload{n}"] = entry
        del dev
    return res


if __name__ == "__main__":
    main()
