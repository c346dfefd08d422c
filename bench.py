"""Benchmark: Skip-Softmax attention on one MI355X.

A step is one Skip-Softmax prefill over the 16K-token Llama-3.1-8B attention
shape (B=1, Hq=32, Hkv=8, d=128, L=16384, causal, Br=128, Bc=64) with the
threshold calibrated so that about half of the causal tiles are skipped.
The headline value is dense-equivalent TFLOP/s (4 d B Hq L(L+1)/2 per step
over the step time). The JSON line also carries the roofline of the prefill
kernel (bf16 MFMA, executed FLOPs), a CPU baseline (the fp64 oracle on a
bounded sample of the same workload), and -- under "extra" -- the 128K
threshold sweep, the decode tokens/s with HBM roofline and the block-sparse
prefill.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 200] [--no-extra]
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(files=("common.h", "launch.h", "prefill.hip")) -> str:
    """Hash of the code the prefill kernel is built from (the counters in
    profiles/ are valid only for this exact kernel). Comments and runs of
    white space are dropped first, so an edit that cannot change the
    compiled kernel keeps the hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_long_skip_amd", "csrc")
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(f.encode() + text.encode())
    return h.hexdigest()[:16]


def load_traffic(name: str, per_launch_units: float):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        c = json.load(open(path))
    except Exception:
        return None
    if c.get("source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def dev_bf16(bits, torch, np):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# The GPU clock ramps up over the first few hundred milliseconds of load (the
# 16K prefill launch takes 1.63 ms after 5 warm-up launches, 1.60 after 50 and
# 1.59 after 200 on one box), so every timed region follows at least this much
# back-to-back work.
WARM_S = 0.3


def time_launches(fn, steps, warmup, torch, warm_s=WARM_S):
    """Warm up (`warmup` calls, then further batches of calls until `warm_s`
    seconds of them have run), then time `steps` calls: wall clock between
    synchronisations and HIP events around each call (on the current stream,
    where the library launches). Returns (ms per step, mean event ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [a.elapsed_time(b) for a, b in evs]
    return (t1 - t0) * 1e3 / steps, sum(ev) / len(ev)


def prefill_work(state, Br, Bc, d):
    """(visited, kept, executed FLOPs) from the per-tile decisions."""
    vis = int((state != 0).sum())
    kept = int((state == 1).sum())
    return vis, kept, 2.0 * Br * Bc * d * (vis + kept)


def visited_tiles_count(B, Hq, L, Br, Bc, causal, block_idx=None, block_cnt=None):
    """Key tiles the prefill visits, summed over all decision units: every
    tile up to the causal limit of the query tile (dense), or the list entries
    that are in range and within the causal limit (block list). Host
    arrays."""
    import numpy as np
    nQ, nK = -(-L // Br), -(-L // Bc)
    last_row = np.minimum((np.arange(nQ) + 1) * Br, L) - 1
    if block_idx is None:
        per = (last_row // Bc + 1) if causal else np.full(nQ, nK)
        return int(per.sum()) * B * Hq
    idx = np.asarray(block_idx)
    cnt = np.clip(np.asarray(block_cnt), 0, idx.shape[-1])
    pos = np.arange(idx.shape[-1])
    ok = (pos < cnt[..., None]) & (idx >= 0) & (idx < nK)
    if causal:
        ok &= idx * Bc <= last_row[None, None, :, None]
    return int(ok.sum())


def decode_loaded_bytes(lens, B, Hq, Hkv, d, Bc, T, kept_tiles):
    """Algorithmic HBM bytes of one split-K decode call: K of every valid key
    (bf16), V of every kept tile (bf16, a ragged last tile counted whole, as
    its rows are read), q read and out written (bf16), lse written (fp32),
    and the split partials -- d + 2 fp32 per (sequence, query head, split) --
    written by the split kernel and read by the combine kernel."""
    def ceil_div(a, b):
        return -(-a // b)
    lens = [max(int(n), 0) for n in lens]
    k_bytes = 2 * d * Hkv * sum(lens)
    v_bytes = 2 * d * Bc * int(kept_tiles)
    io = 2 * (2 * B * Hq * d) + 4 * B * Hq
    splits = sum(ceil_div(ceil_div(n, Bc), T) for n in lens)
    ws = 2 * 4 * Hq * splits * (d + 2)
    return k_bytes + v_bytes + io + ws


def bench_prefill(cfg_id, args, torch, np, ssa, synth, lam=None, target=None, seed=0):
    from sparse_attention_long_skip_amd.calibrate import calibrate_prefill
    c = synth.CONFIGS[cfg_id]
    x = synth.prefill_inputs(cfg_id, seed, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"],
                             block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    res = {"q": q, "k": k, "v": v, "cfg": c}
    if lam is None:
        lam, ratio = calibrate_prefill(q, k, v, target, c["Br"], c["Bc"], c["causal"])
        res["calibrated_ratio"] = ratio
    res["lam"] = lam
    return res


def time_calibration(p, target, torch, ssa):
    """Device threshold calibration of a prefill workload: the dense
    statistics launch that writes the tile margins, and the quantile over
    them (``ssa_lambda_for_ratio``), timed separately."""
    c = p["cfg"]
    q, k, v = p["q"], p["k"], p["v"]
    B, Hq, L, d = q.shape
    out = torch.empty_like(q)
    kw = dict(Br=c["Br"], Bc=c["Bc"], causal=c["causal"], lse=False, out=out)
    ms_m, ev_m = time_launches(lambda: ssa.prefill(q, k, v, -math.inf, margins=True, **kw), 3, 1, torch)
    mm = ssa.prefill(q, k, v, -math.inf, margins=True, **kw)["tile_margin"]
    ws = torch.empty(ssa.calibrate_workspace_size(mm.numel()), dtype=torch.uint8, device=q.device)
    r = torch.empty(4, dtype=torch.float64, device=q.device)
    ms_q, ev_q = time_launches(lambda: ssa.lambda_for_ratio(mm, target, workspace=ws, result=r, sync=False),
                               10, 3, torch)
    return {"margins": int(mm.numel()), "visited": int(r[2].item()), "lambda": float(r[0].item()),
            "ratio": round(float(r[1].item()), 5), "margin_launch_ms": round(ev_m, 4),
            "quantile_ms": round(ms_q, 4), "quantile_event_ms": round(ev_q, 4)}


def run_prefill(p, lam, steps, warmup, torch, ssa, check_stats=True, warm_s=WARM_S):
    """Time the plain prefill instance (out, lse and per-unit skip counts).
    The kept-tile count comes from the skip counts of the last timed launch;
    with ``check_stats`` a statistics launch (per-tile decisions) beforehand
    must agree with it. Returns (visited, kept, ms per step, event ms)."""
    c = p["cfg"]
    q, k, v = p["q"], p["k"], p["v"]
    B, Hq, L, d = q.shape
    out = torch.empty_like(q)
    counts = torch.empty((B, Hq, -(-L // c["Br"])), dtype=torch.int32, device=q.device)
    fn = lambda: ssa.prefill(q, k, v, lam, Br=c["Br"], Bc=c["Bc"], causal=c["causal"], out=out,
                             skip_counts=counts)
    ms, ev_ms = time_launches(fn, steps, warmup, torch, warm_s)
    vis = visited_tiles_count(B, Hq, L, c["Br"], c["Bc"], c["causal"])
    kept = vis - int(counts.sum().item())
    if check_stats:
        st = ssa.prefill(q, k, v, lam, Br=c["Br"], Bc=c["Bc"], causal=c["causal"], stats=True, lse=False)
        torch.cuda.synchronize()
        s_vis, s_kept, _ = prefill_work(st["tile_state"].cpu().numpy(), c["Br"], c["Bc"], d)
        if (s_vis, s_kept) != (vis, kept):
            raise RuntimeError(f"timed launch counts ({vis}, {kept}) differ from the statistics launch "
                               f"({s_vis}, {s_kept})")
        del st
    return vis, kept, ms, ev_ms


def time_prefill_legs(q, k, v, lam, kw, steps, warmup, torch, ssa):
    """Time the plain prefill instance with keyword arguments ``kw`` (tile
    sizes, causal, block list or N:M). Kept tiles come from the timed
    launches' own skip counts; a statistics launch must agree. Returns
    (visited, kept, ms per step, event ms)."""
    B, Hq, L, d = q.shape
    Br = kw["Br"]
    out = torch.empty_like(q)
    counts = torch.empty((B, Hq, -(-L // Br)), dtype=torch.int32, device=q.device)
    ms, ev = time_launches(lambda: ssa.prefill(q, k, v, lam, out=out, skip_counts=counts, **kw),
                           steps, warmup, torch)
    bi, bc = kw.get("block_idx"), kw.get("block_cnt")
    vis = visited_tiles_count(B, Hq, L, Br, kw["Bc"], kw["causal"],
                              None if bi is None else bi.cpu().numpy(),
                              None if bc is None else bc.cpu().numpy())
    kept = vis - int(counts.sum().item())
    st = ssa.prefill(q, k, v, lam, stats=True, lse=False, **kw)
    torch.cuda.synchronize()
    s_vis, s_kept, _ = prefill_work(st["tile_state"].cpu().numpy(), Br, kw["Bc"], d)
    if (s_vis, s_kept) != (vis, kept):
        raise RuntimeError(f"timed launch counts ({vis}, {kept}) differ from the statistics launch "
                           f"({s_vis}, {s_kept})")
    return vis, kept, ms, ev


def dense_flops(c):
    L = c["L"]
    return 4.0 * c["d"] * c["B"] * c["Hq"] * L * (L + 1) / 2


# ---- CPU baseline: the fp64 oracle, in parallel worker processes ----------
#
# One process per core of this process's affinity set (at most 16), each with
# single-threaded BLAS; every task is one decision unit (or one head) of the
# same seeded workload, read from memory-mapped copies of the inputs. Tasks
# run until the wall-clock budget is spent; the rate counts finished tasks.

CPU_WORKERS_MAX = 16
_W = {}


def cpu_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(CPU_WORKERS_MAX, n))


def _worker_init(paths):
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    for name, path in paths.items():
        _W[name] = np.load(path, mmap_mode="r")


def _noop(x):
    return x


def _prefill_unit_task(args):
    import oracle
    unit, lam, Br, Bc, causal, nm_kw = args
    oracle.prefill(_W["q"], _W["k"], _W["v"], lam, Br, Bc, causal, units=[unit], bits=True, **nm_kw)
    return unit


def _decode_unit_task(args):
    import oracle
    unit, lam, Bc, T = args
    oracle.decode(_W["q"], _W["k_cache"], _W["v_cache"], _W["seqlens"], lam, Bc, T, units=[unit],
                  bits=True)
    return unit


def _sparse_head_task(args):
    """Block mask of one head, then the block-sparse prefill of its query
    blocks; returns the two times."""
    import oracle
    h, lam, pool, topk, sink, window = args
    q = _W["q"][:, h:h + 1]
    k = _W["k"][:, h:h + 1]
    t0 = time.perf_counter()
    m = oracle.block_mask(q, k, pool, topk, sink, window, bits=True)
    t1 = time.perf_counter()
    oracle.prefill(q, k, _W["v"][:, h:h + 1], lam, pool, pool, True, block_idx=m["block_idx"],
                   block_cnt=m["block_cnt"], bits=True)
    return h, t1 - t0, time.perf_counter() - t1


def _masked_head_task(args):
    """One head: the oracle's mask predictor (SpargeAttn stage one or
    vertical-slash), then the block-sparse prefill over its lists."""
    import oracle
    h, kind, mkw, lam, pool = args
    q = _W["q"][:, h:h + 1]
    k = _W["k"][:, h:h + 1]
    if kind == "sparge":
        m = oracle.sparge_mask(q, k, pool, mkw["theta"], mkw["tau"], "mass", bits=True)
    else:
        m = oracle.vertical_slash_mask(q, k, mkw["last_q"], mkw["n_vertical"], mkw["n_slash"], pool, bits=True)
    oracle.prefill(q, k, _W["v"][:, h:h + 1], lam, pool, pool, True, block_idx=m["block_idx"],
                   block_cnt=m["block_cnt"], bits=True)
    return h


def run_cpu_pool(arrays: dict, fn, tasks, budget_s: float):
    """Run ``fn`` over ``tasks`` in worker processes: every worker is kept
    busy until the budget is spent, then the tasks in flight finish and
    count (so a task longer than the budget is not lost). Returns (finished
    task results, wall seconds, workers)."""
    import multiprocessing as mp
    import queue
    import shutil
    import tempfile
    import numpy as np
    tmp = tempfile.mkdtemp(prefix="ssa_oracle_")
    try:
        paths = {}
        for name, a in arrays.items():
            paths[name] = os.path.join(tmp, name + ".npy")
            np.save(paths[name], np.ascontiguousarray(a))
        nw = cpu_workers()
        ctx = mp.get_context("spawn")
        with ctx.Pool(nw, initializer=_worker_init, initargs=(paths,)) as pool:
            pool.map(_noop, range(4 * nw))
            finished = queue.Queue()
            todo = iter(tasks)

            def submit():
                t = next(todo, None)
                if t is None:
                    return False
                pool.apply_async(fn, (t,), callback=finished.put, error_callback=finished.put)
                return True

            done = []
            t0 = time.perf_counter()
            in_flight = sum(1 for _ in range(nw) if submit())
            while in_flight:
                r = finished.get()
                in_flight -= 1
                if isinstance(r, BaseException):
                    raise r
                done.append(r)
                if time.perf_counter() - t0 <= budget_s and submit():
                    in_flight += 1
            dt = time.perf_counter() - t0
        return done, dt, nw
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def cpu_baseline_prefill(cfg_id, lam, budget_s, np, synth, label, Br=None, nm_kw=None):
    """The oracle on the decision units (query tiles of Br rows) of a prefill
    workload, in a seeded random order (the whole workload if the budget
    allows); ``nm_kw`` adds N:M sparse softmax."""
    c = synth.CONFIGS[cfg_id]
    Br = Br or c["Br"]
    x = synth.prefill_inputs(cfg_id, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"],
                             frac=c["frac"])
    nQ = math.ceil(c["L"] / Br)
    units = [(b, h, i) for b in range(c["B"]) for h in range(c["Hq"]) for i in range(nQ)]
    # the first and last query tile of every head always, the rest in a seeded random order
    ends = [j for j, u in enumerate(units) if u[2] in (0, nQ - 1)]
    rest = np.random.default_rng(1234).permutation([j for j, u in enumerate(units) if u[2] not in (0, nQ - 1)])
    tasks = [(units[j], lam, Br, c["Bc"], c["causal"], nm_kw or {}) for j in [*ends, *rest]]
    done, dt, nw = run_cpu_pool({"q": x["q"], "k": x["k"], "v": x["v"]}, _prefill_unit_task, tasks, budget_s)
    flops = 0.0
    for (_, _, i) in done:
        r0, r1 = i * Br, min(c["L"], (i + 1) * Br)
        # dense-equivalent work of these rows: 4 d per allowed (row, key) pair
        flops += 4.0 * c["d"] * (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2
    full = 4.0 * c["d"] * c["B"] * c["Hq"] * c["L"] * (c["L"] + 1) / 2
    return {"value": flops / dt / 1e12, "unit": "dense-equiv TFLOP/s", "cores": nw, "kind": "oracle",
            "sample": f"{len(done)} of {len(units)} {Br}-row query tiles (the first and last of every head, "
                      f"the rest in random order) of the {label} workload, fp64 numpy, one process per core, "
                      f"{dt:.1f} s ({flops / full:.1%} of the work; the whole workload at this rate: "
                      f"{full / (flops / dt):.3g} s)"}


def cpu_baseline_masked(x, c, kind, mkw, budget_s, label):
    """The oracle's mask predictor and block-sparse prefill, one task per head."""
    tasks = [(h, kind, mkw, c["lam"], c["pool"] if "pool" in c else 64) for h in range(c["Hq"])]
    done, dt, nw = run_cpu_pool({"q": x["q"], "k": x["k"], "v": x["v"]}, _masked_head_task, tasks, budget_s)
    flops = 4.0 * c["d"] * c["L"] * (c["L"] + 1) / 2 * len(done)
    return {"value": flops / dt / 1e12, "unit": "dense-equiv TFLOP/s", "cores": nw, "kind": "oracle",
            "sample": f"{len(done)} of {c['Hq']} heads (mask + block-sparse prefill) of the {label} "
                      f"workload, fp64 numpy, one process per core, {dt:.1f} s"}


def with_cpu(res, args, what, fn):
    """Attach a CPU baseline to a leg's result unless --no-cpu; an error is
    reported in place of the figure."""
    if args.no_cpu:
        return res
    log(f"cpu baseline: oracle on {what}")
    try:
        res["cpu_baseline"] = fn()
    except Exception as e:  # report, keep the GPU figures
        res["cpu_baseline"] = {"error": repr(e)}
    return res


def cpu_baseline_decode(y, c, lam, budget_s, np):
    """The oracle on (sequence, KV head) units of the decode workload;
    tokens/s = finished units / Hkv per second."""
    B, Hkv = c["B"], c["Hkv"]
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    order = np.random.default_rng(1235).permutation(len(units))
    tasks = [(units[j], lam, c["Bc"], c["split_tiles"]) for j in order]
    arrays = {"q": y["q"], "k_cache": y["k_cache"], "v_cache": y["v_cache"], "seqlens": y["seqlens"]}
    done, dt, nw = run_cpu_pool(arrays, _decode_unit_task, tasks, budget_s)
    return {"value": len(done) / Hkv / dt, "unit": "tokens/s", "cores": nw, "kind": "oracle",
            "sample": f"{len(done)} of {len(units)} (sequence, KV head) units (random order) of the "
                      f"decode workload, fp64 numpy, one process per core, {dt:.1f} s"}


def cpu_baseline_sparse(x, c, budget_s, np):
    """The oracle's block mask and block-sparse prefill, one task per head."""
    tasks = [(h, c["lam"], c["pool"], c["topk"], c["sink_blocks"], c["window_tokens"]) for h in range(c["Hq"])]
    done, dt, nw = run_cpu_pool({"q": x["q"], "k": x["k"], "v": x["v"]}, _sparse_head_task, tasks, budget_s)
    flops = 4.0 * c["d"] * c["L"] * (c["L"] + 1) / 2 * len(done)
    return {"value": flops / dt / 1e12, "unit": "dense-equiv TFLOP/s", "cores": nw, "kind": "oracle",
            "sample": f"{len(done)} of {c['Hq']} heads (mask + block-sparse prefill) of the 32K block-sparse "
                      f"workload, fp64 numpy, one process per core, {dt:.1f} s"}


def extra_128k(args, torch, np, ssa, synth):
    p = bench_prefill(3, args, torch, np, ssa, synth, lam=-math.inf)
    c = p["cfg"]
    rows = []
    for lam in c["lam_sweep"]:
        vis, kept, ms, ev = run_prefill(p, lam, 3, 1, torch, ssa, check_stats=False)
        ex = 2.0 * c["Br"] * c["Bc"] * c["d"] * (vis + kept)
        rows.append({"lambda": lam, "ms": round(ms, 3), "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                     "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "skip_pct": round(100.0 * (vis - kept) / vis, 3)})
    # also at a calibrated ~50% point
    cal = time_calibration(p, 0.5, torch, ssa)
    lam50 = cal["lambda"]
    vis, kept, ms, ev = run_prefill(p, lam50, 3, 1, torch, ssa, check_stats=False)
    ex = 2.0 * c["Br"] * c["Bc"] * c["d"] * (vis + kept)
    rows.append({"lambda": round(lam50, 5), "label": "calibrated ~50% (extra point)", "ms": round(ms, 3),
                 "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                 "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "skip_pct": round(100.0 * (vis - kept) / vis, 3)})
    del p
    torch.cuda.empty_cache()
    res = {"workload": "prefill 128K B=1 Hq=8 Hkv=1 d=128 causal Br=128 Bc=64, 5% planted", "sweep": rows,
           "calibration": cal}
    # the oracle at the first sweep point, on a random sample of the query tiles
    return with_cpu(res, args, "a sample of the 128K workload",
                    lambda: cpu_baseline_prefill(3, c["lam_sweep"][0], args.cpu_budget / 2, np, synth, "128K"))


def extra_decode(args, torch, np, ssa, synth):
    from sparse_attention_long_skip_amd.calibrate import calibrate_decode
    c = synth.CONFIGS[2]
    y = synth.decode_inputs(2, 0, c["B"], c["Hq"], c["Hkv"], c["S_max"], c["d"], c["len_lo"],
                            c["len_hi"], block=c["Bc"], frac=c["frac"])
    q = dev_bf16(y["q"], torch, np)
    kc = dev_bf16(y["k_cache"], torch, np)
    vc = dev_bf16(y["v_cache"], torch, np)
    lens = y["seqlens"]
    seq = torch.from_numpy(lens.astype(np.int32)).cuda()
    T, Bc = c["split_tiles"], c["Bc"]
    lam, _ = calibrate_decode(q, kc, vc, seq, c["target_skip"], T, Bc)
    ws = torch.empty(ssa.decode_workspace_size(c["B"], c["Hq"], c["S_max"], c["d"], Bc, T),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((c["B"], c["Hq"]), dtype=torch.float32, device=q.device)
    nS = math.ceil(math.ceil(c["S_max"] / Bc) / T)
    counts = torch.empty((c["B"], c["Hkv"], nS), dtype=torch.int32, device=q.device)
    fn = lambda: ssa.decode(q, kc, vc, seq, lam, split_tiles=T, workspace=ws, out=out, lse_out=lse,
                            skip_counts=counts)
    ms, ev = time_launches(fn, 20, 5, torch)
    # kept V tiles from the timed launches' own skip counts, checked against
    # a statistics launch
    vis = c["Hkv"] * sum(math.ceil(int(n) / Bc) for n in lens)
    kept = vis - int(counts.sum().item())
    st = ssa.decode(q, kc, vc, seq, lam, split_tiles=T, stats=True, lse=False)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    if (int((state != 0).sum()), int((state == 1).sum())) != (vis, kept):
        raise RuntimeError("decode: timed launch counts differ from the statistics launch")
    loaded = float(decode_loaded_bytes(lens, c["B"], c["Hq"], c["Hkv"], c["d"], Bc, T, kept))
    res = {"workload": f"decode B=32 Hq=32 Hkv=8 d=128 lens U[16K,32K] split {T} tiles",
           "lambda": round(lam, 5), "tokens_per_s": round(c["B"] / (ms * 1e-3), 1), "ms": round(ms, 4),
           "event_ms": round(ev, 4), "skip_pct_v_tiles": round(100.0 * (vis - kept) / vis, 3),
           "visited_tiles": vis, "kept_tiles": kept,
           "loaded_bytes": loaded, "hbm_gbs": round(loaded / (ev * 1e-3) / 1e9, 1),
           "hbm_frac": round(loaded / (ev * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del q, kc, vc, st
    if not args.no_cpu:
        log("cpu baseline: oracle on the decode workload")
        try:
            res["cpu_baseline"] = cpu_baseline_decode(y, c, lam, args.cpu_budget, np)
        except Exception as e:  # report, keep the GPU figures
            res["cpu_baseline"] = {"error": repr(e)}
    return res


def extra_sparse(args, torch, np, ssa, synth):
    c = synth.CONFIGS[4]
    x = synth.prefill_inputs(4, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    m = ssa.block_mask(q, k, c["pool"], c["topk"], c["sink_blocks"], c["window_tokens"])
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    ws = m["workspace"]
    fm = lambda: ssa.block_mask(q, k, c["pool"], c["topk"], c["sink_blocks"], c["window_tokens"], workspace=ws)
    ms_mask, ev_mask = time_launches(fm, 10, 3, torch)
    kw = dict(Br=64, Bc=64, causal=True, block_idx=m["block_idx"], block_cnt=cnt)
    vis, kept, ms_p, ev_p = time_prefill_legs(q, k, v, c["lam"], kw, 10, 3, torch, ssa)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    res = {"workload": "block-sparse prefill 32K H=16 d=64, pooled top-64 + sink + 1024 window, lambda=-6",
            "mask_ms": round(ms_mask, 4), "mask_hbm_gbs": round(2 * 2 * c["Hq"] * c["L"] * c["d"] / (ev_mask * 1e-3) / 1e9, 1),
            "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
            "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
            "combined_sparsity": round(1 - kept / n_causal, 4),
            "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
            "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, m
    if not args.no_cpu:
        log("cpu baseline: oracle on the block-sparse workload")
        try:
            res["cpu_baseline"] = cpu_baseline_sparse(x, c, args.cpu_budget, np)
        except Exception as e:  # report, keep the GPU figures
            res["cpu_baseline"] = {"error": repr(e)}
    return res


def extra_sparge(args, torch, np, ssa, synth):
    """SpargeAttn two-stage filter on the 32K block-sparse shape with drifting
    blocks: stage one (self-similarity gate, compressed map, Top-tau mass)
    builds the lists, stage two (the skip rule) runs inside the prefill."""
    c = synth.SPARGE
    x = synth.prefill_inputs(c["cfg_id"], 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"],
                             frac=c["frac"], drift=c["drift"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    m = ssa.sparge_mask(q, k, c["theta"], c["tau"], "mass", c["pool"])
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    kw = dict(Br=64, Bc=64, causal=True, block_idx=m["block_idx"], block_cnt=cnt)
    ws = m["workspace"]
    fm = lambda: ssa.sparge_mask(q, k, c["theta"], c["tau"], "mass", c["pool"], workspace=ws)
    ms_mask, ev_mask = time_launches(fm, 10, 3, torch)
    vis, kept, ms_p, ev_p = time_prefill_legs(q, k, v, c["lam"], kw, 10, 3, torch, ssa)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    res = {"workload": "SpargeAttn two-stage prefill 32K H=16 d=64, drifting blocks, "
                       f"theta={c['theta']} tau={c['tau']} (P_hat mass), lambda={c['lam']}",
           "mask_ms": round(ms_mask, 4),
           "mask_hbm_gbs": round(2 * 2 * c["Hq"] * c["L"] * c["d"] / (ev_mask * 1e-3) / 1e9, 1),
           "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
           "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
           "combined_sparsity": round(1 - kept / n_causal, 4),
           "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
           "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, m
    return with_cpu(res, args, "the SpargeAttn workload",
                    lambda: cpu_baseline_masked(x, c, "sparge", {"theta": c["theta"], "tau": c["tau"]},
                                                args.cpu_budget / 2, "32K SpargeAttn"))


def extra_vslash(args, torch, np, ssa, synth):
    """Vertical-slash estimator (last 64 queries, 1000 vertical keys, 64
    slash offsets) and the block-sparse prefill over its tile cover, on the
    32K block-sparse shape."""
    c = synth.CONFIGS[4]
    x = synth.prefill_inputs(4, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    nv, ns, R = 1000, 64, 64
    m = ssa.vertical_slash_mask(q, k, nv, ns, R)
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    kw = dict(Br=64, Bc=64, causal=True, block_idx=m["block_idx"], block_cnt=cnt)
    ws = m["workspace"]
    ms_mask, ev_mask = time_launches(lambda: ssa.vertical_slash_mask(q, k, nv, ns, R, workspace=ws),
                                     10, 3, torch)
    vis, kept, ms_p, ev_p = time_prefill_legs(q, k, v, c["lam"], kw, 10, 3, torch, ssa)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    res = {"workload": f"vertical-slash estimator 32K H=16 d=64 (last {R} queries, {nv} vertical, "
                       f"{ns} slash) + block-sparse prefill over its tiles, lambda={c['lam']}",
           "estimator_ms": round(ms_mask, 4),
           "estimator_k_read_gbs": round(c["Hq"] * c["L"] * c["d"] * 2 / (ev_mask * 1e-3) / 1e9, 1),
           "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
           "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
           "combined_sparsity": round(1 - kept / n_causal, 4),
           "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
           "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, m
    return with_cpu(res, args, "the vertical-slash workload",
                    lambda: cpu_baseline_masked(x, c, "vslash", {"last_q": R, "n_vertical": nv, "n_slash": ns},
                                                args.cpu_budget / 2, "32K vertical-slash"))


def extra_nm(args, torch, np, ssa, synth):
    """N:M (2:4) sparse softmax on the 16K GQA shape, alone and with ~50% tile skipping."""
    from sparse_attention_long_skip_amd.calibrate import calibrate_prefill
    c = synth.CONFIGS[1]
    x = synth.prefill_inputs(1, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    kw = dict(Br=c["Br"], Bc=c["Bc"], causal=True, nm=(2, 4), dense_sink=64, dense_recent=256)
    lam50, _ = calibrate_prefill(q, k, v, 0.5, **kw)
    rows = []
    for lam in (-math.inf, lam50):
        vis, kept, ms, ev = time_prefill_legs(q, k, v, lam, kw, 10, 3, torch, ssa)
        rows.append({"lambda": None if lam == -math.inf else round(lam, 5), "ms": round(ms, 4),
                     "skip_pct": round(100.0 * (vis - kept) / vis, 3),
                     "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                     "mfma_frac_executed": round(2.0 * 128 * 64 * 128 * (vis + kept) / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    del q, k, v
    res = {"workload": "N:M 2:4 sparse softmax, 16K GQA shape, dense sink 64 + recent 256 tokens", "runs": rows}
    nm_kw = {"nm": (2, 4), "dense_sink": 64, "dense_recent": 256}
    return with_cpu(res, args, "the N:M workload",
                    lambda: cpu_baseline_prefill(1, lam50, args.cpu_budget / 2, np, synth, "16K N:M 2:4",
                                                 nm_kw=nm_kw))


def extra_warp_units(args, torch, np, ssa, synth):
    """Br = 32 decision units (the per-warp variant) on the 16K GQA shape,
    lambda calibrated to ~50% of the 32-row units' tiles skipped. Four units
    share a 128-row workgroup: every wave computes the scores of the tiles
    the workgroup visits, and the exponentials and P.V of the tiles its own
    unit keeps."""
    from sparse_attention_long_skip_amd.calibrate import calibrate_prefill
    c = synth.CONFIGS[1]
    x = synth.prefill_inputs(1, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    kw = dict(Br=32, Bc=c["Bc"], causal=True)
    lam, _ = calibrate_prefill(q, k, v, 0.5, **kw)
    vis, kept, ms, ev = time_prefill_legs(q, k, v, lam, kw, 10, 3, torch, ssa)
    wg_vis = visited_tiles_count(c["B"], c["Hq"], c["L"], 128, c["Bc"], True)
    ex = 2.0 * 32 * 64 * c["d"] * (4 * wg_vis + kept)
    del q, k, v
    res = {"workload": "Br=32 decision units (per-warp skip), 16K GQA shape, lambda calibrated to ~50% unit skip",
           "lambda": round(lam, 5), "ms": round(ms, 4), "skip_pct": round(100.0 * (vis - kept) / vis, 3),
           "unit_tiles_visited": vis, "unit_tiles_kept": kept, "workgroup_tiles_visited": wg_vis,
           "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
           "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return with_cpu(res, args, "the 32-row-unit workload",
                    lambda: cpu_baseline_prefill(1, lam, args.cpu_budget / 2, np, synth, "16K", Br=32))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="wall seconds per CPU-baseline leg (the oracle in worker processes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baselines")
    ap.add_argument("--only-main", action="store_true", help="skip extra and cpu baseline (profiling)")
    ap.add_argument("--leg", choices=["prefill_128k", "decode", "block_sparse_32k", "sparge_32k",
                                      "vslash_32k", "nm_2of4_16k", "warp_units_16k"],
                    help="run only this extra leg and print its JSON (profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the main leg, copy a 1 GiB buffer 5 times (HBM counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels shard by "
              "(batch, head) with no communication, so no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import sparse_attention_long_skip_amd as ssa

    ssa.lib()
    torch.cuda.set_device(0)
    legs = {"prefill_128k": extra_128k, "decode": extra_decode, "block_sparse_32k": extra_sparse,
            "sparge_32k": extra_sparge, "vslash_32k": extra_vslash, "nm_2of4_16k": extra_nm,
            "warp_units_16k": extra_warp_units}
    if args.leg:
        print(json.dumps({args.leg: legs[args.leg](args, torch, np, ssa, synth)}), flush=True)
        return
    c = synth.CONFIGS[1]
    log("generating the 16K prefill workload")
    p = bench_prefill(1, args, torch, np, ssa, synth, target=c["target_skip"])
    lam = p["lam"]
    log(f"lambda {lam:.5f} (calibrated ratio {p['calibrated_ratio']:.4f}); timing {args.steps} steps")
    # exactly args.warmup untimed launches (the default, 200, is ~0.3 s of them)
    vis, kept, ms, ev_ms = run_prefill(p, lam, args.steps, args.warmup, torch, ssa, warm_s=0.0)
    ex = 2.0 * c["Br"] * c["Bc"] * c["d"] * (vis + kept)
    dense = dense_flops(c)
    value = dense / (ms * 1e-3) / 1e12
    achieved = ex / (ev_ms * 1e-3) / 1e12
    log(f"prefill {ms:.3f} ms/step (events {ev_ms:.3f} ms), {value:.1f} dense-equiv TFLOP/s, "
        f"MFMA {achieved:.1f} TFLOP/s executed, skip {(vis - kept) / vis * 100:.2f}%")
    traffic = load_traffic("prefill_16k", 1)
    result = {
        "metric": "prefill dense-equiv TFLOP/s @16K (Skip-Softmax, ~50% tiles skipped)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded planted-direction generator)",
        "config": {"workload": "prefill B=1 Hq=32 Hkv=8 d=128 L=16384 causal Br=128 Bc=64, "
                               "10% planted + sink, lambda calibrated to ~50% skip",
                   "global_batch": 1, "seq_len": c["L"], "parallelism": "single GPU",
                   "lambda": round(lam, 6), "skip_pct": round(100.0 * (vis - kept) / vis, 3),
                   "visited_tiles": vis, "kept_tiles": kept},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "prefill_kernel<128, 128, false, false, false, 4>", "kernel_ms": round(ev_ms, 4),
                     "executed_flops": ex},
    }
    if not args.only_main:
        result["config"]["calibration"] = time_calibration(p, c["target_skip"], torch, ssa)
    del p
    torch.cuda.empty_cache()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        ms_c, ev_c = time_launches(lambda: dst.copy_(src), 5, 1, torch)
        log(f"copy probe: 1 GiB copy {ev_c:.3f} ms ({2 * (1 << 30) / (ev_c * 1e-3) / 1e9:.1f} GB/s)")
        result["copy_probe"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "ms": round(ev_c, 4)}
        del src, dst
    extra = {}
    if not (args.no_extra or args.only_main):
        for name, fn in legs.items():
            try:
                log(f"extra: {name}")
                extra[name] = fn(args, torch, np, ssa, synth)
            except Exception as e:  # report, keep the headline
                extra[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        result["extra"] = extra
    if not (args.only_main or args.no_cpu):
        log("cpu baseline: oracle on the 16K workload")
        result["cpu_baseline"] = cpu_baseline_prefill(1, lam, args.cpu_budget, np, synth, "16K")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
