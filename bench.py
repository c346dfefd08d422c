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

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-extra]
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


def time_launches(fn, steps, warmup, torch):
    """Warm up, then time `steps` calls: wall clock between synchronisations
    and HIP events around each call (on the current stream, where the
    library launches). Returns (ms per step, mean event ms)."""
    for _ in range(warmup):
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


def run_prefill(p, lam, steps, warmup, torch, ssa):
    c = p["cfg"]
    q, k, v = p["q"], p["k"], p["v"]
    st = ssa.prefill(q, k, v, lam, Br=c["Br"], Bc=c["Bc"], causal=c["causal"], stats=True)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    out = torch.empty_like(q)
    fn = lambda: ssa.prefill(q, k, v, lam, Br=c["Br"], Bc=c["Bc"], causal=c["causal"], out=out)
    ms, ev_ms = time_launches(fn, steps, warmup, torch)
    return state, ms, ev_ms


def dense_flops(c):
    L = c["L"]
    return 4.0 * c["d"] * c["B"] * c["Hq"] * L * (L + 1) / 2


def cpu_baseline_prefill(cfg_id, lam, budget_s, np, synth):
    """Time the oracle on a seeded sample of query tiles of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    c = synth.CONFIGS[cfg_id]
    x = synth.prefill_inputs(cfg_id, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"],
                             frac=c["frac"])
    nQ = math.ceil(c["L"] / c["Br"])
    rng = np.random.default_rng(1234)
    units = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, c["Hq"], 4096),
                                                 rng.integers(0, nQ, 4096))]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for u in units:
        oracle.prefill(x["q"], x["k"], x["v"], lam, c["Br"], c["Bc"], c["causal"], units=[u],
                       bits=True)
        i = u[2]
        r0, r1 = i * c["Br"], min(c["L"], (i + 1) * c["Br"])
        # dense-equivalent work of these rows: 4 d per allowed (row, key) pair
        flops += 4.0 * c["d"] * sum(r + 1 for r in range(r0, r1))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "dense-equiv TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} random query tiles (of {c['Hq'] * nQ}) of the 16K workload, "
                      f"fp64 numpy, {dt:.1f} s"}


def extra_128k(args, torch, np, ssa, synth):
    p = bench_prefill(3, args, torch, np, ssa, synth, lam=-math.inf)
    c = p["cfg"]
    rows = []
    for lam in c["lam_sweep"]:
        state, ms, ev = run_prefill(p, lam, 3, 1, torch, ssa)
        vis, kept, ex = prefill_work(state, c["Br"], c["Bc"], c["d"])
        rows.append({"lambda": lam, "ms": round(ms, 3), "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                     "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "skip_pct": round(100.0 * (vis - kept) / vis, 3)})
    # also at a calibrated ~50% point
    from sparse_attention_long_skip_amd.calibrate import calibrate_prefill
    lam50, _ = calibrate_prefill(p["q"], p["k"], p["v"], 0.5, c["Br"], c["Bc"], True)
    state, ms, ev = run_prefill(p, lam50, 3, 1, torch, ssa)
    vis, kept, ex = prefill_work(state, c["Br"], c["Bc"], c["d"])
    rows.append({"lambda": round(lam50, 5), "label": "calibrated ~50% (extra point)", "ms": round(ms, 3),
                 "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                 "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "skip_pct": round(100.0 * (vis - kept) / vis, 3)})
    del p
    return {"workload": "prefill 128K B=1 Hq=8 Hkv=1 d=128 causal Br=128 Bc=64, 5% planted", "sweep": rows}


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
    del y
    T = c["split_tiles"]
    lam, _ = calibrate_decode(q, kc, vc, seq, c["target_skip"], T, c["Bc"])
    st = ssa.decode(q, kc, vc, seq, lam, split_tiles=T, stats=True)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    vis, kept = int((state != 0).sum()), int((state == 1).sum())
    ws = st["workspace"]
    out = torch.empty_like(q)
    fn = lambda: ssa.decode(q, kc, vc, seq, lam, split_tiles=T, workspace=ws, out=out)
    ms, ev = time_launches(fn, 20, 5, torch)
    d, Hkv, Bc = c["d"], c["Hkv"], c["Bc"]
    nS = math.ceil(math.ceil(c["S_max"] / Bc) / T)
    k_bytes = 2.0 * d * Hkv * float(lens.sum())
    v_bytes = 2.0 * d * Bc * kept
    io = 2.0 * 2 * c["B"] * c["Hq"] * d
    wsb = 2.0 * 4 * c["B"] * c["Hq"] * sum(math.ceil(math.ceil(n / Bc) / T) for n in lens) * (d + 2)
    loaded = k_bytes + v_bytes + io + wsb
    return {"workload": f"decode B=32 Hq=32 Hkv=8 d=128 lens U[16K,32K] split {T} tiles",
            "lambda": round(lam, 5), "tokens_per_s": round(c["B"] / (ms * 1e-3), 1), "ms": round(ms, 4),
            "event_ms": round(ev, 4), "skip_pct_v_tiles": round(100.0 * (vis - kept) / vis, 3),
            "loaded_bytes": loaded, "hbm_gbs": round(loaded / (ev * 1e-3) / 1e9, 1),
            "hbm_frac": round(loaded / (ev * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def extra_sparse(args, torch, np, ssa, synth):
    c = synth.CONFIGS[4]
    x = synth.prefill_inputs(4, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    m = ssa.block_mask(q, k, c["pool"], c["topk"], c["sink_blocks"], c["window_tokens"])
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    st = ssa.prefill(q, k, v, c["lam"], Br=64, Bc=64, causal=True, block_idx=m["block_idx"],
                     block_cnt=cnt, stats=True)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    vis, kept = int((state != 0).sum()), int((state == 1).sum())
    ws = m["workspace"]
    fm = lambda: ssa.block_mask(q, k, c["pool"], c["topk"], c["sink_blocks"], c["window_tokens"], workspace=ws)
    ms_mask, ev_mask = time_launches(fm, 10, 3, torch)
    out = torch.empty_like(q)
    fp = lambda: ssa.prefill(q, k, v, c["lam"], Br=64, Bc=64, causal=True, block_idx=m["block_idx"],
                             block_cnt=cnt, out=out)
    ms_p, ev_p = time_launches(fp, 10, 3, torch)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    return {"workload": "block-sparse prefill 32K H=16 d=64, pooled top-64 + sink + 1024 window, lambda=-6",
            "mask_ms": round(ms_mask, 4), "mask_hbm_gbs": round(2 * 2 * c["Hq"] * c["L"] * c["d"] / (ev_mask * 1e-3) / 1e9, 1),
            "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
            "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
            "combined_sparsity": round(1 - kept / n_causal, 4),
            "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
            "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def extra_sparge(args, torch, np, ssa, synth):
    """SpargeAttn two-stage filter on the 32K block-sparse shape with drifting
    blocks: stage one (self-similarity gate, compressed map, Top-tau mass)
    builds the lists, stage two (the skip rule) runs inside the prefill."""
    c = synth.SPARGE
    x = synth.prefill_inputs(c["cfg_id"], 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"],
                             frac=c["frac"], drift=c["drift"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    m = ssa.sparge_mask(q, k, c["theta"], c["tau"], "mass", c["pool"])
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    kw = dict(Br=64, Bc=64, causal=True, block_idx=m["block_idx"], block_cnt=cnt)
    st = ssa.prefill(q, k, v, c["lam"], stats=True, **kw)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    vis, kept = int((state != 0).sum()), int((state == 1).sum())
    ws = m["workspace"]
    fm = lambda: ssa.sparge_mask(q, k, c["theta"], c["tau"], "mass", c["pool"], workspace=ws)
    ms_mask, ev_mask = time_launches(fm, 10, 3, torch)
    out = torch.empty_like(q)
    ms_p, ev_p = time_launches(lambda: ssa.prefill(q, k, v, c["lam"], out=out, **kw), 10, 3, torch)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    return {"workload": "SpargeAttn two-stage prefill 32K H=16 d=64, drifting blocks, "
                        f"theta={c['theta']} tau={c['tau']} (P_hat mass), lambda={c['lam']}",
            "mask_ms": round(ms_mask, 4),
            "mask_hbm_gbs": round(2 * 2 * c["Hq"] * c["L"] * c["d"] / (ev_mask * 1e-3) / 1e9, 1),
            "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
            "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
            "combined_sparsity": round(1 - kept / n_causal, 4),
            "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
            "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def extra_vslash(args, torch, np, ssa, synth):
    """Vertical-slash estimator (last 64 queries, 1000 vertical keys, 64
    slash offsets) and the block-sparse prefill over its tile cover, on the
    32K block-sparse shape."""
    c = synth.CONFIGS[4]
    x = synth.prefill_inputs(4, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    nv, ns, R = 1000, 64, 64
    m = ssa.vertical_slash_mask(q, k, nv, ns, R)
    torch.cuda.synchronize()
    cnt = m["block_cnt"]
    nB = cnt.shape[-1]
    n_causal = c["Hq"] * nB * (nB + 1) / 2
    kw = dict(Br=64, Bc=64, causal=True, block_idx=m["block_idx"], block_cnt=cnt)
    st = ssa.prefill(q, k, v, c["lam"], stats=True, **kw)
    torch.cuda.synchronize()
    state = st["tile_state"].cpu().numpy()
    vis, kept = int((state != 0).sum()), int((state == 1).sum())
    ws = m["workspace"]
    ms_mask, ev_mask = time_launches(lambda: ssa.vertical_slash_mask(q, k, nv, ns, R, workspace=ws),
                                     10, 3, torch)
    out = torch.empty_like(q)
    ms_p, ev_p = time_launches(lambda: ssa.prefill(q, k, v, c["lam"], out=out, **kw), 10, 3, torch)
    ex = 2.0 * 64 * 64 * c["d"] * (vis + kept)
    return {"workload": f"vertical-slash estimator 32K H=16 d=64 (last {R} queries, {nv} vertical, "
                        f"{ns} slash) + block-sparse prefill over its tiles, lambda={c['lam']}",
            "estimator_ms": round(ms_mask, 4),
            "estimator_k_read_gbs": round(c["Hq"] * c["L"] * c["d"] * 2 / (ev_mask * 1e-3) / 1e9, 1),
            "prefill_ms": round(ms_p, 4), "mask_density": round(vis / n_causal, 4),
            "in_mask_skip_pct": round(100.0 * (vis - kept) / vis, 3),
            "combined_sparsity": round(1 - kept / n_causal, 4),
            "dense_equiv_tflops": round(dense_flops(c) / (ms_mask + ms_p) / 1e9, 1),
            "mfma_frac_executed": round(ex / (ev_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def extra_nm(args, torch, np, ssa, synth):
    """N:M (2:4) sparse softmax on the 16K GQA shape, alone and with ~50% tile skipping."""
    from sparse_attention_long_skip_amd.calibrate import lambda_for_ratio
    c = synth.CONFIGS[1]
    x = synth.prefill_inputs(1, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    kw = dict(Br=c["Br"], Bc=c["Bc"], causal=True, nm=(2, 4), dense_sink=64, dense_recent=256)
    m = ssa.prefill(q, k, v, -math.inf, margins=True, lse=False, **kw)["tile_margin"].cpu().numpy()
    rows = []
    out = torch.empty_like(q)
    for lam in (-math.inf, lambda_for_ratio(m, 0.5)):
        st = ssa.prefill(q, k, v, lam, stats=True, **kw)
        torch.cuda.synchronize()
        s = st["tile_state"].cpu().numpy()
        vis, kept = int((s != 0).sum()), int((s == 1).sum())
        ms, ev = time_launches(lambda: ssa.prefill(q, k, v, lam, out=out, **kw), 10, 3, torch)
        rows.append({"lambda": None if lam == -math.inf else round(lam, 5), "ms": round(ms, 4),
                     "skip_pct": round(100.0 * (vis - kept) / vis, 3),
                     "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
                     "mfma_frac_executed": round(2.0 * 128 * 64 * 128 * (vis + kept) / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    return {"workload": "N:M 2:4 sparse softmax, 16K GQA shape, dense sink 64 + recent 256 tokens", "runs": rows}


def extra_warp_units(args, torch, np, ssa, synth):
    """Br = 32 decision units (the per-warp variant) on the 16K GQA shape,
    lambda calibrated to ~50% of the 32-row units' tiles skipped."""
    from sparse_attention_long_skip_amd.calibrate import lambda_for_ratio
    c = synth.CONFIGS[1]
    x = synth.prefill_inputs(1, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = (dev_bf16(x[n], torch, np) for n in ("q", "k", "v"))
    del x
    kw = dict(Br=32, Bc=c["Bc"], causal=True)
    m = ssa.prefill(q, k, v, -math.inf, margins=True, lse=False, **kw)["tile_margin"].cpu().numpy()
    lam = lambda_for_ratio(m, 0.5)
    st = ssa.prefill(q, k, v, lam, stats=True, **kw)
    torch.cuda.synchronize()
    s = st["tile_state"].cpu().numpy()  # [B, Hq, L / 32, nK]
    vis, kept = int((s != 0).sum()), int((s == 1).sum())
    # four 32-row units share a 128-row workgroup: every wave computes the
    # scores of the tiles the workgroup visits and the P.V of the tiles any
    # of its units keeps
    g = s.reshape(s.shape[0], s.shape[1], -1, 4, s.shape[-1])
    wg_vis = int((g != 0).any(axis=3).sum())
    wg_kept = int((g == 1).any(axis=3).sum())
    out = torch.empty_like(q)
    ms, ev = time_launches(lambda: ssa.prefill(q, k, v, lam, out=out, **kw), 10, 3, torch)
    ex = 2.0 * 32 * 64 * c["d"] * 4 * (wg_vis + wg_kept)
    return {"workload": "Br=32 decision units (per-warp skip), 16K GQA shape, lambda calibrated to ~50% unit skip",
            "lambda": round(lam, 5), "ms": round(ms, 4), "skip_pct": round(100.0 * (vis - kept) / vis, 3),
            "pv_tiles_run_vs_kept": round(4 * wg_kept / max(kept, 1), 3),
            "dense_equiv_tflops": round(dense_flops(c) / ms / 1e9, 1),
            "mfma_frac_executed": round(ex / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
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
    state, ms, ev_ms = run_prefill(p, lam, args.steps, args.warmup, torch, ssa)
    vis, kept, ex = prefill_work(state, c["Br"], c["Bc"], c["d"])
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
    if not args.only_main:
        log("cpu baseline: oracle on a sample of the 16K workload")
        result["cpu_baseline"] = cpu_baseline_prefill(1, lam, args.cpu_budget, np, synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
