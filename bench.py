#!/usr/bin/env python3
"""Benchmark of the WaveFilter per-step path on one MI355X.

Workload: the 64K-token layer (32 heads, head dim 128, bfloat16, prompt
N_p = 65536, generated cache N_g = 512, query block 64, Haar L = 6, budgets
64, 118, 214, 384, 683, 1195, 2048).  One step is one pass of every stage
of the path over one synthetic layer: wf_build_pyramid (Haar pyramid of the
prompt keys) followed by wf_select_attend (coarse scores, coarse Top-K,
recursive refinement, sparse attention).  Inputs are resident in HBM before
the timed region; the loop rotates over R device copies of the layer at
distinct addresses, so no step finds its inputs in the 256 MB last-level
cache left by the previous one.

Prints one JSON line.  ``value`` is steps/s of the full step; the
select-attend stage alone (the per-denoising-step cost when the pyramid is
reused across steps) is reported beside it, as are both stages' HBM
rooflines and the float64 oracle timed on a bounded sample on the host.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "wf_select_attend steps/s + achieved HBM GB/s vs peak, 1 MI355X, 64K ctx"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pyramid_top_kernel_64k_pmc.txt")
# the files pyramid_top_kernel is compiled from: counter figures taken on
# other code are not reported
KERNEL_SOURCES = [os.path.join(ROOT, "long_context_kv_haar_amd", "csrc", f)
                  for f in ("wf_pyramid.hip", "wf_pyramid.h", "wf_types.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def algorithmic_bytes(cfg):
    """Bytes the method must move (re-reads never counted), per call.

    pyramid: read the prompt keys once, write A_L (float32).
    select-attend, per head: Q, A_L (float32), the K rows of every token the
    kept coarse regions cover (they score every finer level and contain the
    final tokens' keys), V of the kept tokens, K and V of the generated
    positions, O (float32), the kept indices.
    """
    s = 2 if cfg.dtype == "bf16" else 4
    BH, d, L = cfg.batch * cfg.heads, cfg.head_dim, cfg.levels
    b = cfg.budgets
    n_top, k_top, k0 = cfg.n_prompt >> L, b[0], b[-1]
    covered = k_top << L
    pyr = BH * (cfg.n_prompt * d * s + n_top * d * 4)
    sel = BH * (cfg.n_q * d * s + n_top * d * 4 + covered * d * s + k0 * d * s + 2 * cfg.n_gen * d * s
                + cfg.n_q * d * 4 + 4 * k0)
    return pyr, sel


def attend_bytes(cfg):
    """Bytes of attention over a selection made earlier, per call: Q, the
    kept indices, K and V of the kept and the generated rows, O (float32)."""
    s = 2 if cfg.dtype == "bf16" else 4
    BH, d, k0 = cfg.batch * cfg.heads, cfg.head_dim, cfg.budgets[-1]
    return BH * (cfg.n_q * d * s + 4 * k0 + 2 * (k0 + cfg.n_gen) * d * s + cfg.n_q * d * 4)


def read_pmc_traffic():
    """HBM bytes per pyramid launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel code."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m_sha = re.search(r"kernel_source_sha256_12:\s*(\w+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def time_workload(cfg, dev, launches, warmup):
    """Per-layer timings of one workload: wf_build_pyramid and wf_select_attend
    each launched back to back over R device copies of one synthetic layer
    (R sized so the copies exceed the 256 MB last-level cache where they can),
    between one pair of HIP events on the launch stream."""
    import math

    import torch

    import long_context_kv_haar_amd as wf
    from workloads.gen import make_layer

    es = 2 if cfg.dtype == "bf16" else 4
    BH, d, L, budgets = cfg.batch * cfg.heads, cfg.head_dim, cfg.levels, cfg.budgets
    per_copy = BH * (2 * cfg.n_tot + cfg.n_q) * d * es
    R = min(16, max(2, math.ceil((2 << 30) / per_copy)))
    base = make_layer(cfg, 0, device=dev)
    copies = [base] + [type(base)(cfg, 0, base.q.clone(), base.k.clone(), base.v.clone(), base.gen_idx.clone(),
                                  base.spans) for _ in range(R - 1)]
    pbytes = wf.pyramid_bytes(cfg.batch, cfg.heads, cfg.n_prompt, d, L)
    builds, steps, ws = [], [], None
    for c in copies:
        pb = wf.PreparedBuild(c.k, cfg.n_prompt, L, torch.empty(pbytes, dtype=torch.uint8, device=dev))
        pyr = pb()
        if ws is None:
            ws = torch.zeros(wf.workspace_bytes(pyr, cfg.n_q, cfg.n_gen, budgets), dtype=torch.uint8, device=dev)
        out = torch.empty((cfg.batch, cfg.heads, cfg.n_q, d), dtype=torch.float32, device=dev)
        sel = torch.empty((cfg.batch, cfg.heads, budgets[-1]), dtype=torch.int32, device=dev)
        builds.append(pb)
        steps.append(wf.PreparedStep(c.q, pyr, c.k, c.v, c.gen_idx, budgets, out, sel, ws))
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fns):
        for i in range(warmup):
            fns[i % R]()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(launches):
            fns[i % R]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches * 1e3  # us

    build_us = timed(builds)
    sel_us = timed(steps)
    pyr_b, sel_b = algorithmic_bytes(cfg)
    rec = {
        "layers_x_batch_x_heads": f"{cfg.layers}x{cfg.batch}x{cfg.heads}",
        "dtype": cfg.dtype, "n_prompt": cfg.n_prompt, "n_q": cfg.n_q, "levels": L,
        "budgets": ",".join(map(str, budgets)),
        "rotating_copies": R,
        "inputs_fit_in_last_level_cache": R * per_copy < (512 << 20),
        "build_us": round(build_us, 2),
        "build_GBps": round(pyr_b / (build_us * 1e-6) / 1e9, 1),
        "select_attend_us": round(sel_us, 2),
        "select_attend_calls_per_s": round(1e6 / sel_us, 1),
        "select_attend_GBps": round(sel_b / (sel_us * 1e-6) / 1e9, 1),
        "select_attend_frac_of_hbm_peak": round(sel_b / (sel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if cfg.layers > 1:  # every layer has the same shape: the step of all layers
        rec["all_layers_select_attend_ms"] = round(cfg.layers * sel_us * 1e-3, 3)
        rec["all_layers_build_ms"] = round(cfg.layers * build_us * 1e-3, 3)
    del builds, steps, copies, base, ws
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(inp, heads, min_seconds):
    """The float64 oracle, unchanged, on `heads` heads of one step (one thread),
    repeated over those heads until at least `min_seconds` of oracle time."""
    from threadpoolctl import threadpool_limits

    from oracle import select_attend  # the oracle is the CPU baseline
    from workloads.gen import to_f64

    cfg = inp.cfg
    gen = inp.gen_idx.cpu().numpy()
    data = [(to_f64(inp.q[0, h]), to_f64(inp.k[0, h]), to_f64(inp.v[0, h])) for h in heads]
    times = []
    with threadpool_limits(limits=1):
        while not times or sum(times) < min_seconds:
            for q, k, v in data:
                t0 = time.perf_counter()
                select_attend(q, k, v, cfg.n_prompt, gen, cfg.budgets, cfg.levels)
                times.append(time.perf_counter() - t0)
    per_head = sum(times) / len(times)
    return {
        "value": 1.0 / (per_head * cfg.batch * cfg.heads),
        "unit": "steps/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(times)} head-calls over heads 0..{len(heads) - 1} of one step (Haar pyramid + selection "
                  f"+ attention per head, float64 numpy, 1 thread), {sum(times):.1f} s; rate scaled to all "
                  f"{cfg.batch * cfg.heads} heads",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=16, help="device copies of the layer rotated over")
    ap.add_argument("--cpu-heads", type=int, default=8, help="heads of the CPU-baseline sample (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="minimum oracle time of the CPU-baseline sample")
    ap.add_argument("--workloads", type=int, default=1,
                    help="also time every workload's build and select-attend per layer (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the path has no multi-GPU execution "
              "(heads are independent; see the sharding notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_kv_haar_amd as wf
    from workloads.configs import CONFIGS
    from workloads.gen import make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = CONFIGS[4]
    L, budgets = cfg.levels, cfg.budgets
    base = make_layer(cfg, 0, device=dev)
    R = max(1, args.rotate)
    copies = [base] + [type(base)(cfg, 0, base.q.clone(), base.k.clone(), base.v.clone(), base.gen_idx.clone(),
                                  base.spans) for _ in range(R - 1)]
    pbytes = wf.pyramid_bytes(cfg.batch, cfg.heads, cfg.n_prompt, cfg.head_dim, L)
    builds, steps = [], []
    ws = None
    outs = []
    for c in copies:
        pb = wf.PreparedBuild(c.k, cfg.n_prompt, L, torch.empty(pbytes, dtype=torch.uint8, device=dev))
        pyr = pb()
        if ws is None:
            need = wf.workspace_bytes(pyr, cfg.n_q, cfg.n_gen, budgets)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        out = torch.empty((cfg.batch, cfg.heads, cfg.n_q, cfg.head_dim), dtype=torch.float32, device=dev)
        sel = torch.empty((cfg.batch, cfg.heads, budgets[-1]), dtype=torch.int32, device=dev)
        outs.append((out, sel))
        builds.append(pb)
        steps.append(wf.PreparedStep(c.q, pyr, c.k, c.v, c.gen_idx, budgets, out, sel, ws))
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # -- full step: build + select-attend, per-stage HIP events on the launch stream
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        builds[i % R]()
        steps[i % R]()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e0, e1, e2 = ev[i]
        e0.record(stream)
        builds[i % R]()
        e1.record(stream)
        steps[i % R]()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pyr_ms = sum(e0.elapsed_time(e1) for e0, e1, _ in ev) / K
    sel_ms = sum(e1.elapsed_time(e2) for _, e1, e2 in ev) / K

    # -- the pyramid build alone, back to back over the copies: the kernel's average
    #    launch duration (one event pair around all K launches, so no per-launch
    #    event overhead)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(args.warmup):
        builds[i % R]()
    torch.cuda.synchronize()
    s0.record(stream)
    for i in range(K):
        builds[i % R]()
    s1.record(stream)
    torch.cuda.synchronize()
    pyr_only_ms = s0.elapsed_time(s1) / K

    # -- select-attend alone (pyramids reused), rotating over the copies
    for i in range(args.warmup):
        steps[i % R]()
    torch.cuda.synchronize()
    s0.record(stream)
    for i in range(K):
        steps[i % R]()
    s1.record(stream)
    torch.cuda.synchronize()
    sel_only_ms = s0.elapsed_time(s1) / K

    # -- select-attend with the query rows averaged instead of maximised (same bytes)
    steps_mean = []
    for c, pb, (out, sel) in zip(copies, builds, outs):
        steps_mean.append(wf.PreparedStep(c.q, pb.pyramid, c.k, c.v, c.gen_idx, budgets, torch.empty_like(out),
                                          torch.empty_like(sel), ws, agg="mean"))
    for i in range(args.warmup):
        steps_mean[i % R]()
    torch.cuda.synchronize()
    s0.record(stream)
    for i in range(K):
        steps_mean[i % R]()
    s1.record(stream)
    torch.cuda.synchronize()
    mean_ms = s0.elapsed_time(s1) / K

    # -- incremental refresh: every copy (standing in for a layer) rebuilds 64 of its
    #    1024 level-L blocks, all copies in one call
    n_top = cfg.n_prompt >> L
    gref = torch.Generator().manual_seed(7)
    ref_items = [(c.k, pb.pyramid, torch.randperm(n_top, generator=gref)[:64].to(torch.int32).to(dev))
                 for c, pb in zip(copies, builds)]
    refresh = wf.PreparedRefresh(ref_items)
    for _ in range(args.warmup):
        refresh()
    torch.cuda.synchronize()
    s0.record(stream)
    for _ in range(K):
        refresh()
    s1.record(stream)
    torch.cuda.synchronize()
    refresh_ms = s0.elapsed_time(s1) / K
    es = 2 if cfg.dtype == "bf16" else 4
    refresh_units = R * cfg.batch * cfg.heads * 64
    refresh_bytes = refresh_units * ((1 << L) * cfg.head_dim * es + cfg.head_dim * 4)
    # restore every copy's pyramid for what follows
    for pb in builds:
        pb()
    torch.cuda.synchronize()

    # -- the Daubechies four-tap basis: its build stores every band (about 2 GB for this
    #    layer), so one copy is used; finer levels are scored from the stored bands
    db2_bytes = wf.pyramid_bytes(cfg.batch, cfg.heads, cfg.n_prompt, cfg.head_dim, L, wf.WF_PYR_DB2)
    db2_build = wf.PreparedBuild(base.k, cfg.n_prompt, L, torch.empty(db2_bytes, dtype=torch.uint8, device=dev),
                                 flags=wf.WF_PYR_DB2)
    db2_build()
    db2_out = torch.empty_like(outs[0][0])
    db2_sel = torch.empty_like(outs[0][1])
    db2_step = wf.PreparedStep(base.q, db2_build.pyramid, base.k, base.v, base.gen_idx, budgets, db2_out, db2_sel, ws)
    for _ in range(args.warmup):
        db2_step()
    torch.cuda.synchronize()
    s0.record(stream)
    for _ in range(K):
        db2_step()
    s1.record(stream)
    torch.cuda.synchronize()
    db2_ms = s0.elapsed_time(s1) / K
    s0.record(stream)
    db2_build()
    s1.record(stream)
    torch.cuda.synchronize()
    db2_build_ms = s0.elapsed_time(s1)
    del db2_build, db2_step
    torch.cuda.empty_cache()

    # -- attention over the selection each copy's last call made (a later step reusing it)
    reuse = [wf.PreparedAttend(c.q, c.k, c.v, sel, c.gen_idx, torch.empty_like(out), ws)
             for c, (out, sel) in zip(copies, outs)]
    for i in range(args.warmup):
        reuse[i % R]()
    torch.cuda.synchronize()
    s0.record(stream)
    for i in range(K):
        reuse[i % R]()
    s1.record(stream)
    torch.cuda.synchronize()
    reuse_ms = s0.elapsed_time(s1) / K
    reuse_bytes = attend_bytes(cfg)
    reuse_gbs = reuse_bytes / (reuse_ms * 1e-3) / 1e9

    pyr_bytes, sel_bytes = algorithmic_bytes(cfg)
    pyr_gbs = pyr_bytes / (pyr_only_ms * 1e-3) / 1e9
    sel_gbs = sel_bytes / (sel_only_ms * 1e-3) / 1e9
    traffic = read_pmc_traffic()
    rec = {
        "metric": METRIC,
        "value": K / wall,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llada-64k layer: 1 x 32 heads, d=128, bf16, N_p=65536 (Student-t(4) keys, 8 planted "
                        "spans), N_g=512, n_q=64, Haar L=6, budgets " + ",".join(map(str, budgets))
                        + "; step = wf_build_pyramid + wf_select_attend",
            "rotating_copies": R,
        },
        "roofline": {
            "kernel": "pyramid_top_kernel (wf_build_pyramid)",
            "bound": "hbm",
            "achieved": round(pyr_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(pyr_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": pyr_bytes,
            "avg_launch_us": round(pyr_only_ms * 1e3, 2),
            "us_in_step": round(pyr_ms * 1e3, 2),
        },
        "select_attend": {
            "calls_per_s": 1e3 / sel_only_ms,
            "us_per_call": round(sel_only_ms * 1e3, 2),
            "us_per_call_in_step": round(sel_ms * 1e3, 2),
            "algorithmic_bytes": sel_bytes,
            "achieved_GBps": round(sel_gbs, 1),
            "frac_of_hbm_peak": round(sel_gbs / HBM_PEAK_GBS, 4),
        },
        "select_attend_mean_rows": {
            "calls_per_s": 1e3 / mean_ms,
            "us_per_call": round(mean_ms * 1e3, 2),
            "achieved_GBps": round(sel_bytes / (mean_ms * 1e-3) / 1e9, 1),
        },
        "refresh_pyramids": {
            "layers": R,
            "blocks_per_layer": 64,
            "us_per_call": round(refresh_ms * 1e3, 2),
            "algorithmic_bytes": refresh_bytes,
            "achieved_GBps": round(refresh_bytes / (refresh_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(refresh_bytes / (refresh_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "select_attend_db2": {
            "us_per_call": round(db2_ms * 1e3, 2),
            "pyramid_build_us": round(db2_build_ms * 1e3, 1),
            "note": "one copy (the stored bands take about 2 GB), so its inputs may sit in the MALL",
        },
        "attend_selected": {
            "calls_per_s": 1e3 / reuse_ms,
            "us_per_call": round(reuse_ms * 1e3, 2),
            "algorithmic_bytes": reuse_bytes,
            "achieved_GBps": round(reuse_gbs, 1),
            "frac_of_hbm_peak": round(reuse_gbs / HBM_PEAK_GBS, 4),
        },
        "kernel_source_sha256_12": kernel_source_hash(),
    }
    if args.workloads:
        # the other workloads (the 1K, 4K, 16K and 128K-sweep layers are parity cases; their
        # timings are reported here, not as bench lines)
        del steps, builds, steps_mean, reuse, refresh, ref_items, copies, ws, outs
        torch.cuda.empty_cache()
        rec["workloads"] = {CONFIGS[c].name: time_workload(CONFIGS[c], dev, 100 if c < 5 else 40, 10)
                            for c in sorted(CONFIGS)}
    if args.cpu_heads > 0:
        rec["cpu_baseline"] = cpu_baseline(base, list(range(min(args.cpu_heads, cfg.heads))), args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
