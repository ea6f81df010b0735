#!/usr/bin/env python3
"""Sparse decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over one batch, in one call
(``jssa_decode_step``): append the new token's K/V row and project its key,
then the sparse decode (subspace scores -> per-KV-head top-k -> gather-free
indexed attention with a log-sum-exp combine).  In the fused build the append
runs inside the scan launch.  Inputs are seeded synthetic tensors already
resident in HBM; two independent input sets alternate so that the bytes
touched between reuses exceed the 256 MB Infinity Cache.

Prints ONE JSON line on stdout (everything else goes to stderr).  ``value`` is
decode steps/s of the chosen workload (default: 128K context, k = 2048),
timed as K steps between two events with an event every ten steps for the
per-block spread.  Also reported: effective HBM GB/s (projected-key bytes +
selected K/V bytes per step) and its fraction of the 8 TB/s peak; the roofline
of the dominant kernel (the projected-key scan, from its launch's own start
and end events); the library's device diagnostics; the append timed on its
own; the dense full-KV decode on the same inputs; the attention stage
gather-free vs gather-then-attend over rotating index lists; per-KV-head vs
head-shared selection; a graph-captured layer stack where only every m-th
layer selects; recall statistics of the selection; the budget sweep
(k = 512, 8192) and the other workloads (a Llama-3-8B-shaped layer at 32K, the
ragged hybrid batch); and the CPU oracle timed on the host cores.

``--kp fp8`` keeps the projected-key cache in FP8 E4M3 (the pages' own
scoring-cache format) instead of the workload's bf16.  ``--calibrate-copy MB``
instead runs a plain device-to-device copy of MB mebibytes a few times and
exits: the known-size kernel whose hardware byte counters scale those of the
scan kernel.  ``--quick`` times the headline step and its roofline only.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public figure
METRIC = "sparse decode steps/s + effective HBM GB/s (% peak) at 128K, k=2048"
BLOCK = 10  # steps between the timed region's intermediate events


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ctx128k",
                    choices=["tiny", "llama8b_32k", "ctx128k", "hybrid_ragged", "mla"])
    ap.add_argument("--topk", type=int, default=None, help="override the budget k")
    ap.add_argument("--reduce", default="max", choices=["max", "mean"])
    ap.add_argument("--kp", default="native", choices=["native", "fp8"],
                    help="projected-key cache dtype: the workload's own (bf16 / f32) or FP8 E4M3")
    ap.add_argument("--sets", type=int, default=2, help="independent input sets rotated per step")
    ap.add_argument("--quick", action="store_true", help="the headline step and its roofline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense full-KV comparison")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the attention-stage, selection-variant and layer-stack comparisons")
    ap.add_argument("--no-sweep", action="store_true", help="skip the budget sweep and the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a device copy of MB MiB (counter calibration) and exit")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


def spread(xs):
    """Median, 10th / 90th percentiles and mean of a list of timings."""
    import numpy as np
    xs = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(xs)), 2), "p10": round(float(np.percentile(xs, 10)), 2),
            "p90": round(float(np.percentile(xs, 90)), 2), "mean": round(float(xs.mean()), 2), "n": int(xs.size)}


def up(x, dev):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


class Case:
    """One workload's descriptor, its device-resident input sets and the step's
    output buffers and workspace.  With ``keep_host`` the host copy of input
    set 0 is kept, with the step's new rows written into it as the device
    step writes them."""

    def __init__(self, J, w, kpt, reduce, n_sets, dev, keep_host=False):
        import numpy as np
        import torch
        from synth import generate, to_bf16_bits
        self.w = w
        dt = J.BF16 if w.dtype == "bf16" else J.F32
        self.dt, self.kpt = dt, kpt
        self.desc = J.Desc(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, d_k=w.d_k, d_v=w.d_v,
                           rank=w.rank, t_max=w.t_max, topk=w.topk, window=w.window, kv_dtype=dt, kp_dtype=kpt,
                           out_dtype=J.F32, reduce=reduce, layout=J.LAYOUT_MLA if w.mla else J.LAYOUT_GQA,
                           scale=w.scale)
        tdt = torch.bfloat16 if dt == J.BF16 else torch.float32
        kpdt = torch.uint8 if kpt == J.FP8_E4M3 else tdt
        store = (lambda x: to_bf16_bits(x)) if dt == J.BF16 else (lambda x: x)
        self.sets, self.host = [], None
        for si in range(n_sets):
            t0 = time.time()
            inp = generate(w, seed=w.seed + 100 * si)
            s = {k: up(inp[k], dev) for k in ("q", "P", "k_cache", "seq_lens")}
            s["v_cache"] = None if w.mla else up(inp["v_cache"], dev)  # MLA: the value is a prefix of K
            s["kp"] = torch.empty((w.batch, w.n_kv_heads, w.t_max, w.rank), dtype=kpdt, device=dev)
            J.append_projection(self.desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device=dev),
                                s["P"], s["k_cache"], s["kp"])
            # the new token of each step: written at position T_b - 1
            rng = np.random.default_rng(w.seed + 7 + si)
            kn = store(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_k)).astype(np.float32))
            vn = store(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32))
            s["k_new"] = up(kn, dev)
            s["v_new"] = None if w.mla else up(vn, dev)
            s["pos"] = (s["seq_lens"] - 1).contiguous()
            self.sets.append(s)
            if si == 0 and keep_host:
                pos = inp["seq_lens"].astype(np.int64) - 1
                for b in range(w.batch):
                    inp["k_cache"][b, pos[b]] = kn[b, 0]
                    if not w.mla:
                        inp["v_cache"][b, pos[b]] = vn[b, 0]
                self.host = {"inp": inp, "kn": kn, "vn": vn}
            del inp
            log(f"{w.name}: input set {si} generated and resident in {time.time() - t0:.1f}s")
        torch.cuda.synchronize()
        self.ws = J.workspace(self.desc, J.OP_DECODE, device=dev)
        self.out = torch.empty((w.batch, w.n_q_heads, w.d_v), device=dev)
        self.lse = torch.empty((w.batch, w.n_q_heads), device=dev)

    def step(self, J, i, events=None, desc=None, ws=None):
        s = self.sets[i % len(self.sets)]
        J.decode_step(desc or self.desc, s["k_new"], s["v_new"], s["pos"], s["q"], s["P"], s["kp"], s["k_cache"],
                      s["v_cache"], s["seq_lens"], self.out, self.lse, self.ws if ws is None else ws,
                      events=events)

    def decode_lists(self, J, si, idx, n_sel):
        s = self.sets[si]
        J.decode(self.desc, s["q"], s["P"], s["kp"], s["k_cache"], s["v_cache"], s["seq_lens"], self.out,
                 self.lse, self.ws, idx_out=idx, n_sel_out=n_sel)

    def bytes_per_step(self, J, topk=None):
        """(projected-key bytes scanned, selected K/V bytes, all K/V bytes) of
        one step; a latent row is counted once for MLA."""
        import numpy as np
        w = self.w
        k = w.topk if topk is None else topk
        L = self.sets[0]["seq_lens"].cpu().numpy().astype(np.int64)
        n_cand = np.maximum(L - w.window, 0)
        n_sel = np.minimum(w.window, L) + np.minimum(k, n_cand)
        eb = 2 if self.dt == J.BF16 else 4
        kp_eb = 1 if self.kpt == J.FP8_E4M3 else eb
        kp_bytes = int(n_cand.sum()) * w.n_kv_heads * w.rank * kp_eb
        row_bytes = w.d_k * eb if w.mla else (w.d_k + w.d_v) * eb
        return kp_bytes, int(n_sel.sum()) * w.n_kv_heads * row_bytes, int(L.sum()) * w.n_kv_heads * row_bytes


def timed_steps(J, case, steps, warmup, stream, desc=None, ws=None):
    """`warmup` untimed steps, then `steps` steps between two events with an
    event after every BLOCK steps: (us per step over the whole region, us per
    step of each block)."""
    import torch
    for i in range(warmup):
        case.step(J, i, desc=desc, ws=ws)
    torch.cuda.synchronize()
    sizes = [BLOCK] * (steps // BLOCK) + ([steps % BLOCK] if steps % BLOCK else [])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    evs[0].record(stream)
    done = 0
    for bi, n in enumerate(sizes):
        for _ in range(n):
            case.step(J, done, desc=desc, ws=ws)
            done += 1
        evs[bi + 1].record(stream)
    torch.cuda.synchronize()
    blocks = [evs[i].elapsed_time(evs[i + 1]) * 1e3 / n for i, n in enumerate(sizes)]
    return evs[0].elapsed_time(evs[-1]) * 1e3 / steps, blocks


def stage_events(J, case, reps, stream, desc=None, ws=None):
    """Per-stage times from the decode's own four stage events, median over
    `reps` steps.  [0] -> [1] brackets the scan launch alone (the launch's own
    start and end events)."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for row in evs:
        for e in row:
            e.record(stream)  # materialise the event objects
    torch.cuda.synchronize()
    for i in range(reps):
        case.step(J, i, events=evs[i], desc=desc, ws=ws)
    torch.cuda.synchronize()
    st = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(3)] for row in evs]) * 1e3
    return np.median(st, axis=0)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: this build runs "
              "the decode path on one GPU only (the multi-GPU sharding is a design note, not built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import token_level_sparse_dim_amd as J
    from synth import WORKLOADS, scaled

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    J.lib()  # fail loudly if the HIP library is missing

    w = WORKLOADS[args.workload]
    if args.topk is not None:
        w = scaled(w, topk=args.topk)
    dev = torch.device("cuda:0")
    dt = J.BF16 if w.dtype == "bf16" else J.F32
    reduce = J.REDUCE_MAX if args.reduce == "max" else J.REDUCE_MEAN
    kpt = J.FP8_E4M3 if args.kp == "fp8" else dt
    want_cpu = not args.no_cpu and not args.quick
    case = Case(J, w, kpt, reduce, args.sets, dev, keep_host=not args.quick)
    stream = torch.cuda.current_stream()

    # ---- timed region ------------------------------------------------------------------------
    J.workspace_status(case.ws)  # clear the diagnostics before the timed steps
    us_step, blocks = timed_steps(J, case, args.steps, args.warmup, stream)
    ms_step = us_step * 1e-3
    log(f"sparse step: {us_step:.2f} us (blocks of {BLOCK}: median {np.median(blocks):.2f}, "
        f"p10 {np.percentile(blocks, 10):.2f}, p90 {np.percentile(blocks, 90):.2f} us)")
    # the library's sticky device diagnostics over the warm-up and timed steps:
    # a bounded in-kernel wait that gave up would make the timed results wrong
    dstat = [int(x) for x in J.workspace_status(case.ws).cpu()]
    if dstat[J.STATUS_WAIT_TIMEOUT]:
        print(f"bench.py: a bounded device wait gave up during the timed steps ({dstat})", file=sys.stderr)
        sys.exit(3)

    # ---- per-stage breakdown from HIP events on the launch stream -------------------------------
    stage_us = stage_events(J, case, min(args.steps, 100), stream)
    # fused GQA build: the scan launch, the select/attend launch (its in-launch
    # merge included), the two back-to-back closing events (their own cost);
    # MLA: score scan, candidate pass, selection + attention + merge
    names = ["score_scan", "candidates", "select+attention+merge"] if w.mla else \
        ["scan", "select_attend_merge", "event_pair"]
    log("stage events (us): " + ", ".join(f"{n}={v:.2f}" for n, v in zip(names, stage_us)))

    # ---- bytes -------------------------------------------------------------------------------
    kp_bytes, sel_bytes, dense_bytes = case.bytes_per_step(J)
    eff_bytes = kp_bytes + sel_bytes
    eff_gbps = eff_bytes / (ms_step * 1e-3) / 1e9
    scan_us = float(stage_us[0])
    achieved = kp_bytes / (scan_us * 1e-6) / 1e9

    traffic = None
    kname = "mla_score_kernel" if w.mla else "scan_kernel"
    wl = args.workload + ("_kpfp8" if kpt == J.FP8_E4M3 else "")
    tpath = os.path.join(ROOT, "profiles", f"{kname}_{wl}_traffic.json")
    if os.path.exists(tpath):
        try:
            with open(tpath) as f:
                rec = json.load(f)
            from token_level_sparse_dim_amd.build import source_digest
            src = "mla.hip" if w.mla else "pipeline.hip"
            if rec.get("source_digest") == source_digest(src) and rec.get("topk") == w.topk:
                traffic = rec.get("hbm_bytes_per_launch")
        except Exception as exc:  # a stale or unreadable record reads as unmeasured
            log(f"traffic record ignored: {exc}")

    result = {
        "metric": METRIC, "value": round(1e3 / ms_step, 1), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == J.BF16 else "f32", "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": w.name + ("-kp-fp8" if kpt == J.FP8_E4M3 else ""), "batch": w.batch,
                   "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.d_k, "value_dim": w.d_v,
                   "layout": "mla" if w.mla else "gqa", "rank": w.rank, "context": w.t_max,
                   "topk": w.topk, "window": w.window, "reduce": args.reduce,
                   "kp_dtype": {J.BF16: "bf16", J.F32: "f32", J.FP8_E4M3: "fp8_e4m3"}[kpt],
                   "step": "append new token + fused sparse decode", "input_sets": args.sets},
        "step_us_blocks": dict(spread(blocks), block_steps=BLOCK),
        "eff_bytes_per_step": eff_bytes, "eff_GBps": round(eff_gbps, 1),
        "pct_peak": round(100.0 * eff_gbps / HBM_PEAK_GBPS, 2),
        "stage_events_us": {n: round(float(v), 2) for n, v in zip(names, stage_us)},
        "device_status": {"wait_timeouts": dstat[J.STATUS_WAIT_TIMEOUT],
                          "exact_reselections": dstat[J.STATUS_EXACT_REDO],
                          "range_split_scans": dstat[J.STATUS_RANGE_SPLIT],
                          "global_cut_rows": dstat[J.STATUS_GLOBAL_CUT],
                          "steps": args.warmup + args.steps},
        "roofline": {"kernel": "mla_score_kernel (MFMA projected-key scan + histogram)" if w.mla
                     else "scan_kernel (projected-key scan + candidate emission)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": kp_bytes, "avg_launch_us": round(scan_us, 2)},
    }
    if w.mla:
        # the score scan runs on the matrix cores: each projected query is split
        # into bf16 hi + lo terms, so the executed products are twice the
        # algorithmic 2 Hq r flops per candidate (MEAN: one query row in a
        # 16-row M-tile)
        rows_m = w.n_q_heads if reduce == J.REDUCE_MAX else 16
        n_cand = int(np.maximum(case.sets[0]["seq_lens"].cpu().numpy().astype(np.int64) - w.window, 0).sum())
        flops = 2 * 2 * rows_m * w.rank * n_cand
        tf = flops / (scan_us * 1e-6) / 1e12
        result["mfma_util"] = {"kernel": "mla_score_kernel", "executed_flops_per_launch": flops,
                               "algorithmic_flops_per_launch": flops // 2, "achieved_tflops": round(tf, 1),
                               "peak_tflops": 2500.0, "frac": round(tf / 2500.0, 4),
                               "counters": "profiles/mla_kernels_mfma.txt (SQ_VALU_MFMA_BUSY_CYCLES)"}
        log(f"mla_score_kernel: {tf:.0f} TFLOP/s bf16 MFMA ({100 * tf / 2500:.1f}% of the dense peak)")
    if args.quick:
        print(json.dumps(result), flush=True)
        return

    result["append"] = append_timing(J, case, stream, us_step)
    if not args.no_dense:
        result["dense"] = dense_timing(J, case, stream, max(10, args.steps // 4), dense_bytes, ms_step)
    if not args.no_ablation:
        result["attention_stage"] = attention_ablation(J, case, stream)
        if not w.mla:
            result["selection_variant"] = selection_variant(J, case, stream, max(20, args.steps // 4))
            result["layer_stack"] = layer_stack(J, case, stream)
    if not w.mla:
        result["sanity"] = sanity(J, case)
    if not args.no_sweep and args.workload == "ctx128k" and args.topk is None:
        result["sweep"] = sweep(J, case, stream, args, reduce, kpt)
    if want_cpu:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, "fp8" if kpt == J.FP8_E4M3 else w.dtype)
    print(json.dumps(result), flush=True)


def timed_calls(fn, reps, stream, warm=3):
    """Average us of `reps` back-to-back calls fn(i) between two events."""
    import torch
    for i in range(warm):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def append_timing(J, case, stream, us_step, reps=100):
    """The step's append alone (jssa_append_kv of one token per sequence) and
    the decode without it (jssa_decode), beside the one-call step."""
    def append(i):
        s = case.sets[i % len(case.sets)]
        J.append_kv(case.desc, s["k_new"], s["v_new"], s["pos"], s["P"], s["k_cache"], s["v_cache"], s["kp"])

    def decode(i):
        s = case.sets[i % len(case.sets)]
        J.decode(case.desc, s["q"], s["P"], s["kp"], s["k_cache"], s["v_cache"], s["seq_lens"], case.out,
                 case.lse, case.ws)

    t_app, t_dec = timed_calls(append, reps, stream), timed_calls(decode, reps, stream)
    log(f"append alone {t_app:.2f} us, decode without append {t_dec:.2f} us, one-call step {us_step:.2f} us")
    return {"append_alone_us": round(t_app, 2), "decode_without_append_us": round(t_dec, 2),
            "step_us": round(us_step, 2), "reps": reps,
            "note": "the one-call step writes and projects the new rows inside its scan launch"}


def dense_timing(J, case, stream, reps, dense_bytes, ms_step):
    """The dense full-KV decode (jssa_dense_decode) on the same input sets."""
    wsd = J.workspace(case.desc, J.OP_DENSE, device=case.out.device)

    def dense(i):
        s = case.sets[i % len(case.sets)]
        J.dense_decode(case.desc, s["q"], s["k_cache"], s["v_cache"], s["seq_lens"], case.out, case.lse, wsd)

    us = timed_calls(dense, reps, stream)
    gbps = dense_bytes / (us * 1e-6) / 1e9
    log(f"dense: {us:.1f} us/step ({gbps:.0f} GB/s), sparse speedup {us / (ms_step * 1e3):.2f}x")
    return {"ms_per_step": round(us * 1e-3, 5), "GBps": round(gbps, 1),
            "pct_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
            "speedup_sparse_vs_dense": round(us / (ms_step * 1e3), 3), "reps": reps}


def rotating_lists(J, case, n_lists):
    """Index lists for the attention comparison: the decode's own lists of
    each input set, then sorted uniform random lists of the same sizes, so
    that the rows touched over one rotation exceed the 256 MB Infinity Cache."""
    import numpy as np
    import torch
    w, dev = case.w, case.out.device
    S = w.topk + w.window
    lists = []
    for si in range(len(case.sets)):
        idx = torch.full((w.batch, w.n_kv_heads, S), -1, dtype=torch.int32, device=dev)
        n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev)
        case.decode_lists(J, si, idx, n_sel)
        lists.append((si, idx, n_sel))
    L = case.sets[0]["seq_lens"].cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(11)
    while len(lists) < n_lists:
        si = len(lists) % len(case.sets)
        idx = np.full((w.batch, w.n_kv_heads, S), -1, np.int32)
        n_sel = np.zeros((w.batch, w.n_kv_heads), np.int32)
        for b in range(w.batch):
            nc = max(int(L[b]) - w.window, 0)
            kk, nw = min(w.topk, nc), min(w.window, int(L[b]))
            for h in range(w.n_kv_heads):
                sel = np.sort(rng.choice(nc, kk, replace=False)) if kk else np.zeros(0, np.int64)
                row = np.concatenate([sel, np.arange(int(L[b]) - nw, int(L[b]))])
                idx[b, h, :row.size] = row
                n_sel[b, h] = row.size
        lists.append((si, torch.from_numpy(idx).to(dev), torch.from_numpy(n_sel).to(dev)))
    torch.cuda.synchronize()
    return lists


def attention_ablation(J, case, stream, n_lists=8, rounds=9):
    """The attention-stage comparison of JSSA summary section 4.7 (the same
    selected tokens attended gather-free vs gathered first) over a rotation of
    `n_lists` index lists: (a) the stand-alone gather-free indexed attention,
    (b) the gather of the selected K/V rows into packed buffers followed by
    the dense decode over them.  Both arms get the same warm-up and
    workspace-per-op; they alternate round by round, a round timing one pass
    over all lists; medians and spreads over the rounds."""
    import torch
    w, dev, desc = case.w, case.out.device, case.desc
    S = w.topk + w.window
    lists = rotating_lists(J, case, n_lists)
    kv = case.sets[0]["k_cache"].dtype
    Kg = torch.empty((w.batch, S, w.n_kv_heads, w.d_k), dtype=kv, device=dev)
    Vg = None if w.mla else torch.empty((w.batch, S, w.n_kv_heads, w.d_v), dtype=kv, device=dev)
    lens = torch.empty((w.batch,), dtype=torch.int32, device=dev)
    pdesc = dataclasses.replace(desc, t_max=S, topk=S, window=0)  # the packed rows as a cache
    ws_a, ws_d = J.workspace(desc, J.OP_ATTN, device=dev), J.workspace(pdesc, J.OP_DENSE, device=dev)

    def free(si, idx, n_sel):
        s = case.sets[si]
        J.indexed_attn(desc, s["q"], s["k_cache"], s["v_cache"], idx, n_sel, case.out, case.lse, ws_a)

    def gather(si, idx, n_sel):
        s = case.sets[si]
        J.gather_kv(desc, s["k_cache"], s["v_cache"], idx, n_sel, Kg, Vg, lens)
        J.dense_decode(pdesc, s["q"], Kg, Vg, lens, case.out, case.lse, ws_d)

    def one_round(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for li in lists:
            fn(*li)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / len(lists)

    for fn in (free, gather):  # the same warm-up for both arms
        for _ in range(2):
            for li in lists:
                fn(*li)
    torch.cuda.synchronize()
    t_free, t_gath = [], []
    for r in range(rounds):
        arms = (free, gather) if r % 2 == 0 else (gather, free)
        for fn in arms:
            (t_free if fn is free else t_gath).append(one_round(fn))
    a, b = spread(t_free), spread(t_gath)
    res = {"gather_free_us": a, "gather_then_attend_us": b,
           "gather_free_speedup": round(b["median"] / a["median"], 3), "lists": n_lists, "rounds": rounds,
           "note": "the arms alternate (order swapped every round); a round is one pass over the rotating lists"}
    log(f"attention stage: gather-free {a['median']:.2f} us, gather-then-attend {b['median']:.2f} us "
        f"({res['gather_free_speedup']:.2f}x)")
    return res


def selection_variant(J, case, stream, reps):
    """Per-KV-head sets (the method's) against head-shared soft voting (one
    set per sequence; JSSA summary section E.3) on the same fp32 scores: the
    stand-alone selection of each, then the indexed attention over each
    selection (same k, the same bytes per KV head).  Averages over `reps`."""
    import torch
    w, dev, desc = case.w, case.out.device, case.desc
    s = case.sets[0]
    S = w.topk + w.window
    scores = torch.empty((w.batch, w.n_kv_heads, w.t_max), device=dev)
    J.score(desc, s["q"], s["P"], s["kp"], s["seq_lens"], scores)
    idx_ph = torch.full((w.batch, w.n_kv_heads, S), -1, dtype=torch.int32, device=dev)
    n_ph = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev)
    idx_sh, n_sh = torch.full_like(idx_ph, -1), torch.zeros_like(n_ph)
    ws_t, ws_v = J.workspace(desc, J.OP_TOPK, device=dev), J.workspace(desc, J.OP_VOTE, device=dev)
    ws_a = J.workspace(desc, J.OP_ATTN, device=dev)
    t_sel_ph = timed_calls(lambda i: J.topk(desc, scores, s["seq_lens"], idx_ph, n_ph, ws_t), reps, stream)
    t_sel_sh = timed_calls(lambda i: J.vote_select(desc, scores, s["seq_lens"], idx_sh, n_sh, ws_v), reps, stream)
    t_att_ph = timed_calls(lambda i: J.indexed_attn(desc, s["q"], s["k_cache"], s["v_cache"], idx_ph, n_ph,
                                                    case.out, case.lse, ws_a), reps, stream)
    t_att_sh = timed_calls(lambda i: J.indexed_attn(desc, s["q"], s["k_cache"], s["v_cache"], idx_sh, n_sh,
                                                    case.out, case.lse, ws_a), reps, stream)
    distinct = int(torch.unique(idx_ph[0, :, :int(n_ph[0, 0])]).numel())
    log(f"selection: per-KV-head top-k {t_sel_ph:.2f} us + attention {t_att_ph:.2f} us; head-shared vote "
        f"{t_sel_sh:.2f} us + attention {t_att_sh:.2f} us")
    return {"per_kv_head": {"select_us": round(t_sel_ph, 2), "attention_us": round(t_att_ph, 2)},
            "head_shared_vote": {"select_us": round(t_sel_sh, 2), "attention_us": round(t_att_sh, 2)},
            "distinct_tokens_seq0_per_kv_head_sets": distinct, "reps": reps}


def layer_stack(J, case, stream, n_layers=4, replays=30):
    """A stack of layers each decoding the step's token (JSSA summary
    appendix C: tokens are selected at indexer layers and the layers after
    them reuse those indices).  Every m-th layer is an indexer layer
    (jssa_decode_step on its own projected-key cache), the others call
    jssa_reuse_step on the latest indexer layer's lists.  Each layer has its
    own K/V caches (input set 0 rotated along the tokens) and its own query;
    the whole stack is captured in one HIP graph and replayed.  Time per
    replay and per layer for m = 1, 2, 4."""
    import torch
    w, dev, desc = case.w, case.out.device, case.desc
    base = case.sets[0]
    S = w.topk + w.window
    layers = []
    for l in range(n_layers):
        K = torch.roll(base["k_cache"], shifts=4099 * l, dims=1) if l else base["k_cache"]
        V = torch.roll(base["v_cache"], shifts=4099 * l, dims=1) if l else base["v_cache"]
        kp = torch.empty_like(base["kp"])
        J.append_projection(desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device=dev), base["P"], K, kp)
        layers.append({"K": K, "V": V, "kp": kp, "q": torch.roll(base["q"], shifts=l, dims=1).contiguous(),
                       "idx": torch.zeros((w.batch, w.n_kv_heads, S), dtype=torch.int32, device=dev),
                       "n_sel": torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev),
                       "out": torch.empty_like(case.out), "lse": torch.empty_like(case.lse)})
    ws = J.workspace(desc, J.OP_DECODE, device=dev)
    torch.cuda.synchronize()

    def stack(m):
        src = None
        for l, y in enumerate(layers):
            if l % m == 0:
                J.decode_step(desc, base["k_new"], base["v_new"], base["pos"], y["q"], base["P"], y["kp"], y["K"],
                              y["V"], base["seq_lens"], y["out"], y["lse"], ws, idx_out=y["idx"],
                              n_sel_out=y["n_sel"])
                src = y
            else:
                J.reuse_step(desc, base["k_new"], base["v_new"], base["pos"], y["q"], y["K"], y["V"], src["idx"],
                             src["n_sel"], y["out"], y["lse"], ws)

    res = {"layers": n_layers, "replays": replays, "captured": "one HIP graph per stack"}
    for m in (1, 2, 4):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                stack(m)  # eager warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            stack(m)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / replays
        res[f"indexer_every_{m}"] = {"stack_us": round(us, 2), "per_layer_us": round(us / n_layers, 2)}
        log(f"layer stack ({n_layers} layers, an indexer layer every {m}): {us:.1f} us per replay, "
            f"{us / n_layers:.2f} us per layer")
        del g
    res["wait_timeouts"] = int(J.workspace_status(ws).cpu()[J.STATUS_WAIT_TIMEOUT])
    del layers, ws
    torch.cuda.empty_cache()
    return res


def sanity(J, case, rows=((0, 0), (1, 3), (2, 5), (3, 7))):
    """Recall statistics of the selection on sampled (sequence, KV head) rows
    of input set 0, from the device's own index lists: the fraction of the
    planted needles selected, and the overlap of the subspace top-k with the
    top-k of the exact full-dimensional scores (max over the group of
    q_g . K_t).  Host-side numpy on the host copy of the inputs."""
    import numpy as np
    import torch
    from synth import bf16_bits_to_f32
    w = case.w
    inp = case.host["inp"]
    S = w.topk + w.window
    idx = torch.full((w.batch, w.n_kv_heads, S), -1, dtype=torch.int32, device=case.out.device)
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device=case.out.device)
    case.decode_lists(J, 0, idx, n_sel)
    gi = idx.cpu().numpy()
    L = inp["seq_lens"].astype(np.int64)
    G = w.group
    as32 = bf16_bits_to_f32 if w.dtype == "bf16" else (lambda x: x.astype(np.float32))
    hits = total = 0
    overlap = []
    for b, h in rows:
        if b >= w.batch or h >= w.n_kv_heads:
            continue
        nc = max(int(L[b]) - w.window, 0)
        kk = min(w.topk, nc)
        if kk == 0:
            continue
        sel = set(gi[b, h, :kk].tolist())
        nd = inp["needles"][b, h]
        hits += sum(int(t) in sel for t in nd)
        total += nd.size
        K = as32(inp["k_cache"][b, :nc, h, :]).astype(np.float64)
        qg = as32(inp["q"][b, h * G:(h + 1) * G]).astype(np.float64)
        exact = (K @ qg.T).max(axis=1)
        top = np.argpartition(-exact, kk - 1)[:kk]
        overlap.append(len(sel & set(top.tolist())) / kk)
    res = {"needle_recall": round(hits / max(total, 1), 4), "needles": int(total),
           "subspace_vs_exact_topk_overlap": round(float(np.mean(overlap)), 4) if overlap else None,
           "rows": len(overlap)}
    log(f"sanity: needle recall {res['needle_recall']:.3f} of {total}, subspace vs exact top-k overlap "
        f"{res['subspace_vs_exact_topk_overlap']}")
    return res


def sweep(J, case, stream, args, reduce, kpt):
    """The budget at 128K swept to k = 512 and k = 8192, then the other
    workloads: one Llama-3-8B-shaped layer at 32K (batch 8) and the ragged
    hybrid batch (16 sequences of 8K..128K, window 512).  Each entry: the
    one-call step timed as the headline (blocks of ten), its stage events and
    the device diagnostics."""
    import torch
    from synth import WORKLOADS
    res = {}
    steps = max(50, args.steps // 2)

    def record(name, c, desc, ws, topk=None):
        J.workspace_status(ws)
        us, blocks = timed_steps(J, c, steps, 10, stream, desc=desc, ws=ws)
        st = stage_events(J, c, 30, stream, desc=desc, ws=ws)
        dstat = [int(x) for x in J.workspace_status(ws).cpu()]
        kp_b, sel_b, _ = c.bytes_per_step(J, topk)
        gbps = (kp_b + sel_b) / (us * 1e-6) / 1e9
        res[name] = {"workload": c.w.name, "batch": c.w.batch, "context": c.w.t_max, "topk": topk or c.w.topk,
                     "window": c.w.window, "us_per_step": round(us, 2), "steps_per_s": round(1e6 / us, 1),
                     "step_us_blocks": spread(blocks), "eff_GBps": round(gbps, 1),
                     "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                     "scan_kernel_us": round(float(st[0]), 2),
                     "scan_GBps": round(kp_b / (float(st[0]) * 1e-6) / 1e9, 1),
                     "select_attend_us": round(float(st[1]), 2),
                     "device_status": dict(zip(["wait_timeouts", "exact_reselections", "range_split_scans",
                                                "global_cut_rows"], dstat)), "steps": steps}
        log(f"sweep {name}: {us:.2f} us/step, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}%), scan "
            f"{st[0]:.2f} us, select/attend {st[1]:.2f} us")

    for k in (512, 8192):
        d = dataclasses.replace(case.desc, topk=k)
        ws = J.workspace(d, J.OP_DECODE, device=case.out.device)
        record(f"ctx128k_k{k}", case, d, ws, topk=k)
        del ws
    for name in ("llama8b_32k", "hybrid_ragged"):
        c = Case(J, WORKLOADS[name], kpt, reduce, 2 if name == "llama8b_32k" else 1, case.out.device)
        record(name, c, c.desc, c.ws)
        del c
        torch.cuda.empty_cache()
    return res


def cpu_baseline(case, budget_s, kp_dtype):
    """The fp64 oracle on one whole step of input set 0: the new token's K/V
    rows written and its key projected into the stored projected-key cache,
    then subspace scores, full-sort top-k and exact softmax attention for every
    sequence and KV head; repeated within the time budget, median per step.
    The oracle's projection of the cached keys is set-up, untimed."""
    import numpy as np
    from oracle import jssa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count() or 1
    w = case.w
    inp, kn, vn = case.host["inp"], case.host["kn"], case.host["vn"]
    seq = inp["seq_lens"]
    pos = seq.astype(np.int64) - 1
    t0 = time.perf_counter()
    kp, _ = O.project_keys(inp["k_cache"], inp["P"], seq, kp_dtype)
    log(f"cpu oracle: projected-key cache built in {time.perf_counter() - t0:.1f}s (set-up)")
    K, V = inp["k_cache"], (inp["k_cache"][..., :w.d_v] if w.mla else inp["v_cache"])
    one = np.ones(w.batch, np.int64)
    times, t_all = [], time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_all < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        for b in range(w.batch):  # the new rows, in place
            K[b, pos[b]] = kn[b, 0]
            if not w.mla:
                V[b, pos[b]] = vn[b, 0]
        new_kp, _ = O.project_keys(kn, inp["P"], one, kp_dtype)
        for b in range(w.batch):
            kp[b, :, pos[b]] = new_kp[b, :, 0]
        O.decode(inp["q"], inp["P"], kp, K, V, seq, w.topk, w.window, w.scale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > 3 * budget_s:
            break
    med = float(np.median(times))
    log(f"cpu oracle: {med:.3f}s per step (median of {len(times)}), {blas} BLAS threads, {host_cores} host cores")
    return {"value": round(1.0 / med, 4), "unit": "steps/s", "cores": blas, "host_cores": host_cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"one whole step of input set 0 (all {w.batch} sequences x {w.n_kv_heads} KV heads, "
                      f"T up to {int(seq.max())}: new rows written and projected, scores, top-k, attention), "
                      f"median of {len(times)} runs; cores = the BLAS threads of the oracle's numpy "
                      f"(its elementwise work runs on one)"}


if __name__ == "__main__":
    main()
