#!/usr/bin/env python3
"""Benchmark of the block-sparse video attention hot path on one MI355X.

One step is one pass of the whole path over one synthetic layer input, with
inputs already resident in HBM:
  radial workloads: build_mask_radial -> compact_block_lists -> sparse_attn_fwd
  pooled workload:  build_mask_pooled -> compact_block_lists -> sparse_attn_fwd
  skip workload:    compact_block_lists (all tiles minus carried skips)
                    -> sparse_attn_fwd (with tile gaps) -> update_skip_mask,
                    one denoising step per bench step (cycling the 10 steps)
Prints one JSON line: computed-tile TFLOP/s of the step, the forward kernel's
ms per call and % of the bf16 MFMA peak, the roofline of the forward kernel
(timed with HIP events on the stream it runs on) and the fp64 CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps 20] [--warmup 3] [--workload wan14b_720p]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse_attn_fwd ms/call + computed-tile TFLOPS as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
MI355X_SIMDS = 1024         # 256 compute units x 4 SIMDs
MI355X_XCDS = 8
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_flashattention_amd", "csrc",
                          "attn_bf16.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def tile_flops(row_ptr: np.ndarray, kv_idx: np.ndarray, N: int, Bq: int, Bk: int, d: int,
               nQ: int, reps: int) -> float:
    """4 d |R_a| |C_c| summed over listed tiles (true ragged sizes), times reps
    (the (b, h) pairs a shared list serves)."""
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    a = rows % nQ
    ra = np.minimum(N, (a + 1) * Bq) - a * Bq
    cc = np.minimum(N, (kv_idx.astype(np.int64) + 1) * Bk) - kv_idx.astype(np.int64) * Bk
    return 4.0 * d * float(np.sum(ra * cc)) * reps


def pyramid_flops(row_ptr, kv_idx, kv_q, N, Bq, Bk, d, nQ, rb) -> float:
    """4 d |R_a| (keys of the selected eighths) summed over pyramid tiles; a
    level-l tile's keys are pooled rows, N >> l of them in level l."""
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    a = rows % nQ
    ra = np.minimum(N, (a + 1) * Bq) - a * Bq
    ab = kv_idx.astype(np.int64)
    lev = np.searchsorted(np.asarray(rb[1:]), ab, side="right")
    start = (ab - np.asarray(rb)[lev]) * Bk
    valid = np.clip((N >> lev) - start, 0, Bk)
    keys = np.zeros_like(ab)
    for e in range(8):
        on = (kv_q.astype(np.int64) >> e) & 1
        keys += on * np.clip(valid - (Bk // 8) * e, 0, Bk // 8)
    return 4.0 * d * float(np.sum(ra * keys))


def source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stratified_rows(BH: int, nQ: int, per_head: int, N: int, bq: int, F: int, rng) -> np.ndarray:
    """Row blocks for the CPU baseline, per head: the first, the last (ragged), about a
    quarter of them straddling a frame boundary (F tokens per frame), the rest uniform."""
    straddle = [a for a in range(nQ) if (a * bq) // F != (min(N, (a + 1) * bq) - 1) // F]
    picks = []
    for bh in range(BH):
        pick = {0, nQ - 1}
        if straddle:
            pick |= set(rng.choice(straddle, size=min(len(straddle), max(1, per_head // 4)),
                                   replace=False).tolist())
        free = [a for a in range(nQ) if a not in pick]
        more = max(0, min(len(free), per_head - len(pick)))
        pick |= set(rng.choice(free, size=more, replace=False).tolist())
        picks += [bh * nQ + a for a in sorted(pick)]
    return np.array(picks, dtype=np.int64)


def variant_key(args, w) -> str:
    """Name of a measured configuration: the workload plus every option that
    changes what the forward kernel runs on (a counter record is kept per
    key)."""
    parts = [w.name]
    if w.mask == "skip":
        parts.append(f"tau={args.tau_schedule or w.tau}")
        parts.append(f"order={args.order}")
        if args.share_after is not None:
            parts.append(f"share={args.share_after}")
    if args.pooled_mode is not None:
        parts.append(f"mode={args.pooled_mode}:param={args.pooled_param}")
    if args.token_order:
        parts.append(f"order={args.token_order}")
    if args.pyramid:
        parts.append(f"pyramid={args.pyramid}")
    return ":".join(parts)


def _load_records() -> dict:
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    return t.get("records", {}) if isinstance(t, dict) else {}


def counters_for(key: str) -> dict:
    """The counter record of profiles/traffic.json for this configuration when it was taken on
    this kernel source, else {}."""
    t = _load_records().get(key, {})
    if t.get("source_sha256") != source_sha():
        return {}
    return t


def _counter_mean(folder: str, kernel_substr: str, counter: str,
                  window: tuple = (0, None)) -> tuple[float, int]:
    """Mean per-dispatch value of a rocprofv3 counter over the dispatches of a kernel, taking
    only the dispatches window[0]:window[1] of that kernel in dispatch order."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (f, int(r["Dispatch_Id"]))
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    sel = [vals[k] for k in sorted(vals)][window[0]:window[1]]
    if not sel:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {folder} "
                         f"(window {window})")
    return float(np.mean(sel)), len(sel)


def ingest_counters(key: str, window: tuple, fetch_dir: str, write_dir: str, copy_f: str,
                    copy_w: str, sq_dir: str = None):
    """HBM bytes per forward launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for a device copy of 1 GiB each way. With the
    folder of a run that took SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and TA_BUSY_avr it
    also records the fraction of elapsed cycles in which the matrix cores are busy (busy
    cycles summed over the 1,024 SIMDs over 1,024 x elapsed cycles per XCD, GRBM_GUI_ACTIVE
    being summed over the 8 XCDs), the texture-address busy fraction and the L2 hit rate. Stored under the
    configuration's key in profiles/traffic.json. Only the forward dispatches of the timed
    steps count (window: their range in the run's dispatch order)."""
    fetch, nf = _counter_mean(fetch_dir, "attn_bf16_kernel", "FETCH_SIZE", window)
    write, nw = _counter_mean(write_dir, "attn_bf16_kernel", "WRITE_SIZE", window)
    cf, _ = _counter_mean(copy_f, "copyBuffer", "FETCH_SIZE")
    cw, _ = _counter_mean(copy_w, "copyBuffer", "WRITE_SIZE")
    kib = float(1 << 20)  # 1 GiB in KiB, each way
    f_fetch, f_write = kib / cf, kib / cw
    traffic = (fetch * f_fetch + write * f_write) * 1024.0
    out = {"source_sha256": source_sha(),
           "kernel": "attn_bf16_kernel", "dispatches": [nf, nw],
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "copy_fetch_kib_per_gib": cf, "copy_write_kib_per_gib": cw,
           "fetch_scale": f_fetch, "write_scale": f_write,
           "traffic_bytes_per_launch": traffic}
    if sq_dir:
        busy, _ = _counter_mean(sq_dir, "attn_bf16_kernel", "SQ_VALU_MFMA_BUSY_CYCLES", window)
        gui, _ = _counter_mean(sq_dir, "attn_bf16_kernel", "GRBM_GUI_ACTIVE", window)
        out["mfma_busy_cycles"] = busy
        out["grbm_gui_active"] = gui
        out["mfma_busy_frac"] = busy / (MI355X_SIMDS * gui / MI355X_XCDS)
        try:
            ta, _ = _counter_mean(sq_dir, "attn_bf16_kernel", "TA_BUSY_avr", window)
            out["ta_busy_frac"] = ta / (gui / MI355X_XCDS)
        except SystemExit:
            pass
        try:
            hit, _ = _counter_mean(sq_dir, "attn_bf16_kernel", "TCC_HIT_sum", window)
            miss, _ = _counter_mean(sq_dir, "attn_bf16_kernel", "TCC_MISS_sum", window)
            out["l2_hit_frac"] = hit / max(1.0, hit + miss)
        except SystemExit:
            pass
    recs = _load_records()
    recs[key] = out
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"records": recs}, f, indent=1, sort_keys=True)
    print(json.dumps({key: out}))


def _trace_durations(folder: str, kernel_substr: str) -> list:
    """Durations (ms) of the dispatches of a kernel, in dispatch order, from a rocprofv3
    --kernel-trace csv folder."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_substr in r["Kernel_Name"]:
                    rows.append((int(r["Dispatch_Id"]),
                                 (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6))
    if not rows:
        raise SystemExit(f"no {kernel_substr!r} dispatches in {folder}")
    return [d for _, d in sorted(rows)]


def summarize(args, key: str, w, trace_dir: str, bench_log: str):
    """Markdown summary of a profiled bench run: the forward's dispatches split by their role
    in the run (list capture, warm-up, timed, all-tiles, after a cache flush; the order
    bench.py issues them in), the timed calls' mean against the bench line's own HIP-event
    time, and the counter record of this configuration."""
    durs = _trace_durations(trace_dir, "attn_bf16_kernel")
    with open(bench_log) as fh:
        line = [l for l in fh if l.startswith("{") and '"metric"' in l][-1]
    b = json.loads(line)
    n_cap = w.steps if w.mask == "skip" else 1
    roles = ["list capture"] * n_cap + ["warm-up"] * b["warmup"] + ["timed"] * b["steps"]
    if b["config"].get("dense_ms_per_call") is not None:
        roles += ["all tiles"] * 3
    if b["ms_per_call_stats"].get("after_cache_flush") is not None:
        roles += ["after cache flush"] * 3
    if w.mask == "pooled" and b.get("cpu_baseline") is not None:
        roles += ["mask for the CPU sample"]
    if len(roles) != len(durs):
        raise SystemExit(f"{len(durs)} forward dispatches in the trace, {len(roles)} expected")
    timed = [d for r, d in zip(roles, durs) if r == "timed"]
    if w.mask == "skip":
        per = [p["computed_tflop"] * 1e12 for p in b["per_step"]]
        flops = [per[i % len(per)] for i in range(len(timed))]
    else:
        flops = [b["config"]["computed_tflop_per_call"] * 1e12] * len(timed)
    flop = float(np.mean(flops))
    t_mean = float(np.mean(timed))
    frac_trace = float(np.sum(flops)) / (np.sum(timed) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    out = [f"Configuration `{key}`, kernel source sha256 `{source_sha()}`.", "",
           "| dispatches | count | mean ms |", "|---|---|---|"]
    for role in dict.fromkeys(roles):
        ds = [d for r, d in zip(roles, durs) if r == role]
        out.append(f"| {role} | {len(ds)} | {np.mean(ds):.3f} |")
    out += ["", "| quantity | value |", "|---|---|",
            f"| computed-tile TFLOP per call | {flop / 1e12:.4f} |",
            f"| timed calls, trace mean | {t_mean:.3f} ms |",
            f"| timed calls, bench HIP events | {b['ms_per_call']:.3f} ms |",
            f"| fraction of 2,500 TFLOP/s, from the trace | {frac_trace:.4f} |",
            f"| fraction of 2,500 TFLOP/s, bench line | {b['roofline']['frac']:.4f} |",
            f"| trace / bench | {frac_trace / b['roofline']['frac']:.4f} |"]
    if w.mask == "skip":
        out += ["", "| step | listed tiles | sparsity | TFLOP | trace mean ms | % of peak |",
                "|---|---|---|---|---|---|"]
        for p in b["per_step"]:
            ds = [d for i, d in enumerate(timed) if i % len(b["per_step"]) == p["step"]]
            if ds:
                m = float(np.mean(ds))
                out.append(f"| {p['step']} | {p['listed_tiles']} | {p['tile_sparsity']:.3f} | "
                           f"{p['computed_tflop']:.4f} | {m:.3f} | "
                           f"{100 * p['computed_tflop'] / (m * 1e-3) / PEAK_BF16_TFLOPS:.1f} |")
        out.append("")
    c = counters_for(key)
    if c:
        tr = c["traffic_bytes_per_launch"]
        out += [f"| HBM traffic per launch (FETCH_SIZE x {c['fetch_scale']:.5f} + WRITE_SIZE x "
                f"{c['write_scale']:.5f}) | {tr / 1e9:.3f} GB |",
                f"| HBM bandwidth at the trace mean | {tr / (t_mean * 1e-3) / 1e9:.0f} GB/s "
                f"({100 * tr / (t_mean * 1e-3) / 1e9 / PEAK_HBM_GBS:.1f}% of 8 TB/s) |"]
        if "mfma_busy_frac" in c:
            out.append(f"| matrix cores busy (SQ_VALU_MFMA_BUSY_CYCLES / (1,024 x "
                       f"GRBM_GUI_ACTIVE / 8)) | {100 * c['mfma_busy_frac']:.1f}% |")
            out.append(f"| engine clock under the counter run (GRBM_GUI_ACTIVE / 8 per "
                       f"trace-mean call) | {c['grbm_gui_active'] / 8 / (t_mean * 1e-3) / 1e9:.2f} "
                       f"GHz |")
        if "ta_busy_frac" in c:
            out.append(f"| texture address unit busy (TA_BUSY_avr) | "
                       f"{100 * c['ta_busy_frac']:.1f}% |")
        if "l2_hit_frac" in c:
            out.append(f"| L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)) | "
                       f"{100 * c['l2_hit_frac']:.1f}% |")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--tau", type=float, default=None,
                    help="skip-carry threshold override (natural-log units; default: the "
                         "workload's)")
    ap.add_argument("--order", choices=("ascending", "radial"), default="ascending",
                    help="skip carry: visiting order of each row's key blocks (radial = "
                         "centre-out, the order the skip rule reaches the row max soonest in)")
    ap.add_argument("--tau-schedule", default=None, metavar="START:END",
                    help="skip carry: threshold per step, linear from START (step 0) to END "
                         "(last step), natural-log units; overrides --tau")
    ap.add_argument("--share-after", type=int, default=None, metavar="K",
                    help="skip carry: steps >= K share the skip set reached after step K-1 "
                         "(no tile gaps, no update, lists built once)")
    ap.add_argument("--pooled-mode", type=int, default=None, choices=(0, 1, 2, 3),
                    help="pooled workloads: selection rule (0 row top-k, 1 row cumulative mass, "
                         "2 head-wide top-k, 3 head-wide cumulative mass); default: the "
                         "workload's")
    ap.add_argument("--pooled-param", type=float, default=None,
                    help="pooled workloads: k or tau_p for --pooled-mode")
    ap.add_argument("--token-order", default=None, metavar="SPEC",
                    help="pooled workloads: gather Q/K/V into a token order before blocking "
                         "and scatter O back, inside the step: axes:A,B,C (slowest..fastest, "
                         "0 frame 1 row 2 column), boxes:T,H,W (box extent), paro (head h "
                         "takes axis order h mod 6), or choose (each head the axis order whose "
                         "pooled mask keeps the fewest tiles, chosen once before timing)")
    ap.add_argument("--pyramid", default=None, metavar="T0[,T1[,T2[,T3]]]",
                    help="pooled workloads: pyramid attention with these level thresholds "
                         "(cumulative mass; level l pools 2^l tokens); the step builds the "
                         "K/V levels, the level mask and the tile lists, then runs the forward")
    ap.add_argument("--cpu-rows", type=int, default=800,
                    help="row blocks in the CPU oracle sample (0 = skip)")
    ap.add_argument("--no-dense", action="store_true", help="skip the all-tiles timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR",
                    help="turn rocprofv3 --pmc output folders into this configuration's record "
                         "in profiles/traffic.json, no GPU work: FETCH_SIZE and WRITE_SIZE of "
                         "the configuration's bench run, the same two of --calibrate-copy-mib "
                         "1024, and optionally a run with SQ_VALU_MFMA_BUSY_CYCLES, "
                         "GRBM_GUI_ACTIVE and TA_BUSY_avr (4 or 5 folders)")
    ap.add_argument("--summarize", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="print a markdown summary of a rocprofv3 --kernel-trace run of this "
                         "configuration's bench (its folder and the bench's stdout), no GPU work")
    args = ap.parse_args()
    if args.ingest_counters or args.summarize:
        import synth
        w0 = synth.workload(args.workload)
        if args.tau is not None:
            import dataclasses
            w0 = dataclasses.replace(w0, tau=args.tau)
        key = variant_key(args, w0)
        if args.ingest_counters:
            if len(args.ingest_counters) not in (4, 5):
                raise SystemExit("--ingest-counters takes 4 or 5 folders")
            lo = (w0.steps if w0.mask == "skip" else 1) + args.warmup
            ingest_counters(key, (lo, lo + args.steps), *args.ingest_counters)
        else:
            summarize(args, key, w0, *args.summarize)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_flashattention_amd as bsa
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}))
        return

    w = synth.workload(args.workload)
    import dataclasses
    if args.tau is not None:
        w = dataclasses.replace(w, tau=args.tau)
    if args.pooled_mode is not None:
        if args.pooled_param is None:
            sys.exit("--pooled-mode needs --pooled-param")
        w = dataclasses.replace(w, pooled_mode=args.pooled_mode, pooled_param=args.pooled_param)
    log(f"workload {w.name}: B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} N={w.N} "
        f"Bq={w.Bq} Bk={w.Bk} mask={w.mask}")
    t0 = time.time()
    x = synth.make_qkv(w, step=0 if w.mask == "skip" else None)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    s = bsa.shape(w.B, w.H, w.d, w.T, w.Hs, w.Ws, w.Bq, w.Bk)
    nQ, nK, BH = s.nQ, s.nK, w.B * w.H
    o = torch.empty_like(q)
    lse = torch.empty(BH * w.N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    shared = 1 if w.mask == "radial" else 0
    R = nQ if shared else BH * nQ
    mask = torch.empty((nQ * nK) if shared else (BH * nQ * nK), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device=dev)
    kv_idx = torch.empty(R * nK, dtype=torch.int32, device=dev)
    ws = None
    step_inputs = None
    skip = gap = ones = None
    if w.mask == "pooled":
        ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=dev)
    order = bsa.ORDER_RADIAL if args.order == "radial" else bsa.ORDER_ASCENDING
    taus = None
    kv_asc = None
    if w.mask == "skip":
        ones = torch.ones(nQ * nK, dtype=torch.uint8, device=dev)
        skip = torch.zeros(BH * nQ * nK, dtype=torch.uint8, device=dev)
        gap = torch.empty(BH * nQ * nK, dtype=torch.float32, device=dev)
        if order != bsa.ORDER_ASCENDING:
            kv_asc = torch.empty(R * nK, dtype=torch.int32, device=dev)
        if args.tau_schedule:
            t_a, t_b = (float(x) for x in args.tau_schedule.split(":"))
            taus = [t_a + (t_b - t_a) * si / max(1, w.steps - 1) for si in range(w.steps)]
        else:
            taus = [w.tau] * w.steps
        step_inputs = [(q, k)]
        for st in range(1, w.steps):
            y = synth.make_step_qk(w, st)
            step_inputs.append((to_dev(y["q"]), to_dev(y["k"])))
        log(f"{w.steps} denoising-step inputs resident")

    perm = None
    vv = v
    if args.token_order:
        if w.mask != "pooled":
            sys.exit("--token-order applies to pooled workloads (radial masks are defined on "
                     "the (t, y, x) order)")
        import itertools
        orders = list(itertools.permutations(range(3)))
        perm = torch.empty(w.H * w.N, dtype=torch.int32, device=dev)   # one order per head
        spec = args.token_order
        chosen = None
        if spec == "choose":
            # per-head order chosen once, before timing, by the kept-tile count of the pooled
            # selection under each of the six axis orders
            dtc = bsa.BSA_BF16 if q.dtype == torch.bfloat16 else bsa.BSA_F32
            wso = torch.empty(bsa.bsa_token_orders_workspace_bytes(s, dtc), dtype=torch.uint8,
                              device=dev)
            och = torch.empty(w.H, dtype=torch.int32, device=dev)
            cnt = torch.empty((w.H, 6), dtype=torch.int64, device=dev)
            bsa.bsa_choose_token_orders(s, q, k, w.scale, w.pooled_mode, w.pooled_param, och,
                                        cnt, wso)
            torch.cuda.synchronize()
            chosen = och.cpu().tolist()
            log(f"chosen orders per head {chosen}; kept tiles identity "
                f"{cnt[:, 0].sum().item()}, chosen {cnt[torch.arange(w.H), och.long()].sum().item()}")
            del wso
        for h in range(w.H):
            sl = perm[h * w.N:(h + 1) * w.N]
            if spec == "choose":
                bsa.bsa_make_token_permutation(s, bsa.PERM_AXES, bsa.AXIS_ORDERS[chosen[h]], sl)
            elif spec == "paro":
                bsa.bsa_make_token_permutation(s, bsa.PERM_AXES, orders[h % 6], sl)
            else:
                kind, vals = spec.split(":")
                ax = [int(z) for z in vals.split(",")]
                bsa.bsa_make_token_permutation(
                    s, bsa.PERM_AXES if kind == "axes" else bsa.PERM_BOXES, ax, sl)
        qp, kp, vp, op = (torch.empty_like(q) for _ in range(4))
        vv = vp

    taus_pyr = None
    if args.pyramid:
        if w.mask != "pooled" or args.token_order:
            sys.exit("--pyramid applies to pooled workloads in (t, y, x) order")
        taus_pyr = [float(z) for z in args.pyramid.split(",")]
        n_lev = len(taus_pyr)
        prow = bsa.bsa_pyramid_rows(s, n_lev)
        kpyr = torch.empty((w.B, max(prow, 1), w.H, w.d), dtype=q.dtype, device=dev)
        vpyr = torch.empty_like(kpyr)
        rb_p = [0]
        for l in range(1, n_lev + 1):
            rb_p.append(rb_p[-1] + -(-(w.N >> (l - 1)) // w.Bk))
        cap_p = BH * nQ * rb_p[-1]
        kv_idx = torch.empty(cap_p, dtype=torch.int32, device=dev)
        kv_q = torch.empty(cap_p, dtype=torch.int32, device=dev)

    fwd_events = []
    aux_events = []  # skip carry: (kind, start, end, step) of compaction and update
    state = {"i": 0, "capture": None}

    def step(record: bool):
        if w.mask == "radial":
            bsa.bsa_build_mask_radial(s, w.h0, w.beta, mask)
            bsa.bsa_compact_block_lists(s, mask, 0, None, row_ptr, kv_idx)
            qq, kk_ = q, k
        elif w.mask == "pooled" and taus_pyr is not None:
            qq, kk_ = q, k
            bsa.bsa_build_kv_pyramid(s, n_lev, k, v, kpyr, vpyr)
            bsa.bsa_build_mask_pyramid(s, q, k, w.scale, taus_pyr, mask, ws)
            bsa.bsa_compact_pyramid_lists(s, n_lev, mask, nQ * nK, row_ptr, kv_idx, kv_q)
        elif w.mask == "pooled":
            qq, kk_ = q, k
            if perm is not None:
                for a, b in ((q, qp), (k, kp), (v, vp)):
                    bsa.bsa_permute_tokens(s, perm, w.N, 0, a, b)
                qq, kk_ = qp, kp
            bsa.bsa_build_mask_pooled(s, qq, kk_, w.scale, w.pooled_mode, w.pooled_param, mask,
                                      ws)
            bsa.bsa_compact_block_lists(s, mask, nQ * nK, None, row_ptr, kv_idx)
        else:
            si = state["i"] % w.steps
            if si == 0:
                skip.zero_()
            qq, kk_ = step_inputs[si]
            frozen = args.share_after is not None and si >= args.share_after
            if record:
                c0 = torch.cuda.Event(enable_timing=True)
                c1 = torch.cuda.Event(enable_timing=True)
                c0.record(stream)
            if not frozen or si == args.share_after:
                if kv_asc is None:
                    bsa.bsa_compact_block_lists(s, ones, 0, skip, row_ptr, kv_idx)
                else:
                    bsa.bsa_compact_block_lists(s, ones, 0, skip, row_ptr, kv_asc)
                    bsa.bsa_order_block_lists(s, order, row_ptr, 0, kv_asc, kv_idx)
            if record:
                c1.record(stream)
                aux_events.append(("compact", c0, c1, si))
        if state["capture"] is not None:
            torch.cuda.synchronize()
            rp_c = row_ptr.cpu().numpy().astype(np.int64)
            nz = int(rp_c[-1])
            state["capture"].append((rp_c, kv_idx[:nz].cpu().numpy(),
                                     kv_q[:nz].cpu().numpy() if taus_pyr is not None else None))
        use_gap = w.mask == "skip" and not frozen
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        if taus_pyr is not None:
            bsa.bsa_pyramid_attn_fwd(s, q, k, v, kpyr, vpyr, n_lev, o, lse, row_ptr, kv_idx,
                                     kv_q, w.scale)
        else:
            bsa.bsa_sparse_attn_fwd(s, qq, kk_, vv, op if perm is not None else o, lse, row_ptr,
                                    kv_idx, shared, w.scale, gap if use_gap else None)
        if record:
            e1.record(stream)
            fwd_events.append((e0, e1, state["i"] % max(1, w.steps)))
        if perm is not None:
            bsa.bsa_permute_tokens(s, perm, w.N, 1, op, o)
        if use_gap:
            if record:
                u0 = torch.cuda.Event(enable_timing=True)
                u1 = torch.cuda.Event(enable_timing=True)
                u0.record(stream)
            bsa.bsa_update_skip_mask(s, row_ptr, kv_idx, gap, taus[si], skip)
            if record:
                u1.record(stream)
                aux_events.append(("update", u0, u1, si))
        state["i"] += 1

    # lists of every distinct step, for the FLOP count (outside the timed region)
    nsteps_distinct = w.steps if w.mask == "skip" else 1
    state["i"] = 0
    state["capture"] = []
    for _ in range(nsteps_distinct):
        step(False)
    torch.cuda.synchronize()
    captured, state["capture"] = state["capture"], None
    if taus_pyr is not None:
        per_step_flops = [pyramid_flops(rp, kvh, qmh, w.N, w.Bq, w.Bk, w.d, nQ, rb_p)
                          for rp, kvh, qmh in captured]
    else:
        per_step_flops = [tile_flops(rp, kvh, w.N, w.Bq, w.Bk, w.d, nQ, BH if shared else 1)
                          for rp, kvh, _ in captured]
    per_step_tiles = [int(rp[-1]) for rp, _, _ in captured]
    rp = captured[-1][0]
    state["i"] = 0
    nnz_tiles = int(rp[-1]) if w.mask != "skip" else None
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    fwd_events.clear()
    aux_events.clear()
    state["i"] = 0
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    fwd_ms_each = [e0.elapsed_time(e1) for e0, e1, _ in fwd_events]
    fwd_ms = float(np.mean(fwd_ms_each))
    flops_each = [per_step_flops[si % nsteps_distinct] for _, _, si in fwd_events]
    flops_total = float(np.sum(flops_each))
    step_tflops = flops_total / (ms_step * args.steps * 1e-3) / 1e12
    fwd_tflops = flops_total / (np.sum(fwd_ms_each) * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms, forward {fwd_ms:.3f} ms/call "
        f"({fwd_tflops:.1f} TFLOP/s, {100 * fwd_tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")

    dense_speedup = None
    dense_ms = None
    if not args.no_dense and w.mask != "skip":
        reps = 2
        bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, None, None, 0, w.scale)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, None, None, 0, w.scale)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        dense_speedup = dense_ms / fwd_ms
        log(f"all tiles: {dense_ms:.3f} ms/call, dense-equivalent speedup {dense_speedup:.2f}x")

    # Forward after evicting the caches: write a 1 GiB buffer (beyond the 256 MB Infinity
    # Cache and the L2s), then time one call; the lists and inputs stay as in the last step.
    cold_ms = None
    if w.mask != "skip" and taus_pyr is None and perm is None:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(3):
            scratch.fill_(1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, row_ptr, kv_idx, shared, w.scale)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch
        cold_ms = float(np.median(cold))
        log(f"after a 1 GiB cache flush: {cold_ms:.3f} ms/call (median of 3)")

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same rows
    cpu = None
    if args.cpu_rows > 0:
        import oracle
        rng = np.random.default_rng(12345)
        if w.mask == "radial":
            mask_h = mask.cpu().numpy().reshape(nQ, nK)
            mhs = 0
        else:
            if w.mask == "skip":
                skip.zero_()
                bsa.bsa_compact_block_lists(s, ones, 0, skip, row_ptr, kv_idx)
                torch.cuda.synchronize()
                mask_h = np.ones((BH, nQ, nK), np.uint8)
            else:
                step(False)
                torch.cuda.synchronize()
                mask_h = mask.cpu().numpy().reshape(BH, nQ, nK)
            mhs = nQ * nK
        rows = stratified_rows(BH, nQ, max(4, args.cpu_rows // BH), w.N, w.Bq, w.Hs * w.Ws, rng)
        rr = rows % nQ
        ra = np.minimum(w.N, (rr + 1) * w.Bq) - rr * w.Bq
        per_row_keys = []
        for r in rows:
            bh, a = divmod(int(r), nQ)
            mrow = mask_h[a] if mhs == 0 else mask_h[bh, a]
            cs = np.nonzero(mrow)[0]
            per_row_keys.append(int(np.sum(np.minimum(w.N, (cs + 1) * w.Bk) - cs * w.Bk)))
        sample_flops = 4.0 * w.d * float(np.sum(ra * np.array(per_row_keys)))
        log(f"CPU oracle on {len(rows)} row blocks ({sample_flops / 1e9:.1f} GFLOP), "
            f"{oracle.num_threads()} threads")
        t0 = time.time()
        oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mask_h, mhs, rows=rows)
        cpu_s = time.time() - t0
        # the same count over every row block (the oracle computes kept tiles at full size)
        bsz = (np.minimum(w.N, (np.arange(nK) + 1) * w.Bk) - np.arange(nK) * w.Bk).astype(
            np.float64)
        rsz = (np.minimum(w.N, (np.arange(nQ) + 1) * w.Bq) - np.arange(nQ) * w.Bq).astype(
            np.float64)
        kept = (mask_h != 0).astype(np.float64) @ bsz
        full_flops = 4.0 * w.d * float(np.sum(kept * rsz)) * (BH if mhs == 0 else 1)
        cpu = {"value": sample_flops / cpu_s / 1e12, "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{len(rows)} of {BH * nQ} row blocks of {w.name} (first step's mask), "
                         f"stratified per head: first, last (ragged), frame-straddling and "
                         f"uniform ones; {sample_flops / 1e9:.1f} GFLOP fp64 in {cpu_s:.1f} s",
               "extrapolated_full_call_s": cpu_s * full_flops / sample_flops,
               "extrapolation": "sample time scaled by computed-tile flop of the whole call "
                                "(an extrapolation, not a measurement)"}
        log(f"CPU oracle: {cpu['value'] * 1e3:.3f} GFLOP/s")

    ctr = counters_for(variant_key(args, w))
    traffic = ctr.get("traffic_bytes_per_launch")
    out = {
        "metric": METRIC,
        "value": step_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_call": fwd_ms,
        "ms_per_call_stats": {"median": float(np.median(fwd_ms_each)),
                              "min": float(np.min(fwd_ms_each)),
                              "max": float(np.max(fwd_ms_each)),
                              "after_cache_flush": cold_ms},
        "pct_of_bf16_peak": 100.0 * fwd_tflops / PEAK_BF16_TFLOPS,
        "dense_equiv_speedup": dense_speedup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "head_dim": w.d,
            "grid_T_H_W": [w.T, w.Hs, w.Ws], "tokens": w.N, "block_q": w.Bq,
            "block_k": w.Bk, "mask": w.mask,
            "knobs": {"h0": w.h0, "decay_base": w.beta} if w.mask == "radial" else (
                {"mode": w.pooled_mode, "tau_p": w.pooled_param} if w.mask == "pooled"
                else {"tau": taus, "steps": w.steps, "order": args.order,
                      "share_after": args.share_after}),
            "token_order": args.token_order,
            "pyramid_levels_tau": taus_pyr,
            "kept_tiles": nnz_tiles,
            "tile_sparsity": (1.0 - nnz_tiles / (R * nK)) if nnz_tiles is not None else None,
            "computed_tflop_per_call": float(np.mean(per_step_flops)) / 1e12,
            "dense_ms_per_call": dense_ms,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": fwd_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": fwd_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "hbm_gbs": traffic / (fwd_ms * 1e-3) / 1e9 if traffic else None,
            "mfma_busy_frac": ctr.get("mfma_busy_frac"),
            "counters": variant_key(args, w) if ctr else None,
        },
        "cpu_baseline": cpu,
    }
    if w.mask == "skip":
        by = {}
        for (e0, e1, si), ms in zip(fwd_events, fwd_ms_each):
            by.setdefault(si, []).append(ms)
        aux = {}
        for kind, e0, e1, si in aux_events:
            aux.setdefault((kind, si), []).append(e0.elapsed_time(e1))
        def aux_ms(kind, si):
            v = aux.get((kind, si))
            return float(np.mean(v)) if v else None
        out["per_step"] = [{"step": si, "fwd_ms": float(np.mean(by[si])) if si in by else None,
                            "compact_ms": aux_ms("compact", si),
                            "update_ms": aux_ms("update", si),
                            "computed_tflop": per_step_flops[si] / 1e12,
                            "listed_tiles": per_step_tiles[si],
                            "tile_sparsity": 1.0 - per_step_tiles[si] / (R * nK)}
                           for si in range(nsteps_distinct)]
        log("per step (sparsity, fwd ms): " + ", ".join(
            f"{p['tile_sparsity']:.3f}/{p['fwd_ms']:.2f}" for p in out["per_step"]))
        log("per step (compact + order ms, update ms): " + ", ".join(
            f"{p['compact_ms'] or 0:.3f}/{p['update_ms'] or 0:.3f}" for p in out["per_step"]))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
