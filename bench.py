"""Throughput of one native-MTP speculative cycle on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload model_greedy]

One step = one whole cycle of the hot path over one batch of synthetic input:
k draft-head calls (first 64,000 rows of a 152,064 x 2560 bf16 head, one hidden row per
request), one verify pass over the k+1 = 8 rows, acceptance, and the commit of the
accepted row's recurrent-state snapshot (36 layers x 16 heads x 128 x 128 fp32 = 36 MiB
per snapshot, 8 snapshots) with the trim of rejected KV rows (12 layers, fp16 4 x 256).
Inputs are resident in HBM before the timed region.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense MFMA, bf16
METRIC = "verify cycles/s (k=7, V=152,064, d=2560 bf16) + achieved HBM GB/s vs peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "mfma_valu.json")
# sources the LM-head kernels are compiled from: counters taken on other sources are stale
KERNEL_SRCS = [os.path.join(ROOT, "speculative_decoding_head_amd", "csrc", f)
               for f in ("lmhead.hip", "lmhead_wide.hip", "lmhead_common.hpp", "common.hpp", "kernels.hpp")]

# recurrent state and KV per request (the model's 36 recurrent layers x 16 heads x 128x128
# fp32, 12 attention layers with fp16 4 x 256 KV rows)
STATE_LAYERS, STATE_HEADS, STATE_DIM = 36, 16, 128
KV_LAYERS, KV_HEADS, KV_DIM, KV_ROWS = 12, 4, 256, 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="model_greedy", choices=["model_greedy", "q4_greedy", "q4_sampled", "exact_sampled", "batched_commit",
                                                      "tiny_greedy", "tiny_sampled"])
    ap.add_argument("--cpu-cycles", type=int, default=0, help="oracle cycles for the CPU baseline (0 = auto)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record per-kernel HIP events in every N-th timed cycle (each event is a queue packet "
                         "that adds a few microseconds of gap, so timing every cycle would slow the cycles it times)")
    ap.add_argument("--rotate-heads", type=int, default=3,
                    help="after the timed region, time the draft head rotating over this many copies of the "
                         "head (each call reads weights no cache holds); 0 or 1 = skip")
    ap.add_argument("--planted-alpha", type=float, default=0.75,
                    help="after the timed region, time whole cycles whose acceptance depth is planted per "
                         "request with P(depth >= j) = alpha^j; 0 = skip")
    ap.add_argument("--extra-cycles", type=int, default=30, help="cycles timed by each extra measurement")
    ap.add_argument("--repeats", type=int, default=5,
                    help="after the timed region, time the same K cycles this many more times and report the "
                         "spread of their rates (value stays the first window)")
    ap.add_argument("--adaptive-cycles", type=int, default=200,
                    help="after the planted-acceptance cycles (one request only), run this many cycles whose "
                         "width the native controller picks, and as many at each fixed width 1..k, all "
                         "synchronising every cycle; 0 = skip")
    ap.add_argument("--draft-ids", type=int, default=0, metavar="N_TOP",
                    help="draft from an id list instead of the first n_draft ids: the N_TOP highest ids (a "
                         "special-token block at the end of the vocabulary) plus the lowest ones, n_draft in all, "
                         "gathered once into their own head; 0 = the first n_draft ids")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-commit", action="store_true", help="leave the commit out of the step")
    ap.add_argument("--overlap-commit", action="store_true",
                    help="run each cycle's commit on a second stream beside the next cycle's draft calls (the next "
                         "verify waits for it) instead of on the launch stream after the accept; measured slower: "
                         "the copy and the draft head share HBM")
    ap.add_argument("--no-read-peak", action="store_true", help="skip the 1 GiB read-ceiling measurement")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="model_greedy only: skip timing the 16 x 8-row batched cycle and the 4-bit head cycle")
    ap.add_argument("--row-major", action="store_true",
                    help="keep the head row-major instead of repacking it once into the tiled layout")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (the HBM counter reference)")
    ap.add_argument("--summarize-utilisation", nargs=2, action="append", metavar=("WORKLOAD", "CSV"),
                    help="turn a rocprofv3 --pmc MfmaUtil VALUBusy MfmaFlopsBF16 CSV of a run of WORKLOAD into "
                         "profiles/mfma_valu.json (repeat once per workload)")
    ap.add_argument("--summarize-counters", nargs=3, action="append", metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="turn the rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE) of a run of WORKLOAD into "
                         "profiles/traffic.json (repeat once per workload)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


KERNEL_KEYS = ("mtp_draft_head_kernel", "mtp_verify_logits_kernel", "mtp_verify_wide_kernel",
               "mtp_verify_wide_merge_kernel", "mtp_accept_sample_kernel", "mtp_commit_state_kernel")


def summarize_counters(runs) -> None:
    """Per-kernel HBM bytes per launch from rocprofv3 counter CSVs, per workload, scaled by
    the counters of a plain copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES) in the
    same run."""
    import csv
    from collections import defaultdict

    def load(path, counter):
        per = defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                per[row["Kernel_Name"]].append(float(row["Counter_Value"]) * 1024.0)   # KiB -> B
        return per

    def copy_kernel(per):
        # the calibration copy is the multiply-by-one elementwise kernel over COPY_BYTES
        cands = [k for k in per if "elementwise" in k and "Mul" in k]
        if not cands:
            raise SystemExit("no calibration copy kernel in the counter CSV (run bench.py --calibrate-copy)")
        return max(max(per[k]) for k in cands)

    out = {"source_digest": source_digest(), "copy_bytes": COPY_BYTES, "workloads": {}}
    for workload, fetch_csv, write_csv in runs:
        fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
        f_scale = COPY_BYTES / copy_kernel(fetch)
        w_scale = COPY_BYTES / copy_kernel(write)
        wl = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
        for name in fetch:
            short = next((key for key in KERNEL_KEYS if key + "<" in name or key + "(" in name), None)
            if short is None or short in wl["kernels"]:
                continue
            fb = float(np.median(fetch[name])) * f_scale
            wb = float(np.median(write.get(name, [0.0]))) * w_scale
            wl["kernels"][short] = {"fetch_bytes": int(fb), "write_bytes": int(wb), "bytes_per_launch": int(fb + wb),
                                    "launches": len(fetch[name]), "raw_kernel_name": name}
        out["workloads"][workload] = wl
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def summarize_utilisation(runs) -> None:
    """Per-kernel MFMA and VALU busy percentages and MFMA bf16 flops per launch (medians over
    the run's launches) from rocprofv3 counter CSVs, per workload."""
    import csv
    from collections import defaultdict

    out = {"source_digest": source_digest(), "workloads": {}}
    for workload, path in runs:
        per = defaultdict(lambda: defaultdict(list))
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                short = next((key for key in KERNEL_KEYS if key + "<" in name or key + "(" in name), None)
                if short is not None:
                    per[short][row["Counter_Name"]].append(float(row["Counter_Value"]))
        out["workloads"][workload] = {
            k: {"mfma_busy_pct": round(float(np.median(v["MfmaUtil"])), 2),
                "valu_busy_pct": round(float(np.median(v["VALUBusy"])), 2),
                "mfma_bf16_flops": int(np.median(v["MfmaFlopsBF16"])),
                "launches": len(v["MfmaUtil"])}
            for k, v in per.items() if "MfmaUtil" in v}
    with open(UTIL_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def load_utilisation(workload: str, kernel: str):
    """Counter-measured MFMA/VALU busy of a kernel, if taken on this source."""
    try:
        t = json.load(open(UTIL_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    return t.get("workloads", {}).get(workload, {}).get(kernel)


def source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        if os.path.exists(f):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    k = t.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("bytes_per_launch")


def main():
    args = parse()
    if args.summarize_counters or args.summarize_utilisation:
        if args.summarize_counters:
            summarize_counters(args.summarize_counters)
        if args.summarize_utilisation:
            summarize_utilisation(args.summarize_utilisation)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; run with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import speculative_decoding_head_amd as mtp
    import synth

    wl = synth.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)

    # ---- inputs (seeded, synthetic), resident in HBM -----------------------------
    t0 = time.time()
    rng = np.random.default_rng(wl.seed)
    # a 4-bit head keeps its fp32 draw on the host only to aim the planted rows
    head = synth.make_head(rng, wl.V, wl.d, wl.wtype, keep_source=wl.wtype == "q4a32" and args.planted_alpha > 0)
    h_v, h_d = synth.make_hidden(rng, wl.B, wl.k, wl.d)
    hv = synth.encode_hidden(h_v, wl.htype)
    hd = synth.encode_hidden(h_d, wl.htype)
    # the tiny workloads: fp32 head and hidden rows, row-major, no recurrent state (a cycle is
    # k draft calls + verify + accept)
    tiny = wl.wtype == "f32"

    def dev_rows(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a if wl.htype == "f32" else a.view(np.int16)).to(dev)

    if wl.wtype == "f32":
        dh = mtp.Head(mtp.W_F32, wl.d, wl.V, torch.from_numpy(head.w).to(dev))
    elif wl.wtype == "bf16":
        dh = mtp.Head(mtp.W_BF16, wl.d, wl.V, torch.from_numpy(head.w.view(np.int16)).to(dev))
    else:
        dh = mtp.Head(mtp.W_Q4A32, wl.d, wl.V, torch.from_numpy(head.w).to(dev),
                      torch.from_numpy(head.scale.view(np.int16)).to(dev),
                      torch.from_numpy(head.minv.view(np.int16)).to(dev))
    B, k, nd, V, d, T = wl.B, wl.k, wl.n_draft, wl.V, wl.d, wl.temperature
    # draft vocabulary: the first nd ids, or an ascending id list gathered once into its own
    # head (the draft head reports vocabulary ids; acceptance looks q up through row_of)
    draft_ids = row_of = None
    ddh = dh
    if args.draft_ids > 0:
        n_top = min(args.draft_ids, nd)
        draft_ids = np.concatenate([np.arange(0, nd - n_top), np.arange(V - n_top, V)]).astype(np.int32)
        ddh = mtp.gather_rows(dh, torch.from_numpy(draft_ids).to(dev))
        ro = np.full(V, -1, np.int32)
        ro[draft_ids] = np.arange(nd, dtype=np.int32)
        row_of = torch.from_numpy(ro).to(dev)
    if not args.row_major and not tiny:
        # one-time weight preparation at load: fragment-major tiles (same numbers, same logits)
        dh = mtp.tiled_head(dh)
        ddh = dh if draft_ids is None else mtp.tiled_head(ddh)
        torch.cuda.synchronize()
    exact = T > 0 and wl.accept_rule == "exact"
    rule = mtp.ACCEPT_EXACT if exact else mtp.ACCEPT_RATIO
    hv_t = dev_rows(hv)                                                          # [B][k+1][d]
    hd_slots = [dev_rows(hd[:, i]) for i in range(k)]
    dtok = torch.zeros(B, k, dtype=torch.int32, device=dev)
    dst = mtp.row_stats_empty(B, k)
    # exact-match acceptance reads neither the draft logits nor the verify logits
    dlg = torch.zeros(B, k, nd, dtype=torch.float32, device=dev) if T > 0 and not exact else None
    vst = mtp.row_stats_empty(B, k + 1)
    vlg = torch.zeros(B, k + 1, V, dtype=torch.float32, device=dev) if T > 0 and not exact else None
    out = torch.zeros(B, k + 1, dtype=torch.int32, device=dev)
    nacc = torch.zeros(B, dtype=torch.int32, device=dev)
    nemit = torch.zeros(B, dtype=torch.int32, device=dev)
    flg = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = mtp.workspace(max(mtp.workspace_bytes(mtp.OP_DRAFT, B, nd, B),
                           mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B),
                           mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, B)))
    with_commit = not args.no_commit and not tiny
    state_bytes = STATE_LAYERS * STATE_HEADS * STATE_DIM * STATE_DIM * 4
    kv_row_bytes = KV_HEADS * KV_DIM * 2
    if with_commit:
        g = torch.Generator(device=dev).manual_seed(1)
        snaps = torch.randint(0, 256, (B, k + 1, state_bytes), dtype=torch.uint8, device=dev, generator=g)
        live = torch.zeros(B, state_bytes, dtype=torch.uint8, device=dev)
        # room for every cycle's accepted rows, so the trim never saturates at the cache end
        kv_rows = KV_ROWS + (k + 1) * (args.warmup + args.steps * (1 + args.repeats) + 16 + args.extra_cycles
                                       + (k + 1) * args.adaptive_cycles)
        kv = torch.zeros(B, KV_LAYERS, 2, kv_rows, kv_row_bytes, dtype=torch.uint8, device=dev)
        kv_len = torch.zeros(B, dtype=torch.int32, device=dev)
    # the position verify row 0 predicts: the committed length (exact-match rule)
    positions = kv_len if with_commit else torch.zeros(B, dtype=torch.int32, device=dev)
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream()

    # --overlap-commit: the commit of a cycle runs on a second stream, beside the next cycle's
    # draft calls (they do not read the recurrent state or kv_len; the next verify does, and
    # waits for it)
    commit_stream = torch.cuda.Stream() if (with_commit and args.overlap_commit) else None
    ev_acc, ev_commit = torch.cuda.Event(), torch.cuda.Event()
    commit_pending = [False]

    def cycle(c, events=None, hidden=None):
        hv_c, hd_c = (hv_t, hd_slots) if hidden is None else hidden
        smp = mtp.sampling(T, wl.eos, wl.philox_seed, c, 0, rule, positions if exact else None)
        # an event between two launches puts a marker of a few microseconds between them:
        # the k draft launches run back to back inside one pair of events
        if events is not None:
            events[0].record(stream)
        for i in range(k):
            mtp.mtp_draft_head(ddh, nd, hd_c[i], i, k, smp, dtok, dst, dlg, ws, stream)
        if events is not None:
            events[1].record(stream)
        if commit_pending[0]:
            stream.wait_event(ev_commit)   # the verify reads the committed state and kv_len
            commit_pending[0] = False
        mtp.mtp_verify_logits(dh, hv_c, k, dtok, k, smp, vst, vlg, ws, stream)
        if events is not None:
            events[2].record(stream)
        mtp.mtp_accept_sample(B, k, k, V, nd, smp, dtok, dst, dlg, vst, vlg, out, nacc, nemit, flg, ws, stream,
                              draft_row_of=row_of)
        if events is not None:
            events[3].record(stream)
        if with_commit and commit_stream is None:
            mtp.mtp_commit_state(B, k, nacc, snaps, live, state_bytes, kv, KV_LAYERS, kv_rows, kv_row_bytes,
                                 kv_len, stream)
            if events is not None:
                events[4].record(stream)
        elif with_commit:
            ev_acc.record(stream)
            commit_stream.wait_event(ev_acc)
            mtp.mtp_commit_state(B, k, nacc, snaps, live, state_bytes, kv, KV_LAYERS, kv_rows, kv_row_bytes,
                                 kv_len, commit_stream)
            ev_commit.record(commit_stream)
            commit_pending[0] = True
            if events is not None:
                events[4].record(commit_stream)

    if args.calibrate_copy:
        # a plain kernel copy of known size (multiply by one: reads and writes COPY_BYTES);
        # copy_ itself would go to the DMA engine and show no kernel counters
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.mul(a, 1, out=b)
        torch.cuda.synchronize()
        del a, b

    for c in range(args.warmup):
        cycle(c)
    torch.cuda.synchronize()

    # ---- timed region: K cycles; per-kernel HIP events on the launch stream in every
    #      N-th cycle ------------------------------------------------------------------
    n_ev = 5
    every = max(1, args.event_every)
    timed = [s for s in range(args.steps) if s % every == 0]
    evs = {s: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for s in timed}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        cycle(args.warmup + s, evs.get(s))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    draft_ms = [evs[s][0].elapsed_time(evs[s][1]) / k for s in timed]
    verify_ms = [evs[s][1].elapsed_time(evs[s][2]) for s in timed]
    accept_ms = [evs[s][2].elapsed_time(evs[s][3]) for s in timed]
    commit_ms = ([evs[s][3].elapsed_time(evs[s][4]) for s in timed] if with_commit else [0.0])
    ms_per_step = elapsed * 1e3 / args.steps
    # stability: the same K cycles timed again in further windows (not part of `value`)
    repeat_rates = []
    for r in range(args.repeats):
        torch.cuda.synchronize()
        t_r = time.perf_counter()
        for s_ in range(args.steps):
            cycle(args.warmup + args.steps * (r + 1) + s_)
        torch.cuda.synchronize()
        repeat_rates.append(args.steps / (time.perf_counter() - t_r))
    value = args.steps / elapsed

    # algorithmic bytes per launch (weights read once, hidden rows, outputs)
    wrow = {"f32": d * 4, "bf16": d * 2, "q4a32": d // 2 + 2 * 2 * (d // 32)}[wl.wtype]
    hbytes = d * (4 if wl.htype == "f32" else 2)
    draft_bytes = nd * wrow + B * hbytes + B * (32 + 4) + (B * nd * 4 if dlg is not None else 0)
    verify_bytes = V * wrow + B * (k + 1) * hbytes + B * (k + 1) * 32 + (B * (k + 1) * V * 4 if vlg is not None else 0)
    commit_bytes = (2 * B * state_bytes) if with_commit else 0
    cycle_bytes = k * draft_bytes + verify_bytes + commit_bytes
    d_avg = float(np.mean(draft_ms)) * 1e-3
    v_avg = float(np.mean(verify_ms)) * 1e-3

    def roof(bytes_per_launch, avg_s, kernel, flops=None):
        ach = bytes_per_launch / avg_s / 1e9
        tr = load_traffic(args.workload, kernel)
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": tr,
             "kernel": kernel, "avg_launch_us": round(avg_s * 1e6, 2),
             "algorithmic_bytes_per_launch": int(bytes_per_launch)}
        if flops is not None:
            # the verify product runs on MFMA: its algorithmic rate against the dense bf16 peak
            r["mfma"] = {"algorithmic_flops_per_launch": int(flops),
                         "achieved_TFLOPs": round(flops / avg_s / 1e12, 1),
                         "frac_of_dense_bf16_peak": round(flops / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                         # rocprofv3 MfmaUtil / VALUBusy of the same kernel (profiles/mfma_valu.json)
                         "counters": load_utilisation(args.workload, kernel)}
        return r

    draft_kernel = "mtp_draft_head_kernel"
    # up to 16 rows one kernel; 17..128 rows the wide kernel plus its per-row merge
    verify_kernel = "mtp_verify_logits_kernel" if B * (k + 1) <= 16 else "mtp_verify_wide_kernel"
    dominant = "draft" if k * d_avg >= v_avg else "verify"
    roofline = roof(draft_bytes, d_avg, draft_kernel) if dominant == "draft" else roof(verify_bytes, v_avg, verify_kernel)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "q4a32": "q4a32"}[wl.wtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "d": d, "V": V, "n_draft": nd, "k": k, "batch": B,
                   "temperature": T, "accept_rule": wl.accept_rule if T > 0 else "exact (greedy)",
                   "weights": wl.wtype, "layout": "row-major" if (args.row_major or tiny) else "tiled",
                   "accumulate": "fp32",
                   "draft_vocabulary": (f"id list: the lowest {nd - min(args.draft_ids, nd):,} and the highest "
                                        f"{min(args.draft_ids, nd):,} ids" if draft_ids is not None else
                                        f"the first {nd:,} ids"),
                   "step": f"{k} draft-head calls + verify ({B * (k + 1)} rows) + accept"
                           + (" + commit (36 MiB snapshot select, 12-layer KV trim)" if with_commit else ""),
                   "commit_stream": ("second stream, beside the next cycle's draft calls (the next verify waits "
                                     "for it)" if commit_stream is not None else "the launch stream")
                                    if with_commit else None},
        "roofline": roofline,
        "roofline_verify": roof(verify_bytes, v_avg, verify_kernel, flops=2.0 * V * d * B * (k + 1)),
        "kernel_timing": f"HIP events on the launch stream in {len(timed)} of the {args.steps} timed cycles: "
                         f"one pair around the {k} back-to-back draft launches (average = span / {k}), "
                         f"one pair around each of verify, accept and commit (the commit's from the end of "
                         f"the accept to the end of the commit on its own stream)",
        "stages_us": {"draft_head_avg": round(d_avg * 1e6, 2), "verify_avg": round(v_avg * 1e6, 2),
                      "accept_avg": round(float(np.mean(accept_ms)) * 1e3, 2),
                      "commit_avg": round(float(np.mean(commit_ms)) * 1e3, 2)},
        # spread of the same event samples: 10th and 90th percentiles
        "stages_us_p10_p90": {name: [round(float(np.percentile(v, 10)) * 1e3, 2), round(float(np.percentile(v, 90)) * 1e3, 2)]
                              for name, v in (("draft_head", draft_ms), ("verify", verify_ms), ("accept", accept_ms),
                                              ("commit", commit_ms))},
        "cycle_algorithmic_GBps": round(cycle_bytes * value / 1e9, 1),
        "repeat_cycles_per_s": ({"windows": len(repeat_rates), "min": round(min(repeat_rates), 2),
                                 "median": round(float(np.median(repeat_rates)), 2), "max": round(max(repeat_rates), 2)}
                                if repeat_rates else None),
        "tokens_per_s": round(float(nemit.sum().item()) * value, 1),
        "setup_s": round(setup_s, 1),
    }

    if tiny:
        for key in ("roofline", "roofline_verify"):
            result[key]["note"] = ("the head (4 MiB, draft rows 1 MiB) stays in the caches: the tiny cycle is "
                                   "latency-bound, its fraction of HBM bandwidth is not a target")

    # ---- draft head against HBM proper: rotate over copies of the head, so that no
    #      call finds the previous call's rows in the 256 MB last-level cache ------------
    if args.rotate_heads > 1:
        copies = [ddh] + [mtp.Head(ddh.wtype, ddh.d, ddh.vocab, ddh.w.clone(),
                                   None if ddh.scale is None else ddh.scale.clone(),
                                   None if ddh.minv is None else ddh.minv.clone(), ddh.row_ids)
                          for _ in range(args.rotate_heads - 1)]
        smp = mtp.sampling(T, wl.eos, wl.philox_seed, 0, 0, rule, positions if exact else None)
        n = args.extra_cycles * k
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for j in range(len(copies)):
            mtp.mtp_draft_head(copies[j], nd, hd_slots[0], 0, k, smp, dtok, dst, dlg, ws, stream)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for j in range(n):
            mtp.mtp_draft_head(copies[j % len(copies)], nd, hd_slots[j % k], j % k, k, smp, dtok, dst, dlg, ws,
                               stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        rot = ev[0].elapsed_time(ev[1]) * 1e-3 / n
        result["draft_head_rotated"] = {"copies": len(copies), "launches": n, "avg_launch_us": round(rot * 1e6, 2),
                                        "achieved_GBps": round(draft_bytes / rot / 1e9, 1),
                                        "frac": round(draft_bytes / rot / 1e9 / PEAK_HBM_GBPS, 4)}
        del copies
        torch.cuda.empty_cache()

    # ---- planted acceptance: whole cycles whose per-request depth is drawn with
    #      P(depth >= j) = alpha^j (capped at k), planted into the hidden rows -----------
    if args.planted_alpha > 0:
        prng = np.random.default_rng(wl.seed + 7)
        n_sets = 16
        sets, depth_sum = [], 0
        for _ in range(n_sets):
            pv, pd = synth.make_hidden(prng, B, k, d)
            depths = np.minimum(prng.geometric(1.0 - args.planted_alpha, size=B) - 1, k)
            tg = prng.integers(0, nd, size=(B, k + 1))
            alt = (tg + 1 + prng.integers(0, nd - 1, size=(B, k + 1))) % nd
            if draft_ids is not None:   # planted tokens the draft vocabulary holds
                tg, alt = draft_ids[tg], draft_ids[alt]
            synth.plant_rows(head, pv, pd, depths, tg, alt)
            ev_, ed_ = synth.encode_hidden(pv, wl.htype), synth.encode_hidden(pd, wl.htype)
            sets.append((dev_rows(ev_), [dev_rows(ed_[:, i]) for i in range(k)]))
            depth_sum += int(depths.sum())
        emitted = torch.zeros(B, dtype=torch.int64, device=dev)
        for c in range(n_sets):   # warm-up, also of the counter update (its first call loads a kernel)
            cycle(c, hidden=sets[c])
            emitted += nemit
        emitted.zero_()
        torch.cuda.synchronize()
        pev = {c: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
               for c in range(args.extra_cycles) if c % every == 0}
        t1 = time.perf_counter()
        for c in range(args.extra_cycles):
            cycle(c, pev.get(c), hidden=sets[c % n_sets])
            emitted += nemit
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        tot = int(emitted.sum().item())
        pst = {name: round(float(np.mean([e[a].elapsed_time(e[b]) for e in pev.values()])) * 1e3 / div, 2)
               for name, a, b, div in (("draft_head_avg", 0, 1, k), ("verify_avg", 1, 2, 1),
                                       ("accept_avg", 2, 3, 1))}
        if with_commit:
            pst["commit_avg"] = round(float(np.mean([e[3].elapsed_time(e[4]) for e in pev.values()])) * 1e3, 2)
        result["planted_alpha"] = {
            "alpha": args.planted_alpha, "cycles": args.extra_cycles, "hidden_sets": n_sets,
            "cycles_per_s": round(args.extra_cycles / el, 2), "tokens_per_s": round(tot / el, 1),
            "mean_tokens_per_request_cycle": round(tot / (args.extra_cycles * B), 3),
            "planted_mean_depth": round(depth_sum / (n_sets * B), 3), "stages_us": pst}

        # ---- adaptive verify width: the native controller picks k for every cycle from its
        #      per-depth acceptance averages and its fitted cycle cost (the cycle's device time),
        #      against the full width with the same per-cycle synchronisation (the controller
        #      needs each cycle's outcome before it picks the next width) --------------------
        if args.adaptive_cycles > 0 and B == 1:
            def run_width(kk, c, hidden):
                hv_c, hd_c = hidden
                hv_k = hv_c[:, :kk + 1].contiguous()
                smp = mtp.sampling(T, wl.eos, wl.philox_seed, c, 0, rule, positions if exact else None)
                for i in range(kk):
                    mtp.mtp_draft_head(ddh, nd, hd_c[i], i, k, smp, dtok, dst, dlg, ws, stream)
                # one request: the first kk + 1 verify rows of every buffer are a contiguous prefix
                vst_k, out_k = vst[:, :kk + 1], out[:, :kk + 1]
                vlg_k = None if vlg is None else vlg[:, :kk + 1]
                mtp.mtp_verify_logits(dh, hv_k, kk, dtok, k, smp, vst_k, vlg_k, ws, stream)
                mtp.mtp_accept_sample(B, kk, k, V, nd, smp, dtok, dst, dlg, vst_k, vlg_k, out_k, nacc, nemit, flg,
                                      ws, stream, draft_row_of=row_of)
                if with_commit:
                    mtp.mtp_commit_state(B, kk, nacc, snaps[:, :kk + 1], live, state_bytes, kv, KV_LAYERS, kv_rows,
                                         kv_row_bytes, kv_len, stream)

            aw = {"alpha": args.planted_alpha, "cycles": args.adaptive_cycles, "fixed": {}}
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for mode in ["adaptive"] + list(range(1, k + 1)):
                ctl = mtp.WidthController(k_max=k)
                hist, toks, dev_s = [0] * (k + 1), 0, 0.0
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                for c in range(args.adaptive_cycles):
                    kk = ctl.choose() if mode == "adaptive" else mode
                    e0.record(stream)
                    run_width(kk, c, sets[c % n_sets])
                    e1.record(stream)
                    e1.synchronize()
                    sec = e0.elapsed_time(e1) * 1e-3
                    ctl.observe(kk, nacc, flg, sec)
                    toks += int(nemit.sum().item())
                    hist[kk] += 1
                    dev_s += sec
                el = time.perf_counter() - t1
                entry = {"tokens_per_s": round(toks / el, 1), "tokens_per_device_s": round(toks / dev_s, 1),
                         "mean_tokens_per_cycle": round(toks / args.adaptive_cycles, 3)}
                if mode == "adaptive":
                    entry.update({"width_histogram": {str(w): n for w, n in enumerate(hist) if n},
                                  "final_width": ctl.choose(),
                                  "acceptance_by_depth": [round(a, 3) for a in ctl.alpha[:k]],
                                  "cost_fit_us": {"c0": round(ctl.cost(0) * 1e6, 1),
                                                  "c1": round((ctl.cost(1) - ctl.cost(0)) * 1e6, 1)}})
                    aw["adaptive"] = entry
                else:
                    aw["fixed"][str(mode)] = entry
            best_w = max(aw["fixed"], key=lambda w: aw["fixed"][w]["tokens_per_device_s"])
            aw["full_width"] = aw["fixed"][str(k)]
            aw["best_fixed"] = {"width": int(best_w), "tokens_per_device_s": aw["fixed"][best_w]["tokens_per_device_s"]}
            aw["adaptive_over_best_fixed"] = round(aw["adaptive"]["tokens_per_device_s"]
                                                   / aw["fixed"][best_w]["tokens_per_device_s"], 4)
            result["adaptive_width"] = aw

    # ---- the other model-scale configurations, timed in the same run (not part of `value`):
    #      the 128-row verify + commit of 16 requests, and the 4-bit head ----------------
    if args.workload == "model_greedy" and not args.no_extra_configs and not args.row_major:
        result["configs"] = {}
        result["configs"]["batched_16x8"] = bench_batched(torch, mtp, synth, dh, nd, stream, args.extra_cycles,
                                                          every, state_bytes, kv_row_bytes)
        torch.cuda.empty_cache()
        result["configs"]["q4_greedy"] = bench_q4(torch, mtp, synth, stream, args.extra_cycles, every, state_bytes,
                                                  kv_row_bytes)
        torch.cuda.empty_cache()

    # ---- measured read ceiling: the library's streaming probe (the LM-head kernels' 1 KiB
    #      per wave non-temporal loads, no arithmetic) over 1 GiB, best launch shape ----------
    if not args.no_read_peak:
        rp = read_peak(torch, stream)
        result["read_peak"] = rp
        for key in ("roofline", "roofline_verify"):
            result[key]["frac_of_read_peak"] = round(result[key]["achieved"] / rp["GBps"], 4)
        for cfg in result.get("configs", {}).values():
            for part in cfg.get("kernels", {}).values():
                part["frac_of_read_peak"] = round(part["achieved_GBps"] / rp["GBps"], 4)

    # ---- CPU baseline: the oracle, as it stands, on a bounded sample --------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, head, hv, hd, args.cpu_cycles, with_commit, state_bytes)
    print(json.dumps(result), flush=True)


def _stage_events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _kernel_entry(name, launch_bytes, avg_s, flops=None, traffic_of=None):
    """traffic_of: (workload, [kernel keys]) whose counter-measured HBM bytes per launch
    (profiles/traffic.json, while it matches these sources) are summed into "traffic"."""
    e = {"kernel": name, "avg_launch_us": round(avg_s * 1e6, 2), "algorithmic_bytes_per_launch": int(launch_bytes),
         "achieved_GBps": round(launch_bytes / avg_s / 1e9, 1),
         "frac": round(launch_bytes / avg_s / 1e9 / PEAK_HBM_GBPS, 4)}
    if flops is not None:
        e["mfma_frac_of_dense_bf16_peak"] = round(flops / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4)
    if traffic_of is not None:
        parts = [load_traffic(traffic_of[0], k) for k in traffic_of[1]]
        e["traffic"] = None if any(t is None for t in parts) else int(sum(parts))
    return e


def _time_cycles(torch, stream, run, n, every):
    """n cycles of run(c, events) back to back; events in every `every`-th cycle; returns
    (seconds, {cycle: events})."""
    for c in range(3):
        run(c, None)
    torch.cuda.synchronize()
    evs = {c: _stage_events(torch, 5) for c in range(n) if c % every == 0}
    t0 = time.perf_counter()
    for c in range(n):
        run(c, evs.get(c))
    torch.cuda.synchronize()
    return time.perf_counter() - t0, evs


def _span_avg(evs, a, b, div=1):
    return float(np.mean([e[a].elapsed_time(e[b]) for e in evs.values()])) * 1e-3 / div


def bench_batched(torch, mtp, synth, dh, nd, stream, n, every, state_bytes, kv_row_bytes):
    """16 requests x 8 verify rows on the model-scale bf16 head: 7 draft-head calls of 16 rows,
    the 128-row verify (wide kernel + per-row merge), acceptance, and the commit of 16 x 36 MiB
    snapshots with the KV trim.  Raw random hidden rows, greedy."""
    wl = synth.WORKLOADS["batched_commit"]
    B, k, V, d = wl.B, wl.k, wl.V, wl.d
    rng = np.random.default_rng(wl.seed + 1)
    h_v, h_d = synth.make_hidden(rng, B, k, d)
    hv = torch.from_numpy(synth.encode_hidden(h_v, "bf16").view(np.int16)).cuda()
    hds = [torch.from_numpy(np.ascontiguousarray(synth.encode_hidden(h_d, "bf16")[:, i]).view(np.int16)).cuda()
           for i in range(k)]
    dtok = torch.zeros(B, k, dtype=torch.int32, device="cuda")
    dst, vst = mtp.row_stats_empty(B, k), mtp.row_stats_empty(B, k + 1)
    out = torch.zeros(B, k + 1, dtype=torch.int32, device="cuda")
    nacc, nemit, flg = (torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(3))
    ws = mtp.workspace(max(mtp.workspace_bytes(mtp.OP_DRAFT, B, nd, B), mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B),
                           mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, B)))
    g = torch.Generator(device="cuda").manual_seed(5)
    snaps = torch.randint(0, 256, (B, k + 1, state_bytes), dtype=torch.uint8, device="cuda", generator=g)
    live = torch.zeros(B, state_bytes, dtype=torch.uint8, device="cuda")
    kv_rows = KV_ROWS + (k + 1) * (n + 8)
    kv = torch.zeros(B, KV_LAYERS, 2, kv_rows, kv_row_bytes, dtype=torch.uint8, device="cuda")
    kv_len = torch.zeros(B, dtype=torch.int32, device="cuda")

    def run(c, e):
        smp = mtp.sampling(0.0, -1, 0, c, 0)
        if e:
            e[0].record(stream)
        for i in range(k):
            mtp.mtp_draft_head(dh, nd, hds[i], i, k, smp, dtok, dst, None, ws, stream)
        if e:
            e[1].record(stream)
        mtp.mtp_verify_logits(dh, hv, k, dtok, k, smp, vst, None, ws, stream)
        if e:
            e[2].record(stream)
        mtp.mtp_accept_sample(B, k, k, V, nd, smp, dtok, dst, None, vst, None, out, nacc, nemit, flg, ws, stream)
        if e:
            e[3].record(stream)
        mtp.mtp_commit_state(B, k, nacc, snaps, live, state_bytes, kv, KV_LAYERS, kv_rows, kv_row_bytes, kv_len,
                             stream)
        if e:
            e[4].record(stream)

    el, evs = _time_cycles(torch, stream, run, n, every)
    d_s, v_s, a_s, c_s = _span_avg(evs, 0, 1, k), _span_avg(evs, 1, 2), _span_avg(evs, 2, 3), _span_avg(evs, 3, 4)
    draft_bytes = nd * 2 * d + B * 2 * d + B * 36
    verify_bytes = V * 2 * d + B * (k + 1) * (2 * d + 32)
    commit_bytes = 2 * B * state_bytes
    r = {"workload": "batched_16x8", "requests": B, "verify_rows": B * (k + 1), "cycles": n,
         "step": f"{k} draft-head calls ({B} rows) + verify ({B * (k + 1)} rows) + accept + commit "
                 f"({B} x 36 MiB snapshot select, 12-layer KV trim)",
         "cycles_per_s": round(n / el, 2),
         "kernel_timing": "HIP events on the launch stream in every " + str(every) + "th cycle (the verify span "
                          "covers the wide kernel and its per-row merge)",
         "kernels": {"draft_head_16_rows": _kernel_entry("mtp_draft_head_kernel", draft_bytes, d_s,
                                                         traffic_of=("batched_commit", ["mtp_draft_head_kernel"])),
                     "verify_128_rows": _kernel_entry("mtp_verify_wide_kernel + mtp_verify_wide_merge_kernel",
                                                      verify_bytes, v_s, flops=2.0 * V * d * B * (k + 1),
                                                      traffic_of=("batched_commit", ["mtp_verify_wide_kernel",
                                                                                      "mtp_verify_wide_merge_kernel"])),
                     "commit": _kernel_entry("mtp_commit_state_kernel", commit_bytes, c_s,
                                             traffic_of=("batched_commit", ["mtp_commit_state_kernel"]))},
         "accept_us": round(a_s * 1e6, 2)}
    del snaps, live, kv
    return r


def bench_q4(torch, mtp, synth, stream, n, every, state_bytes, kv_row_bytes):
    """The 4-bit affine head (152,064 x 2560, 32-value groups, bf16 scale and min, tiled):
    7 draft-head calls, the 8-row verify, acceptance and the commit of one request, greedy,
    raw random hidden rows (the q4_greedy workload's draws)."""
    wl = synth.WORKLOADS["q4_greedy"]
    B, k, V, d, nd = wl.B, wl.k, wl.V, wl.d, wl.n_draft
    rng = np.random.default_rng(wl.seed)
    head = synth.make_head(rng, V, d, "q4a32")
    h_v, h_d = synth.make_hidden(rng, B, k, d)
    dh = mtp.tiled_head(mtp.Head(mtp.W_Q4A32, d, V, torch.from_numpy(head.w).cuda(),
                                 torch.from_numpy(head.scale.view(np.int16)).cuda(),
                                 torch.from_numpy(head.minv.view(np.int16)).cuda()))
    torch.cuda.synchronize()
    hv = torch.from_numpy(synth.encode_hidden(h_v, "bf16").view(np.int16)).cuda()
    hds = [torch.from_numpy(np.ascontiguousarray(synth.encode_hidden(h_d, "bf16")[:, i]).view(np.int16)).cuda()
           for i in range(k)]
    dtok = torch.zeros(B, k, dtype=torch.int32, device="cuda")
    dst, vst = mtp.row_stats_empty(B, k), mtp.row_stats_empty(B, k + 1)
    out = torch.zeros(B, k + 1, dtype=torch.int32, device="cuda")
    nacc, nemit, flg = (torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(3))
    ws = mtp.workspace(max(mtp.workspace_bytes(mtp.OP_DRAFT, B, nd, B), mtp.workspace_bytes(mtp.OP_VERIFY, B * (k + 1), V, B),
                           mtp.workspace_bytes(mtp.OP_ACCEPT, 0, V, B)))
    g = torch.Generator(device="cuda").manual_seed(6)
    snaps = torch.randint(0, 256, (B, k + 1, state_bytes), dtype=torch.uint8, device="cuda", generator=g)
    live = torch.zeros(B, state_bytes, dtype=torch.uint8, device="cuda")
    kv_rows = KV_ROWS + (k + 1) * (n + 8)
    kv = torch.zeros(B, KV_LAYERS, 2, kv_rows, kv_row_bytes, dtype=torch.uint8, device="cuda")
    kv_len = torch.zeros(B, dtype=torch.int32, device="cuda")

    def run(c, e):
        smp = mtp.sampling(0.0, -1, 0, c, 0)
        if e:
            e[0].record(stream)
        for i in range(k):
            mtp.mtp_draft_head(dh, nd, hds[i], i, k, smp, dtok, dst, None, ws, stream)
        if e:
            e[1].record(stream)
        mtp.mtp_verify_logits(dh, hv, k, dtok, k, smp, vst, None, ws, stream)
        if e:
            e[2].record(stream)
        mtp.mtp_accept_sample(B, k, k, V, nd, smp, dtok, dst, None, vst, None, out, nacc, nemit, flg, ws, stream)
        if e:
            e[3].record(stream)
        mtp.mtp_commit_state(B, k, nacc, snaps, live, state_bytes, kv, KV_LAYERS, kv_rows, kv_row_bytes, kv_len,
                             stream)
        if e:
            e[4].record(stream)

    el, evs = _time_cycles(torch, stream, run, n, every)
    d_s, v_s, a_s, c_s = _span_avg(evs, 0, 1, k), _span_avg(evs, 1, 2), _span_avg(evs, 2, 3), _span_avg(evs, 3, 4)
    wrow = d // 2 + 2 * 2 * (d // 32)
    draft_bytes = nd * wrow + B * 2 * d + B * 36
    verify_bytes = V * wrow + B * (k + 1) * (2 * d + 32)
    r = {"workload": "q4_greedy", "cycles": n, "weights": "4-bit affine, 32-value groups, bf16 scale and min (1,600 B/row)",
         "step": f"{k} draft-head calls + verify ({B * (k + 1)} rows) + accept + commit (36 MiB snapshot select)",
         "cycles_per_s": round(n / el, 2),
         "kernel_timing": "HIP events on the launch stream in every " + str(every) + "th cycle",
         "kernels": {"draft_head": _kernel_entry("mtp_draft_head_kernel", draft_bytes, d_s,
                                                 traffic_of=("q4_greedy", ["mtp_draft_head_kernel"])),
                     "verify_8_rows": _kernel_entry("mtp_verify_logits_kernel", verify_bytes, v_s,
                                                    traffic_of=("q4_greedy", ["mtp_verify_logits_kernel"]))},
         "accept_us": round(a_s * 1e6, 2), "commit_us": round(c_s * 1e6, 2)}
    del snaps, live, kv, dh
    return r


def read_peak(torch, stream, nbytes: int = 1 << 30):
    """Read-only bandwidth ceiling: libmtp_probe's stream_read over nbytes (4x the 256 MB
    last-level cache), every depth x grid shape, best of 5 launches each; bytes read / time."""
    import ctypes
    from speculative_decoding_head_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.mtp_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mtp_probe_stream_read.restype = ctypes.c_int
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)                       # every lane's fold is 0 or 0x01010101, never the magic value
    grids, depths = (256, 512, 1024, 2048), (8, 16, 32)
    sink = torch.zeros(max(grids) * 512, dtype=torch.int32, device="cuda")
    sp = stream.cuda_stream
    table = {}
    for depth in depths:
        for grid in grids:
            def launch():
                rc = lib.mtp_probe_stream_read(buf.data_ptr(), nbytes, grid, depth, 0x9E3779B9, sink.data_ptr(), sp)
                if rc != 0:
                    raise RuntimeError(f"stream probe failed ({rc})")
            launch()
            torch.cuda.synchronize()
            best = None
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3
                best = t if best is None else min(best, t)
            table[f"depth{depth}_grid{grid}"] = round(nbytes / best / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    key = max(table, key=table.get)
    return {"GBps": table[key], "shape": key, "frac_of_8TBps": round(table[key] / PEAK_HBM_GBPS, 4),
            "kind": "read-only stream of 1 GiB (libmtp_probe: 1 KiB per wave non-temporal loads, the tiled "
                    "LM-head pattern, no arithmetic), best of 5 launches per shape, best shape",
            "shapes_GBps": table}


def cpu_model() -> str:
    """The host CPU's model name (first /proc/cpuinfo entry), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, head, hv, hd, n_cycles, with_commit, state_bytes):
    from oracle import mtp_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count(), "unknown"
    W = O.head_weights_f64(head)                      # setup, not timed
    hv64 = O.hidden_f64(hv, wl.htype)
    hd64 = O.hidden_f64(hd, wl.htype)
    delta = 2e-2
    if with_commit:
        snaps = np.zeros((wl.B, wl.k + 1, state_bytes), np.uint8)
        live = np.zeros((wl.B, state_bytes), np.uint8)
        kv = np.zeros((wl.B, KV_LAYERS, 2, KV_ROWS, KV_HEADS * KV_DIM * 2), np.uint8)
        kv_len = np.zeros(wl.B, np.int32)
    budget_s = 20.0
    done = 0
    t0 = time.perf_counter()
    while True:
        o = O.cycle(W, wl.n_draft, hd64, hv64, wl.temperature, wl.philox_seed, done, wl.eos, delta,
                    rule=wl.accept_rule, positions=np.full(wl.B, done * (wl.k + 1)))
        if with_commit:
            O.commit(snaps, live, kv, kv_len, o["accept"]["n_accept"], wl.k)
        done += 1
        el = time.perf_counter() - t0
        if (n_cycles and done >= n_cycles) or (not n_cycles and el >= budget_s):
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 4), "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole cycles of the {wl.name} workload (numpy fp64, weights pre-converted "
                      f"to fp64 outside the timing), {el:.1f} s",
            "blas": blas, "cpu": cpu_model(),
            "host_cores_visible": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
