"""Decode-step attention benchmark of the FastOCR library on one MI355X.

Workload (default): the 72B-like configuration at tau = 0.05 -- 80 layers,
64 query / 8 KV heads, head_dim 128, batch 8, bf16 KV cache, 12800 image
tokens (80x160 page) + 128 prompt tokens + 2048 decode steps, w = 8 warm-up
steps, |C| = 8 focal layers; synthetic seeded inputs (K, V ~ N(0,1); queries
follow a 3x5 fixation window that moves one cell per step).  The other
workloads (7b-b1, 7b-b16-ragged, 32b-b4-longpage, other tau / sigma of the
72B-like sweep) run with --workload / --tau / --sigma.

A timed step is one decode step of the method through all layers: focal
layers (full attention + image-logit export + combine + head-summed scores +
top-k), non-focal layers (gathered sparse attention + combine), with the
kept set carried across steps on the device.  The warm-up steps and the
focal-layer profiling run once before timing.  The same steps are timed on
the library's FULL path (full attention on every layer) for the speedup.

Output: one JSON line (see the keys at the end of main()).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
SPIN_PROBE_CYCLES = 2_000_000  # spin-kernel length used to convert cycles to ms
EVENT_LAUNCHES_PER_CHUNK = 192  # timed launches queued behind one spin kernel


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="72b-b8-sweep")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--tp-shard", type=int, default=1, metavar="T",
                    help="time one tensor-parallel rank's share of the workload: 1/T of its KV and query "
                         "heads, everything else unchanged (the rank picks from its own heads' scores; the "
                         "cross-rank score all-reduce a T-GPU run adds per focal layer is not included)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline sample (0 disables it)")
    ap.add_argument("--profile-only", action="store_true",
                    help="skip the CPU baseline and the FULL comparison (for profiler runs)")
    # The two extra phases are off by default, so that a kernel trace of the
    # default command averages the same launches as its event timing (the
    # scrubbed replays run MALL-cold, the append variants do more work).
    ap.add_argument("--scrub-mb", type=int, default=0,
                    help="also time steps after a read pass over this many MiB that evicts the 256 MB "
                         "MALL (512 evicts it; 0, the default, disables it)")
    ap.add_argument("--append", action="store_true",
                    help="also compare a separate K/V append kernel with fastocr_attend_append")
    ap.add_argument("--no-append", action="store_true", help="(the default) no append comparison")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with a 256 MiB device-to-device copy, the reference kernel that "
                         "scales hardware byte counters")
    ap.add_argument("--pmc-summary", default=None, nargs="+", metavar="DIR",
                    help="summarise rocprofv3 counter CSVs under the DIRs (and the algorithmic bytes in a "
                         "profiled run's output file, if given) and exit (no GPU use)")
    ap.add_argument("--marker-summary", default=None, nargs="+", metavar="DIR",
                    help="host time per library call kind from a FASTOCR_TRACE=1 rocprofv3 --marker-trace run "
                         "under the DIRs, and exit (no GPU use)")
    ap.add_argument("--counter-summary", default=None, nargs="+", metavar="DIR",
                    help="average every counter per library kernel over rocprofv3 counter CSVs under the DIRs "
                         "and exit (no GPU use)")
    ap.add_argument("--trace-summary", default=None, nargs="+", metavar="ARG",
                    help="DIR COMMAND [BENCH_JSON]: summarise a rocprofv3 kernel trace under DIR made by "
                         "COMMAND, beside the event averages of BENCH_JSON, and exit")
    return ap.parse_args()


CAL_BYTES = 256 << 20
# the library's kernels and the host code that sizes their launches: counter
# summaries taken with other sources no longer describe the launches
LIBRARY_SRC = [os.path.join(ROOT, "dynamic_kv_cache_amd", "csrc", f)
               for f in ("kernels.hip", "fastocr_api.cpp", "internal.h")]
# rates of the read probe: the buffer it cycles through (far above the 256 MB
# MALL, so every read comes from HBM) and the read sizes of the curve
PROBE_BUFFER = 2 << 30
PROBE_SIZES_MB = (1, 2, 4, 8, 16, 32, 64)


def library_source_digest():
    import hashlib
    h = hashlib.sha256()
    for path in LIBRARY_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_CLASSES = ["full_split", "focal_split", "sparse_split", "merge", "topk"]


def kernel_class(name):
    """Timing class of a library kernel from its demangled name."""
    import re
    head = name.split("(")[0]
    m = re.search(r"split_attn_kernel<[^,]+, \d+, (\d)", head)
    if m:
        return KERNEL_CLASSES[int(m.group(1))]
    if "fastocr::split_valu_kernel<" in head:
        return "full_split"  # the VALU variant of the full pass
    if "fastocr::kept_attn_kernel<" in head:
        return "sparse_split"
    if "fastocr::merge_kernel<" in head or "fastocr::kept_merge_kernel<" in head:
        return "merge"
    if "fastocr::topk_kernel" in head:
        return "topk"
    return None


def pmc_summary(args):
    """HBM bytes per dispatch of each library kernel from rocprofv3 counter
    CSVs (one directory per counter pass).  Each counter is scaled by what
    it reads for the calibration kernel (an int64 add that reads and writes
    CAL_BYTES once each).  A file argument is the output of one of the
    profiled runs: its JSON line gives the algorithmic bytes per launch of
    that run's dispatches."""
    import csv
    import glob
    directories = [a for a in args if os.path.isdir(a)]
    run_alg = {}
    for a in args:
        if os.path.isfile(a):
            for line in open(a):
                if line.startswith("{") and "alg_bytes_per_launch_run" in line:
                    run_alg = json.loads(line)["alg_bytes_per_launch_run"]
    acc = {}
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    scale = {}
    for (name, ctr), vals in acc.items():
        if "add<long>" in name and np.mean(vals) > 0.25 * CAL_BYTES / 1024:
            scale[ctr] = CAL_BYTES / 1024 / np.mean(vals)
    print(f"library_source_sha256_16: {library_source_digest()}")
    for ctr, f in sorted(scale.items()):
        print(f"calibration_{ctr}: {f:.4f}  # {CAL_BYTES >> 20} MiB int64 add counts "
              f"{CAL_BYTES / 1024 / f:.0f} KiB")
    per = {}
    for (name, ctr), vals in acc.items():
        cls = kernel_class(name)
        if cls is not None:
            per.setdefault(cls, {})[ctr] = (np.mean(vals), len(vals))
    for cls in [c for c in KERNEL_CLASSES if c in per]:
        ctrs = per[cls]
        for ctr, (v, n) in sorted(ctrs.items()):
            print(f"{cls}.{ctr}_KiB_per_dispatch: {v:.1f}  # {n} dispatches")
        if all(c in ctrs and c in scale for c in ("FETCH_SIZE", "WRITE_SIZE")):
            hbm = sum(ctrs[c][0] * scale[c] * 1024 for c in ("FETCH_SIZE", "WRITE_SIZE"))
            print(f"{cls}.hbm_bytes_per_launch: {hbm:.0f}")
        if cls in run_alg:
            print(f"{cls}.run_alg_bytes_per_launch: {run_alg[cls]}  # K/V rows the same run's dispatches read")


def counter_summary(directories):
    """Per kernel (demangled name up to its argument list) and counter: the
    average value per dispatch over rocprofv3 counter CSVs under the
    directories (raw counts, no calibration)."""
    import csv
    import glob
    acc = {}
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = r["Kernel_Name"].split("(")[0]
                    if kernel_class(name) is None:
                        continue
                    acc.setdefault((name, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    print(f"library_source_sha256_16: {library_source_digest()}")
    for (name, ctr), vals in sorted(acc.items()):
        print(f"{kernel_class(name):12s} {ctr:26s} {np.mean(vals):16.1f}  # {len(vals)} dispatches, {name}")


def marker_summary(directories):
    """Host time of the library's calls from the named ranges a FASTOCR_TRACE=1
    run leaves in a rocprofv3 --marker-trace CSV: per kind of call, the count
    and the median and mean time from entering to leaving the call (the
    host's enqueue cost, not kernel time)."""
    import csv
    import glob
    per = {}
    for directory in directories:
        for path in glob.glob(os.path.join(directory, "**", "*marker_api_trace.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = r["Function"]
                    if not name.startswith("fastocr"):
                        continue
                    kind = "profile" if name == "fastocr profile" else name.split()[-1]
                    dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    per.setdefault(kind, []).append(dt)
    print(f"library_source_sha256_16: {library_source_digest()}")
    print(f"# {'call kind':12s} {'calls':>7s} {'median_us':>10s} {'mean_us':>10s}")
    for kind, v in sorted(per.items()):
        print(f"{kind:14s} {len(v):7d} {float(np.median(v)):10.2f} {float(np.mean(v)):10.2f}")


def trace_summary(directory, command, bench_json=None):
    """Per-kernel durations from a rocprofv3 --kernel-trace --stats run of
    this script, beside the averages that a run of the same command measured
    with its own completion events: `bench_json` (the same command without
    the profiler, whose per-dispatch overhead stretches the event intervals)
    or else bench.json in `directory`."""
    import csv
    import glob
    stats = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    print(f"# command: {command}")
    print(f"library_source_sha256_16: {library_source_digest()}")
    bench = {}
    bj = bench_json or os.path.join(directory, "bench.json")
    if os.path.exists(bj):
        with open(bj) as f:
            bench = json.loads(f.read().strip().splitlines()[-1])
        print(f"# event averages from: {'the same command without the profiler' if bench_json else 'the profiled run'};"
              f" its value {bench.get('value')} {bench.get('unit')}, workload {bench['config'].get('name')}")
    ev = bench.get("per_kernel", {})
    print(f"# {'kernel class':14s} {'calls':>7s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} "
          f"{'bench_event_avg_us':>18s}  name")
    for path in stats:
        with open(path) as f:
            for r in csv.DictReader(f):
                cls = kernel_class(r["Name"])
                if cls is None:
                    continue
                e = ev.get(cls, {}).get("avg_us")
                print(f"{cls:16s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:8.3f} "
                      f"{float(r['MinNs']) / 1e3:8.3f} {float(r['MaxNs']) / 1e3:8.3f} "
                      f"{(f'{e:.3f}' if e is not None else '-'):>18s}  {r['Name'].split('(')[0]}")


def read_traffic(kernel, workload):
    """(HBM bytes per launch of `kernel`, algorithmic bytes per launch of the
    same counter run's dispatches) from the committed counter summary
    (profiles/pmc_<workload>.txt); None when there is none or the kernels
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.txt")
    if not os.path.exists(path):
        return None, None
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0]
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("library_source_sha256_16") != library_source_digest():
        return None, None

    def num(key):
        try:
            return float(vals[key])
        except (KeyError, ValueError):
            return None
    return num(f"{kernel}.hbm_bytes_per_launch"), num(f"{kernel}.run_alg_bytes_per_launch")


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.marker_summary:
        marker_summary(args.marker_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary[:3])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import dynamic_kv_cache_amd as fo
    from workload import DeviceGenerator, get_workload, make_structure

    base = get_workload(args.workload)
    if args.tp_shard < 1 or base.num_kv_heads % args.tp_shard or base.num_q_heads % args.tp_shard:
        print(f"--tp-shard {args.tp_shard} must divide the workload's {base.num_kv_heads} KV heads and "
              f"{base.num_q_heads} query heads", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    overrides = {}
    if args.tau is not None:
        overrides["tau"] = args.tau
    if args.sigma is not None:
        overrides["sigma"] = args.sigma
    T = args.tp_shard
    if T != 1:
        overrides["num_kv_heads"] = base.num_kv_heads // T
        overrides["num_q_heads"] = base.num_q_heads // T
    wl = get_workload(args.workload, **overrides)
    st = make_structure(wl)
    gen = DeviceGenerator(wl, st, device=dev)
    L, B, Hq, Hkv, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    w, W, K = wl.warmup_steps, args.warmup, args.steps
    # Decode steps used: the w warm-up steps and W untimed pruned steps run
    # in order; then each timing phase (graph replays, per-kernel events,
    # replays after a MALL scrub, the two append variants) runs K steps
    # spread over the rest of the trajectory [w + W, T), the phases
    # interleaved, so every phase sees short and long text alike.
    do_scrub = args.scrub_mb > 0 and not args.profile_only and not args.no_graph
    do_append = args.append and not args.no_append and not args.profile_only and not args.no_graph
    # the schedule does not depend on which phases run, so a profiler run of
    # a subset times the same decode steps as the full run
    phases = ["graph", "events", "scrub", "append_separate", "append_fused"]
    t_timed = w + W
    assert t_timed < wl.steps, f"--warmup too large for {wl.steps} decode steps"
    span, n_log = wl.steps - t_timed, len(phases) * K
    phase_steps = {ph: [t_timed + ((k * len(phases) + i) * span) // n_log for k in range(K)]
                   for i, ph in enumerate(phases)}
    if not do_scrub:
        del phase_steps["scrub"]
    if not do_append:
        del phase_steps["append_separate"], phase_steps["append_fused"]
    used = sorted(set(range(t_timed)).union(*phase_steps.values()))
    slot = {t: i for i, t in enumerate(used)}
    io = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    t0 = time.time()
    Kd, Vd, Qall = [], [], torch.empty((len(used), L, B, Hq, d), dtype=io, device=dev)
    for l in range(L):
        k, v = gen.layer_kv(l)
        Kd.append(k)
        Vd.append(v)
        Qall[:, l] = gen.layer_queries(l, used, k)
    lens_all = torch.from_numpy(np.stack([st.lens(t) for t in used])).to(dev)
    q_at = lambda t: Qall[slot[t]]  # noqa: E731  [L, B, Hq, d] of decode step t
    lens_at = lambda t: lens_all[slot[t]]  # noqa: E731
    torch.cuda.synchronize()
    log(f"inputs for {wl.name} ready in {time.time() - t0:.1f}s "
        f"(KV {2 * L * B * Hkv * st.max_seq_len * d * Kd[0].element_size() / 1e9:.2f} GB)")

    stream = torch.cuda.Stream()

    def make(mode):
        cfg = fo.Config(num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, batch=B,
                        max_seq_len=st.max_seq_len, max_img_tokens=int(st.n_img.max()),
                        min_img_tokens=int(st.n_img.min()), max_text_tokens=int(st.n_prompt.max()) + wl.steps,
                        tau=wl.tau, num_focal=wl.num_focal,
                        warmup_steps=w, dtype=wl.dtype, mode=mode)
        return fo.fastocr_create(cfg, stream)

    q_stage = torch.empty((L, B, Hq, d), dtype=io, device=dev)
    lens_stage = torch.empty((B, 2), dtype=torch.int32, device=dev)
    out_stage = torch.empty((L, B, Hq, d), dtype=io, device=dev)

    def eager_step(h, t, out):
        for l in range(L):
            fo.fastocr_attend(h, l, q_at(t)[l], Kd[l], Vd[l], lens_at(t), out[l])

    def time_steps(h, steps, graph):
        """Wall time per step over `steps` (HIP events on the library stream)."""
        with torch.cuda.stream(stream):
            if graph is not None:
                q_stage.copy_(q_at(steps[0]))
                lens_stage.copy_(lens_at(steps[0]))
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for t in steps:
                if graph is not None:
                    q_stage.copy_(q_at(t))
                    lens_stage.copy_(lens_at(t))
                    graph.replay()
                else:
                    eager_step(h, t, out_stage)
            ev1.record(stream)
            torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / len(steps)

    scrub = None
    if do_scrub:
        scrub = torch.ones((args.scrub_mb << 20) // 8, dtype=torch.int64, device=dev)
        scrub_out = torch.zeros((), dtype=torch.int64, device=dev)

    def time_steps_scrubbed(steps, graph):
        """Mean time of single replays: every other one right after a read
        pass over `scrub` (a reduction, which evicts the cache rows and
        indices of the previous step from the MALL and leaves no dirty lines
        to write back), the others right after a spin kernel as long as that
        pass (the control: same launch, warm MALL).  The preceding kernel
        keeps the GPU busy while the host enqueues the replay and lies
        outside the timed interval."""
        torch.sum(scrub, dim=0, out=scrub_out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(scrub, dim=0, out=scrub_out)
        b.record()
        torch.cuda.synchronize()
        spin = int(cycles_per_ms * a.elapsed_time(b))
        evs = {True: [], False: []}
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            for i, t in enumerate(steps):
                q_stage.copy_(q_at(t))
                lens_stage.copy_(lens_at(t))
                scrubbed = i % 2 == 0
                if scrubbed:
                    torch.sum(scrub, dim=0, out=scrub_out)
                else:
                    torch.cuda._sleep(spin)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                graph.replay()
                b.record(stream)
                evs[scrubbed].append((a, b))
            torch.cuda.synchronize()
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in evs.items()}

    # the current token's K/V of every layer at the append-timing steps (the
    # cache already holds them: the appends rewrite the same values)
    if do_append:
        app_steps = phase_steps["append_separate"] + phase_steps["append_fused"]
        bi = torch.arange(B, device=dev)
        cur_all = (lens_all[[slot[t] for t in app_steps], :, 1] - 1).long()  # [S, B]
        kn_all = torch.stack([torch.stack([Kd[l][bi, :, cur_all[i]] for l in range(L)]) for i in range(len(app_steps))])
        vn_all = torch.stack([torch.stack([Vd[l][bi, :, cur_all[i]] for l in range(L)]) for i in range(len(app_steps))])
        kn_stage = torch.empty_like(kn_all[0])  # [L, B, Hkv, d]
        vn_stage = torch.empty_like(vn_all[0])

    def capture_append(h, fused):
        """One step with the current token's K/V appended: by an indexed copy
        kernel per layer before fastocr_attend, or by fastocr_attend_append."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            q_stage.copy_(q_at(app_steps[0]))
            lens_stage.copy_(lens_at(app_steps[0]))
            kn_stage.copy_(kn_all[0])
            vn_stage.copy_(vn_all[0])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            if not fused:
                ci = (lens_stage[:, 1] - 1).long()
            for l in range(L):
                if fused:
                    fo.fastocr_attend_append(h, l, q_stage[l], kn_stage[l], vn_stage[l], Kd[l], Vd[l],
                                             lens_stage, out_stage[l])
                else:
                    Kd[l][bi, :, ci] = kn_stage[l]
                    Vd[l][bi, :, ci] = vn_stage[l]
                    fo.fastocr_attend(h, l, q_stage[l], Kd[l], Vd[l], lens_stage, out_stage[l])
        torch.cuda.synchronize()
        return g

    def time_append(h, steps, idx0, fused):
        g = capture_append(h, fused)
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i, t in enumerate(steps):
                q_stage.copy_(q_at(t))
                lens_stage.copy_(lens_at(t))
                kn_stage.copy_(kn_all[idx0 + i])
                vn_stage.copy_(vn_all[idx0 + i])
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / len(steps)

    def capture(h):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            q_stage.copy_(q_at(phase_steps["graph"][0]))
            lens_stage.copy_(lens_at(phase_steps["graph"][0]))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for l in range(L):
                fo.fastocr_attend(h, l, q_stage[l], Kd[l], Vd[l], lens_stage, out_stage[l])
        torch.cuda.synchronize()
        return g

    def spin_ms(cycles):
        with torch.cuda.stream(stream):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            torch.cuda._sleep(cycles)
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b)

    spin_ms(SPIN_PROBE_CYCLES)  # first launch of the spin kernel
    cycles_per_ms = SPIN_PROBE_CYCLES / max(spin_ms(2 * SPIN_PROBE_CYCLES) - spin_ms(SPIN_PROBE_CYCLES), 1e-3)

    def kernel_times(h, steps, out_hist):
        """Per-kernel-class launch durations from HIP events.

        Every launch records an event when its kernel completes, and a
        launch's time is the interval since the previous completion.  Each
        chunk of steps is queued behind a bounded spin kernel that outlasts
        the host's enqueueing of the chunk, so the kernels run back to back
        and those intervals are their durations (the first launch of a chunk,
        which follows the spin, is not timed).
        """
        fo.fastocr_set_timing(h, True)
        fo.fastocr_reset_timing(h)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            eager_step(h, steps[0], out_hist[0])  # sizing pass (launch count, host time)
        host_ms = (time.perf_counter() - t0) * 1e3
        per_step = max(sum(v["launches"] for v in fo.fastocr_get_timing(h).values()), 1)
        chunk = max(1, EVENT_LAUNCHES_PER_CHUNK // per_step)
        spin_target = 3.0 * host_ms * chunk + 2.0  # ms; the host needs about host_ms per step
        spin = int(cycles_per_ms * spin_target)
        fo.fastocr_reset_timing(h)
        worst_host = 0.0
        for c0 in range(1, len(steps), chunk):
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                torch.cuda._sleep(spin)
                t0 = time.perf_counter()
                for i in range(c0, min(c0 + chunk, len(steps))):
                    eager_step(h, steps[i], out_hist[i])
                worst_host = max(worst_host, (time.perf_counter() - t0) * 1e3)
            kt = fo.fastocr_get_timing(h)  # synchronises and accumulates
        fo.fastocr_set_timing(h, False)
        log(f"kernel timing: {len(steps) - 1} steps in chunks of {chunk}, each enqueued in at most "
            f"{worst_host:.1f} ms behind a {spin_target:.1f} ms spin")
        if worst_host > 0.8 * spin_target:
            log("warning: the spin may have ended before a chunk was enqueued; kernel times include idle gaps")
        return kt, len(steps) - 1

    def record_step(h, t, focal):
        k_max = fo.fastocr_get_info(h)["k_max"]
        with torch.cuda.stream(stream):
            rec = {"t": t, "outs": torch.empty((L, B, Hq, d), dtype=io, device=dev),
                   "sel": torch.zeros((L, B, k_max), dtype=torch.int32, device=dev),
                   "cnt": torch.zeros((L, B), dtype=torch.int32, device=dev)}
            for l in range(L):
                if l not in focal:
                    fo.fastocr_get_selection(h, rec["sel"][l], rec["cnt"][l])
                fo.fastocr_attend(h, l, q_at(t)[l], Kd[l], Vd[l], lens_at(t), rec["outs"][l])
                if l in focal:
                    fo.fastocr_get_selection(h, rec["sel"][l], rec["cnt"][l])
        torch.cuda.synchronize()
        return {"t": t, "outs": rec["outs"].float().cpu().numpy().astype(np.float64),
                "sel": rec["sel"].cpu().numpy(), "cnt": rec["cnt"].cpu().numpy()}

    results = {}
    outs = {}
    recorded = None
    for mode in (["pruned"] if args.profile_only else ["pruned", "full"]):
        h = make(mode)
        with torch.cuda.stream(stream):
            focal = None
            for t in range(w):  # warm-up steps (full attention on every layer in both modes)
                eager_step(h, t, out_stage)
            if mode == "pruned":
                torch.cuda.synchronize()
                p0 = time.perf_counter()
                focal = fo.fastocr_profile_warmup(h)
                profile_ms = (time.perf_counter() - p0) * 1e3
                gpu_ratios = fo.fastocr_get_layer_ratios(h)
            for t in range(w, t_timed):  # untimed steps
                eager_step(h, t, out_stage)
        torch.cuda.synchronize()
        r = {"focal": focal}
        timed_steps = phase_steps["graph"]
        # capture one step (the capture itself advances the kept set by one
        # step, so it runs at t_timed - 1's inputs into a scratch copy)
        g = capture(h) if not args.no_graph else None
        r["step_ms"] = time_steps(h, timed_steps, g)
        # per-kernel timing + recorded outputs on the next K steps
        out_hist = torch.empty((K, L, B, Hq, d), dtype=io, device=dev)
        r["kernels"], r["kernel_steps"] = kernel_times(h, phase_steps["events"], out_hist)
        if do_scrub:
            r["scrubbed_step_ms"] = time_steps_scrubbed(phase_steps["scrub"], g)
        del g
        if do_append:
            # each capture advances the kept set by one step, so the two
            # variants run on consecutive step ranges
            r["append_separate_ms"] = time_append(h, phase_steps["append_separate"], 0, False)
            r["append_fused_ms"] = time_append(h, phase_steps["append_fused"], K, True)
        outs[mode] = out_hist.float()
        if mode == "pruned" and not args.profile_only:
            # one more step, eager and recorded, for the oracle check beside
            # the CPU baseline: every layer's output, the set each non-focal
            # layer attends with and the set each focal layer picks
            recorded = record_step(h, phase_steps["events"][-1], focal)
        fo.fastocr_destroy(h)
        results[mode] = r
        log(f"{mode}: {r['step_ms']:.4f} ms/step ({'eager' if args.no_graph else 'graph'})")

    if args.calibrate_copy:
        # int64 add: reads and writes CAL_BYTES once each with a kernel of its own
        src = torch.empty(CAL_BYTES // 8, dtype=torch.int64, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {CAL_BYTES >> 20} MiB done")

    focal = results["pruned"]["focal"]
    ev_steps = phase_steps["events"]

    # algorithmic K/V bytes (rows read x 2*Hkv*d*e)
    e = 2 if wl.dtype == "bf16" else 4
    R = 2 * Hkv * d * e
    from_k = lambda n: max(1, min(n, math.ceil(wl.tau * n - 1e-9))) if n > 0 else 0  # noqa: E731
    n_img = st.n_img.astype(np.int64)
    kb = np.array([from_k(int(n)) for n in n_img])
    lens_ev = np.stack([st.lens(t)[:, 1] for t in ev_steps]).astype(np.int64)  # [K, B]
    rows_focal = lens_ev.sum(axis=1).mean()
    rows_sparse = (kb[None, :] + lens_ev - n_img[None, :]).sum(axis=1).mean()
    C = len(focal)
    bytes_pruned = R * (C * rows_focal + (L - C) * rows_sparse)
    bytes_full = R * L * rows_focal

    def run_alg_bytes():
        """Average algorithmic K/V bytes per launch of each split class over
        every dispatch of a profile-only run (warm-up, untimed, graph-phase
        and event-phase steps of the pruned handle), for comparison with
        hardware counters taken over the same run."""
        pruned_steps = list(range(w, t_timed)) + phase_steps["graph"] + phase_steps["events"]
        n = {"full_split": [0, 0.0], "focal_split": [0, 0.0], "sparse_split": [0, 0.0]}
        for t in range(w):
            n["full_split"][0] += L
            n["full_split"][1] += L * R * float(st.lens(t)[:, 1].sum())
        # a focal layer followed by a focal layer runs the full pass alone
        unused = (sum(1 for l in focal if l + 1 < L and l + 1 in focal)
                  if os.environ.get("FASTOCR_SKIP_DEAD_PICKS", "1") != "0" else 0)
        for t in pruned_steps:
            ln = st.lens(t)[:, 1].astype(np.int64)
            n["focal_split"][0] += C - unused
            n["focal_split"][1] += (C - unused) * R * float(ln.sum())
            n["full_split"][0] += unused
            n["full_split"][1] += unused * R * float(ln.sum())
            other = "full_split" if wl.tau >= 1.0 else "sparse_split"
            rows = ln.sum() if wl.tau >= 1.0 else (kb + ln - n_img).sum()
            n[other][0] += L - C
            n[other][1] += (L - C) * R * float(rows)
        return {k: int(v[1] / v[0]) for k, v in n.items() if v[0]}

    def per_step(r):
        """Per kernel class: average launch time and launches per step."""
        out = {}
        for k, v in r["kernels"].items():
            if v["timed"]:
                out[k] = (v["total_ms"] / v["timed"], v["launches"] / r["kernel_steps"])
        return out

    kp = per_step(results["pruned"])
    kernel_sum_ms = sum(a * n for a, n in kp.values())
    pr_ms = results["pruned"]["step_ms"]
    value_us = pr_ms * 1e3

    # the attention pass with the most time per step and its roofline (the
    # merge and top-k are latency-bound: at B=1 the merges can take longer
    # in sum than the kept-token passes)
    passes = [k for k in kp if k in ("full_split", "focal_split", "sparse_split")]
    dom = max(passes, key=lambda k: kp[k][0] * kp[k][1])
    dom_avg_ms = kp[dom][0]
    # algorithmic K/V bytes per launch of the split kernels (a non-focal
    # layer at tau = 1 runs the full pass)
    split_bytes = {"focal_split": R * rows_focal, "sparse_split": R * rows_sparse, "full_split": R * rows_focal}
    per_launch_bytes = split_bytes.get(dom)
    roofline = None
    if per_launch_bytes is not None:
        achieved = per_launch_bytes / (dom_avg_ms * 1e-3) / 1e9
        traffic, traffic_alg = read_traffic(dom, wl.name)
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "avg_launch_us": round(dom_avg_ms * 1e3, 3),
                    "bytes_per_launch": int(per_launch_bytes),
                    # the algorithmic bytes per launch of the counter run's own dispatches
                    "traffic_run_alg_bytes": traffic_alg}
    def kernel_table(kr):
        """Per kernel class: launch time, launches and time per step; for the
        split kernels also the algorithmic K/V bytes per launch and the rate."""
        tab = {}
        for k, (a, n) in kr.items():
            e = {"avg_us": round(a * 1e3, 3), "launches_per_step": n, "us_per_step": round(a * n * 1e3, 3)}
            if k in split_bytes:
                e["alg_bytes_per_launch"] = int(split_bytes[k])
                e["GBps"] = round(split_bytes[k] / (a * 1e-3) / 1e9, 1)
            tab[k] = e
        return tab

    per_kernel = kernel_table(kp)
    extra = {
        "focal_layers": focal,
        "kernel_sum_us_per_step": round(kernel_sum_ms * 1e3, 2),
        "algorithmic_MB_per_step": round(bytes_pruned / 1e6, 2),
        "GBps_vs_step_time": round(bytes_pruned / (pr_ms * 1e-3) / 1e9, 1),
        "GBps_vs_kernel_sum": round(bytes_pruned / (kernel_sum_ms * 1e-3) / 1e9, 1),
        "per_kernel": per_kernel,
    }
    if "full" in results:
        fr = results["full"]
        full_ms = fr["step_ms"]
        full_kernel_ms = sum(a * n for a, n in per_step(fr).values())
        extra.update({
            "full_us_per_step": round(full_ms * 1e3, 2),
            "full_kernel_sum_us_per_step": round(full_kernel_ms * 1e3, 2),
            "full_algorithmic_MB_per_step": round(bytes_full / 1e6, 2),
            "full_GBps_vs_step_time": round(bytes_full / (full_ms * 1e-3) / 1e9, 1),
            "full_per_kernel": kernel_table(per_step(fr)),
            "speedup_vs_full": round(full_ms / pr_ms, 3),
            "speedup_vs_full_kernel_sum": round(full_kernel_ms / kernel_sum_ms, 3),
        })
        # pruned-vs-full deviation on non-focal layers
        a, b = outs["pruned"], outs["full"]
        nf = [l for l in range(L) if l not in focal]
        diff = (a[:, nf] - b[:, nf])
        extra["deviation_nonfocal"] = {
            "max_abs": round(float(diff.abs().max()), 4),
            "rel_l2": round(float(diff.norm() / b[:, nf].norm()), 4)}
        fl = (a[:, focal] - b[:, focal]).abs().max()
        extra["deviation_focal_max_abs"] = float(fl)

    if "scrubbed_step_ms" in results["pruned"]:
        # single replays, each after a MALL scrub or after a spin of the same
        # length (control)
        sc = {"scrub_MiB": args.scrub_mb}
        for mode in ("pruned", "full"):
            if mode in results and "scrubbed_step_ms" in results[mode]:
                v = results[mode]["scrubbed_step_ms"]
                sc[f"{mode}_us_per_step"] = round(v[True] * 1e3, 2)
                sc[f"{mode}_control_us_per_step"] = round(v[False] * 1e3, 2)
        if "full_us_per_step" in sc:
            sc["speedup_vs_full"] = round(sc["full_us_per_step"] / sc["pruned_us_per_step"], 3)
        extra["mall_scrubbed"] = sc
    if "append_fused_ms" in results["pruned"]:
        ap = {}
        for mode in ("pruned", "full"):
            if mode in results and "append_fused_ms" in results[mode]:
                ap[f"{mode}_separate_append_us_per_step"] = round(results[mode]["append_separate_ms"] * 1e3, 2)
                ap[f"{mode}_fused_append_us_per_step"] = round(results[mode]["append_fused_ms"] * 1e3, 2)
        extra["append"] = ap
    if "full" in results:
        # periodic re-selection (reprofile_every = R): every R pruned steps
        # cost a window of w full-attention steps plus one profile call
        R = 256
        over = (w * (results["full"]["step_ms"] - pr_ms) + profile_ms) / (R + w)
        extra["reselection"] = {"profile_call_us": round(profile_ms * 1e3, 1), "every_R": R,
                                "amortized_us_per_step": round(over * 1e3, 2)}
    if focal is not None and len(focal) < L:
        # how clearly the warm-up separates the focal layers: the gap between
        # the |C|-th and the (|C|+1)-th layer's image-attention ratio
        ranked = sorted(gpu_ratios, reverse=True)
        C = len(focal)
        extra["focal_margin"] = {"ratio_C": round(ranked[C - 1], 7), "ratio_next": round(ranked[C], 7),
                                 "abs": float(f"{ranked[C - 1] - ranked[C]:.3e}"),
                                 "rel": float(f"{(ranked[C - 1] - ranked[C]) / ranked[C - 1]:.3e}")}
    if not args.profile_only:
        extra["pack_image_first"] = pack_probe(torch, fo, Kd, Vd, st.n_img, stream)
        extra["platform"] = platform_probe(torch, fo, stream)

    cpu = None
    if args.cpu_seconds > 0 and not args.profile_only:
        cpu, extra["oracle_check"] = cpu_baseline(wl, st, Kd, Vd, Qall, slot, focal, args.cpu_seconds, recorded)

    if args.profile_only:
        extra["alg_bytes_per_launch_run"] = run_alg_bytes()
    line = {
        "metric": "decode-step attention us (all layers) + HBM GB/s, tau=0.05 vs full attention",
        "value": round(value_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(pr_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) KV, moving fixation-window queries)",
        "config": {"workload": wl.description, "name": wl.name, "batch": B, "layers": L,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "tau": wl.tau,
                   "num_focal": wl.num_focal, "warmup_steps": w,
                   "timing": "hip graph replay" if not args.no_graph else "eager",
                   "decode_steps": wl.steps,
                   "timed_steps": f"{K} per phase, spread over decode steps {t_timed}..{wl.steps - 1}",
                   **({"tp_shard": T, "tp_note": f"one rank of {T}: 1/{T} of the heads; the per-focal-layer "
                       "score all-reduce across ranks is not included"} if T != 1 else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


def pack_probe(torch, fo, Kd, Vd, n_img, stream):
    """One-time cost of bringing a two-page layout (the image split into two
    pages behind 20 text tokens, 12 text tokens between them) into the
    image-first layout: every layer's K and V cache gathered once."""
    B, Hkv, S, d = Kd[0].shape
    maps = []
    for b in range(B):
        n = int(n_img[b])
        spans = [(20, n // 2), (32 + n // 2, n - n // 2)]
        maps.append(fo.fastocr_image_first_map(spans, S)[1])
    row_map = torch.tensor(maps, dtype=torch.int32, device=Kd[0].device)
    rows = torch.full((B,), S, dtype=torch.int32, device=Kd[0].device)
    dst = torch.empty_like(Kd[0])
    with torch.cuda.stream(stream):
        fo.fastocr_pack_rows(Kd[0], dst, row_map, rows, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for k, v in zip(Kd, Vd):
            fo.fastocr_pack_rows(k, dst, row_map, rows, stream=stream)
            fo.fastocr_pack_rows(v, dst, row_map, rows, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    moved = 2 * 2 * len(Kd) * Kd[0].numel() * Kd[0].element_size()  # read + write, K and V
    del dst
    return {"us_all_layers": round(ms * 1e3, 1), "launches": 2 * len(Kd),
            "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}


def platform_probe(torch, fo, stream, launches=200, copy_bytes=1 << 30):
    """Context for the kernel times: the per-launch floor of back-to-back
    graph-replayed null kernels, a device-to-device copy rate, the HBM read
    rate of the library's stream-read probe over 1 GiB, and the probe's time
    per launch for reads of 1-64 MB (graph-replayed back to back, each launch
    reading a region no earlier launch of the series read, so it comes from
    HBM and not from the MALL)."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def best_replay(g, reps=4):
        best = None
        with torch.cuda.stream(stream):
            for _ in range(reps):
                a, b = ev(), ev()
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                t = a.elapsed_time(b)
                best = t if best is None else min(best, t)
        return best

    try:
        with torch.cuda.stream(stream):
            torch.cuda._sleep(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(launches):
                torch.cuda._sleep(0)
        out["null_kernel_graph_us"] = round(best_replay(g) * 1e3 / launches, 3)
        del g
    except RuntimeError as exc:  # the spin kernel could not be captured
        out["null_kernel_graph_us"] = None
        log(f"null-kernel probe skipped: {exc}")
    src = torch.ones(copy_bytes // 8, dtype=torch.int64, device="cuda")
    dst = torch.empty_like(src)
    best = None
    with torch.cuda.stream(stream):
        for _ in range(4):
            a, b = ev(), ev()
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
    out["copy_GBps"] = round(2 * copy_bytes / (best * 1e-3) / 1e9, 1)  # read + write
    out["copy_MiB"] = copy_bytes >> 20
    del src, dst

    # stream-read probe
    buf = torch.ones(PROBE_BUFFER // 8, dtype=torch.int64, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    torch.cuda.synchronize()

    def series(nbytes, wgs, count):
        """Per-launch ms of `count` graph-replayed probe launches of `nbytes`
        each, at successive offsets of the buffer."""
        g = torch.cuda.CUDAGraph()
        step = nbytes // 8
        with torch.cuda.stream(stream):
            fo.fastocr_probe_read(buf, nbytes, wgs, sink, stream=stream)  # first launch outside the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                off = (i * step) % (buf.numel() - step + 1)
                fo.fastocr_probe_read(buf[off:], nbytes, wgs, sink, stream=stream)
        torch.cuda.synchronize()
        ms = best_replay(g, reps=3) / count
        del g
        return ms

    peak = {}
    for per_cu in (2, 4, 8):
        ms = series(1 << 30, per_cu * num_cu, 2)
        peak[per_cu] = (1 << 30) / (ms * 1e-3) / 1e9
    best_cu = max(peak, key=peak.get)
    out["read_probe_GBps"] = round(peak[best_cu], 1)
    out["read_probe_workgroups_per_cu"] = best_cu
    curve = {}
    for mb in PROBE_SIZES_MB:
        nbytes = mb << 20
        count = max(8, min(64, (PROBE_BUFFER // nbytes)))
        best = None
        for wgs in sorted({max(1, min(8 * num_cu, nbytes // (256 * 16))),
                           max(1, min(8 * num_cu, nbytes // (256 * 64))), 2 * num_cu}):
            ms = series(nbytes, wgs, count)
            if best is None or ms < best[0]:
                best = (ms, wgs)
        curve[f"{mb}MB"] = {"us_per_launch": round(best[0] * 1e3, 2),
                            "GBps": round(nbytes / (best[0] * 1e-3) / 1e9, 1), "workgroups": best[1]}
    out["read_curve"] = curve
    del buf, sink
    return out


def host_cpu():
    """(nproc, CPU model name, BLAS threads) of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    return os.cpu_count(), model, threads


def cpu_baseline(wl, st, Kd, Vd, Qall, slot, focal_gpu, budget_s, recorded):
    """The CPU oracle, as written, timed on a bounded sample of the same run,
    and the oracle's check of one recorded GPU step.

    The sample is the recorded decode step's layers, focal layers that pick a
    kept set and non-focal layers alternately (spread over the depth), until
    `budget_s` seconds of float64 oracle work: a focal layer is full
    attention + head-summed scores + top-k, a non-focal layer is attention
    over the kept set the GPU attended with.  The step time is the sum over
    all layers of the median time of their kind.  The same layers then run in float32 for the float32 figure.
    Reading a layer's cache back and converting it is not timed.

    The check: every sampled layer's GPU output against the float64 oracle
    (non-focal layers conditioned on the GPU's set), and for focal layers the
    Jaccard overlap of the GPU's kept set with the oracle's own set (the
    oracle's unconditioned pick: a focal layer picks from the full cache).
    """
    from oracle import full_attention, image_scores, kept_count, select_top, sparse_attention

    nproc, model, threads = host_cpu()
    L, B = wl.num_layers, wl.batch
    t = recorded["t"]
    lens = st.lens(t)
    scale = 1.0 / math.sqrt(wl.head_dim)
    focal = [int(x) for x in focal_gpu]
    unused = {l for l in focal if l + 1 < L and l + 1 in focal}
    picking = [l for l in focal if l not in unused]
    nonfocal = [l for l in range(L) if l not in focal]
    # non-focal layers in an order that spreads a short sample over the depth
    spread, stride = [], max(1, len(nonfocal) // 8)
    for start in range(stride):
        spread += nonfocal[start::stride]
    order = []
    for i in range(max(len(picking), len(spread))):
        order += ([("focal", picking[i])] if i < len(picking) else []) + \
                 ([("sparse", spread[i])] if i < len(spread) else [])

    def run_layer(kind, l, K, V, q, dtype):
        outs, sets = [], []
        for b in range(B):
            n, length = int(lens[b, 0]), int(lens[b, 1])
            if kind == "focal":
                out, p = full_attention(q[b], K[b], V[b], length, scale, dtype)
                sets.append(select_top(image_scores(p, n), kept_count(wl.tau, n)))
            else:
                c = int(recorded["cnt"][l, b])
                out = sparse_attention(q[b], K[b], V[b], recorded["sel"][l, b, :c], n, length, scale,
                                       dtype=dtype)
            outs.append(out)
        return np.stack(outs), sets

    times = {np.float64: {"focal": [], "sparse": []}, np.float32: {"focal": [], "sparse": []}}
    worst_abs, worst_rel, jac, checked, per_layer = 0.0, 0.0, [], [], []
    spent = 0.0
    for kind, l in order:
        if spent > budget_s and times[np.float64]["focal"] and times[np.float64]["sparse"]:
            break
        K = Kd[l].float().cpu().numpy()
        V = Vd[l].float().cpu().numpy()
        q = Qall[slot[t], l].float().cpu().numpy()
        for dtype in (np.float64, np.float32):
            Kc, Vc, qc = K.astype(dtype), V.astype(dtype), q.astype(dtype)
            s0 = time.perf_counter()
            out, sets = run_layer(kind, l, Kc, Vc, qc, dtype)
            dt = time.perf_counter() - s0
            times[dtype][kind].append(dt)
            if dtype is np.float64:
                spent += dt
                got = recorded["outs"][l]
                err_abs = float(np.abs(got - out).max())
                err_rel = float(np.linalg.norm(got - out) / max(np.linalg.norm(out), 1e-30))
                worst_abs, worst_rel = max(worst_abs, err_abs), max(worst_rel, err_rel)
                per_layer.append((err_rel, err_abs, l, kind))
                checked.append(l)
                for b, want in enumerate(sets):
                    gpu = set(int(j) for j in recorded["sel"][l, b, :int(recorded["cnt"][l, b])])
                    ours = set(int(j) for j in want)
                    jac.append(len(gpu & ours) / max(len(gpu | ours), 1))
            del Kc, Vc, qc
        del K, V

    def step_us(tt):
        med = {k: float(np.median(v)) for k, v in tt.items() if v}
        f = med.get("focal", med.get("sparse"))
        n_ = med.get("sparse", f)
        return (len(focal) * f + (L - len(focal)) * n_) * 1e6

    us64, us32 = step_us(times[np.float64]), step_us(times[np.float32])
    n_f, n_s = len(times[np.float64]["focal"]), len(times[np.float64]["sparse"])
    log(f"cpu oracle: {n_f} focal + {n_s} non-focal layers of step {t}; step estimate float64 "
        f"{us64 / 1e3:.1f} ms, float32 {us32 / 1e3:.1f} ms; {nproc} CPUs ({model}), BLAS threads {threads}")
    sample = (f"float64 numpy oracle on {n_f} focal and {n_s} non-focal layers of decode step {t} "
              f"(focal: full attention + scores + top-k; non-focal: attention over the GPU's kept set), "
              f"step = {len(focal)} focal + {L - len(focal)} non-focal layers at the median time of their kind")
    cpu = {"value": round(us64, 1), "unit": "us/step", "cores": threads, "kind": "oracle", "sample": sample,
           "nproc": nproc, "cpu_model": model, "blas_threads": threads,
           "float32_value": round(us32, 1), "layers_timed": n_f + n_s}
    tol_abs, tol_rel = (2e-2, 1e-2) if wl.dtype == "bf16" else (1e-5, None)
    check = {"step": t, "layers": checked, "max_abs_err": float(f"{worst_abs:.3e}"),
             "max_rel_l2": float(f"{worst_rel:.3e}"), "tolerance_abs": tol_abs, "tolerance_rel_l2": tol_rel,
             "within_tolerance": bool(worst_abs <= tol_abs and (tol_rel is None or worst_rel <= tol_rel)),
             "jaccard_vs_oracle_sets": round(float(np.mean(jac)), 4) if jac else None,
             "focal_sets_compared": len(jac),
             "worst_layers": [{"layer": l, "kind": k, "max_abs": float(f"{a:.3e}"), "rel_l2": float(f"{r:.3e}")}
                              for r, a, l, k in sorted(per_layer, reverse=True)[:6]]}
    return cpu, check


if __name__ == "__main__":
    main()
