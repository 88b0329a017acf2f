"""Decode-step attention benchmark of the FastOCR library on one MI355X.

Workload (default): Qwen2.5-VL-7B-like decode attention, batch 1, 28 layers,
28 query / 4 KV heads, head_dim 128, bf16 KV cache, 6400 image tokens (80x80
page) + 64 prompt tokens, tau = 0.05, w = 8 warm-up steps, |C| = 4 focal
layers; synthetic seeded inputs (K, V ~ N(0,1); queries follow a 3x5 fixation
window that moves one cell per step).

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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="7b-b1")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline sample (0 disables it)")
    ap.add_argument("--profile-only", action="store_true",
                    help="skip the CPU baseline and the FULL comparison (for profiler runs)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import dynamic_kv_cache_amd as fo
    from workload import DeviceGenerator, get_workload, make_structure

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    overrides = {}
    if args.tau is not None:
        overrides["tau"] = args.tau
    if args.sigma is not None:
        overrides["sigma"] = args.sigma
    wl = get_workload(args.workload, **overrides)
    st = make_structure(wl)
    gen = DeviceGenerator(wl, st, device=dev)
    L, B, Hq, Hkv, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    w, W, K = wl.warmup_steps, args.warmup, args.steps
    # decode steps used: warm-up, untimed pruned, timed (graph), timed (per-kernel events)
    t_timed = w + W
    t_events = t_timed + K
    n_steps = t_events + K
    assert n_steps <= wl.steps, f"--steps/--warmup too large for {wl.steps} decode steps"
    io = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    t0 = time.time()
    Kd, Vd, Qall = [], [], torch.empty((n_steps, L, B, Hq, d), dtype=io, device=dev)
    for l in range(L):
        k, v = gen.layer_kv(l)
        Kd.append(k)
        Vd.append(v)
        Qall[:, l] = gen.layer_queries(l, range(n_steps), k)
    lens_all = torch.from_numpy(np.stack([st.lens(t) for t in range(n_steps)])).to(dev)
    torch.cuda.synchronize()
    log(f"inputs for {wl.name} ready in {time.time() - t0:.1f}s "
        f"(KV {2 * L * B * Hkv * st.max_seq_len * d * Kd[0].element_size() / 1e9:.2f} GB)")

    stream = torch.cuda.Stream()

    def make(mode):
        cfg = fo.Config(num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, batch=B,
                        max_seq_len=st.max_seq_len, max_img_tokens=int(st.n_img.max()),
                        min_img_tokens=int(st.n_img.min()), tau=wl.tau, num_focal=wl.num_focal,
                        warmup_steps=w, dtype=wl.dtype, mode=mode)
        return fo.fastocr_create(cfg, stream)

    q_stage = torch.empty((L, B, Hq, d), dtype=io, device=dev)
    lens_stage = torch.empty((B, 2), dtype=torch.int32, device=dev)
    out_stage = torch.empty((L, B, Hq, d), dtype=io, device=dev)

    def eager_step(h, t, out):
        for l in range(L):
            fo.fastocr_attend(h, l, Qall[t, l], Kd[l], Vd[l], lens_all[t], out[l])

    def time_steps(h, steps, graph):
        """Wall time per step over `steps` (HIP events on the library stream)."""
        with torch.cuda.stream(stream):
            if graph is not None:
                q_stage.copy_(Qall[steps[0]])
                lens_stage.copy_(lens_all[steps[0]])
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for t in steps:
                if graph is not None:
                    q_stage.copy_(Qall[t])
                    lens_stage.copy_(lens_all[t])
                    graph.replay()
                else:
                    eager_step(h, t, out_stage)
            ev1.record(stream)
            torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / len(steps)

    def capture(h):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            q_stage.copy_(Qall[t_timed])
            lens_stage.copy_(lens_all[t_timed])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for l in range(L):
                fo.fastocr_attend(h, l, q_stage[l], Kd[l], Vd[l], lens_stage, out_stage[l])
        torch.cuda.synchronize()
        return g

    results = {}
    outs = {}
    for mode in (["pruned"] if args.profile_only else ["pruned", "full"]):
        h = make(mode)
        with torch.cuda.stream(stream):
            focal = None
            for t in range(w):  # warm-up steps (full attention on every layer in both modes)
                eager_step(h, t, out_stage)
            if mode == "pruned":
                focal = fo.fastocr_profile_warmup(h)
            for t in range(w, t_timed):  # untimed steps
                eager_step(h, t, out_stage)
        torch.cuda.synchronize()
        r = {"focal": focal}
        timed_steps = list(range(t_timed, t_events))
        if not args.no_graph:
            # capture one step (the capture itself advances the kept set by
            # one step, so it runs at t_timed - 1's inputs into a scratch copy)
            g = capture(h)
            r["graph_ms"] = time_steps(h, timed_steps, g)
            del g
        else:
            with torch.cuda.stream(stream):
                for t in timed_steps:
                    eager_step(h, t, out_stage)
        # per-kernel event timing + recorded outputs on the next K steps
        out_hist = torch.empty((K, L, B, Hq, d), dtype=io, device=dev)
        ev_steps = list(range(t_events, n_steps))
        fo.fastocr_set_timing(h, True)
        fo.fastocr_reset_timing(h)
        with torch.cuda.stream(stream):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for i, t in enumerate(ev_steps):
                eager_step(h, t, out_hist[i])
            ev1.record(stream)
        torch.cuda.synchronize()
        r["eager_events_ms"] = ev0.elapsed_time(ev1) / K
        r["kernels"] = fo.fastocr_get_timing(h)
        fo.fastocr_set_timing(h, False)
        outs[mode] = out_hist.float()
        fo.fastocr_destroy(h)
        results[mode] = r
        log(f"{mode}: graph {r.get('graph_ms')} ms/step, eager+events {r['eager_events_ms']:.3f} ms/step")

    focal = results["pruned"]["focal"]
    ev_steps = list(range(t_events, n_steps))

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

    kp = results["pruned"]["kernels"]
    kernel_sum_ms = sum(v["total_ms"] for v in kp.values()) / K
    pr_ms = results["pruned"].get("graph_ms") or results["pruned"]["eager_events_ms"]
    value_us = pr_ms * 1e3

    # dominant kernel of the pruned step and its roofline
    dom = max(kp, key=lambda k: kp[k]["total_ms"])
    dom_avg_ms = kp[dom]["total_ms"] / max(kp[dom]["launches"], 1)
    per_launch_bytes = {
        "focal_split": R * rows_focal,
        "sparse_split": R * rows_sparse,
    }.get(dom)
    roofline = None
    if per_launch_bytes is not None:
        achieved = per_launch_bytes / (dom_avg_ms * 1e-3) / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None, "avg_launch_us": round(dom_avg_ms * 1e3, 3),
                    "bytes_per_launch": int(per_launch_bytes)}
    per_kernel = {k: {"avg_us": round(v["total_ms"] / max(v["launches"], 1) * 1e3, 3),
                      "launches_per_step": v["launches"] / K,
                      "us_per_step": round(v["total_ms"] / K * 1e3, 3)}
                  for k, v in kp.items() if v["launches"]}
    extra = {
        "focal_layers": focal,
        "kernel_sum_us_per_step": round(kernel_sum_ms * 1e3, 2),
        "eager_events_us_per_step": round(results["pruned"]["eager_events_ms"] * 1e3, 2),
        "algorithmic_MB_per_step": round(bytes_pruned / 1e6, 2),
        "GBps_vs_step_time": round(bytes_pruned / (pr_ms * 1e-3) / 1e9, 1),
        "GBps_vs_kernel_sum": round(bytes_pruned / (kernel_sum_ms * 1e-3) / 1e9, 1),
        "per_kernel": per_kernel,
    }
    if "full" in results:
        fr = results["full"]
        full_ms = fr.get("graph_ms") or fr["eager_events_ms"]
        kf = fr["kernels"]
        full_kernel_ms = sum(v["total_ms"] for v in kf.values()) / K
        extra.update({
            "full_us_per_step": round(full_ms * 1e3, 2),
            "full_kernel_sum_us_per_step": round(full_kernel_ms * 1e3, 2),
            "full_algorithmic_MB_per_step": round(bytes_full / 1e6, 2),
            "full_GBps_vs_step_time": round(bytes_full / (full_ms * 1e-3) / 1e9, 1),
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

    cpu = None
    if args.cpu_seconds > 0 and not args.profile_only:
        cpu = cpu_baseline(wl, st, Kd, Vd, Qall, focal, args.cpu_seconds)

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
                   "timing": "hip graph replay" if not args.no_graph else "eager"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, st, Kd, Vd, Qall, focal_gpu, budget_s):
    """The CPU oracle, as written, timed on a bounded sample of the same run.

    Whole decode steps when every layer's cache fits comfortably in host
    memory as float64 (the 7B-like workloads); otherwise one focal and one
    non-focal layer of one pruned step are timed and the step time is
    extrapolated to all layers.
    """
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    from oracle import DecodeOracle, full_attention, sparse_attention, image_scores, kept_count, select_top

    L = wl.num_layers
    host = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    layer_bytes = Kd[0].numel() * 8 * 2
    if L * layer_bytes < 4e9:
        kv64 = [(host(k), host(v)) for k, v in zip(Kd, Vd)]
        q_of = lambda t: (lambda l: host(Qall[t, l]))  # noqa: E731
        orc = DecodeOracle(num_layers=L, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                           head_dim=wl.head_dim, tau=wl.tau, num_focal=wl.num_focal,
                           warmup_steps=wl.warmup_steps)
        t0 = time.time()
        for t in range(wl.warmup_steps):
            orc.step(t, q_of(t), lambda l: kv64[l], st.lens(t))
        warm_s = time.time() - t0
        times = []
        t = wl.warmup_steps
        begin = time.time()
        while time.time() - begin < budget_s and t < Qall.shape[0]:
            s0 = time.time()
            orc.step(t, q_of(t), lambda l: kv64[l], st.lens(t))
            times.append(time.time() - s0)
            t += 1
        us = float(np.median(times)) * 1e6 if times else None
        log(f"cpu oracle: warm-up {warm_s:.1f}s, {len(times)} pruned steps, median {us:.0f} us/step, "
            f"focal {[int(c) for c in orc.focal]} (gpu {focal_gpu})")
        sample = (f"float64 numpy oracle: {wl.warmup_steps} warm-up steps then {len(times)} pruned "
                  f"decode steps (all {L} layers) of the same workload; median per pruned step")
    else:
        t = wl.warmup_steps
        lens = st.lens(t)
        scale = 1.0 / math.sqrt(wl.head_dim)
        lf = int(focal_gpu[0])
        ln = next(l for l in range(L) if l not in focal_gpu)
        Kf, Vf, qf = host(Kd[lf]), host(Vd[lf]), host(Qall[t, lf])
        s0 = time.time()
        sets = []
        for b in range(wl.batch):
            n, length = int(lens[b, 0]), int(lens[b, 1])
            _, p = full_attention(qf[b], Kf[b], Vf[b], length, scale)
            sets.append(select_top(image_scores(p, n), kept_count(wl.tau, n)))
        t_focal = time.time() - s0
        del Kf, Vf
        Kn, Vn, qn = host(Kd[ln]), host(Vd[ln]), host(Qall[t, ln])
        s0 = time.time()
        for b in range(wl.batch):
            n, length = int(lens[b, 0]), int(lens[b, 1])
            sparse_attention(qn[b], Kn[b], Vn[b], sets[b], n, length, scale)
        t_sparse = time.time() - s0
        C = len(focal_gpu)
        us = (C * t_focal + (L - C) * t_sparse) * 1e6
        log(f"cpu oracle (sampled layers): focal layer {t_focal:.2f}s, non-focal layer {t_sparse:.2f}s, "
            f"step estimate {us / 1e6:.1f}s")
        sample = (f"float64 numpy oracle on one focal and one non-focal layer of pruned step "
                  f"{t}, extrapolated to {C} focal + {L - C} non-focal layers")
    return {"value": round(us, 1) if us else None, "unit": "us/step", "cores": threads,
            "kind": "oracle", "sample": sample}


if __name__ == "__main__":
    main()
