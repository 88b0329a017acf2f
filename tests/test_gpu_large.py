"""GPU parity at the full sizes of the large workloads, on sampled steps.

The library runs every decode step of the real shape (the same handle
configuration and launch geometry the benchmark times); the oracle checks
sampled steps one by one, reading the exact device inputs back layer by
layer:
* every warm-up layer ratio for the 16-sequence ragged batch (so the focal
  set is checked exactly); for the 32B/72B-like stacks the ratios of the
  focal layers, the next-ranked layers and a few others (full warm-up
  attention on every layer would take the float64 oracle many minutes);
* at each sampled step, every focal layer (outputs, head-summed scores,
  kept sets under the band rule) and a sample of non-focal layers
  (outputs, conditioned on the kept set the GPU used);
* the warm start of a step equals the set after the previous step's
  deepest focal layer.
"""

import math
import time

import numpy as np
import pytest
import torch

import dynamic_kv_cache_amd as fo
from oracle import (choose_focal_layers, full_attention, image_mass, image_scores, kept_count,
                    select_top, sparse_attention)
from workload import DeviceGenerator, get_workload, make_structure

from gpu_harness import check_out, check_scores, check_set, log, unused_picks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_sampled(wl, sample_steps, all_ratio_layers: bool):
    t0 = time.time()
    st = make_structure(wl)
    gen = DeviceGenerator(wl, st, device=DEV)
    L, B, Hq, d, T = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim, wl.steps
    Kd, Vd, Qd = [], [], []
    for l in range(L):
        k, v = gen.layer_kv(l)
        Kd.append(k)
        Vd.append(v)
        Qd.append(gen.layer_queries(l, range(T), k))
    lens = torch.from_numpy(np.stack([st.lens(t) for t in range(T)])).to(DEV)
    torch.cuda.synchronize()
    log(f"[{wl.name}] inputs in {time.time() - t0:.1f}s")
    cfg = fo.Config(num_layers=L, num_q_heads=Hq, num_kv_heads=wl.num_kv_heads, head_dim=d, batch=B,
                    max_seq_len=st.max_seq_len, max_img_tokens=int(st.n_img.max()),
                    min_img_tokens=int(st.n_img.min()), max_text_tokens=int(st.n_prompt.max()) + T,
                    tau=wl.tau, num_focal=wl.num_focal,
                    warmup_steps=wl.warmup_steps, dtype=wl.dtype)
    h = fo.fastocr_create(cfg)
    k_max = fo.fastocr_get_info(h)["k_max"]
    n_max = int(st.n_img.max())
    rec = {t: {"outs": torch.empty((L, B, Hq, d), dtype=Kd[0].dtype, device=DEV),
               "sets": torch.zeros((L + 1, B, k_max), dtype=torch.int32, device=DEV),
               "cnts": torch.zeros((L + 1, B), dtype=torch.int32, device=DEV),
               "scores": torch.zeros((wl.num_focal, B, n_max), dtype=torch.float32, device=DEV)}
           for t in sample_steps}
    scratch = torch.empty((B, Hq, d), dtype=Kd[0].dtype, device=DEV)
    focal = None
    t1 = time.time()
    for t in range(T):
        if t == wl.warmup_steps:
            focal = fo.fastocr_profile_warmup(h)
            ratios = fo.fastocr_get_layer_ratios(h)
        r = rec.get(t)
        if r is not None and t >= wl.warmup_steps:
            fo.fastocr_get_selection(h, r["sets"][0], r["cnts"][0])
        for l in range(L):
            out = r["outs"][l] if r is not None else scratch
            fo.fastocr_attend(h, l, Qd[l][t], Kd[l], Vd[l], lens[t], out)
            if r is not None and t >= wl.warmup_steps:
                fo.fastocr_get_selection(h, r["sets"][l + 1], r["cnts"][l + 1])
                if l in focal:
                    fo.fastocr_get_scores(h, r["scores"][focal.index(l)])
        if (t + 1) % 512 == 0:
            torch.cuda.synchronize()
            log(f"[{wl.name}] gpu step {t + 1}/{T} ({time.time() - t1:.1f}s)")
    torch.cuda.synchronize()
    assert fo.fastocr_get_status(h) == 0
    fo.fastocr_destroy(h)
    log(f"[{wl.name}] gpu trajectory {time.time() - t1:.1f}s, focal {focal}")
    host_rec = {t: {k: (v.float().cpu().numpy().astype(np.float64) if k in ("outs",) else v.cpu().numpy())
                    for k, v in r.items()} for t, r in rec.items()}
    return dict(wl=wl, st=st, Kd=Kd, Vd=Vd, Qd=Qd, focal=focal, ratios=ratios, rec=host_rec)


def check_sampled(run, sample_steps, ratio_layers, nonfocal_sample):
    wl, st, rec, focal = run["wl"], run["st"], run["rec"], run["focal"]
    L, B, w = wl.num_layers, wl.batch, wl.warmup_steps
    scale = 1.0 / math.sqrt(wl.head_dim)
    deepest = max(focal)
    unused = unused_picks(focal, L)
    layers = sorted(set(ratio_layers) | set(focal) | set(nonfocal_sample) | {0})
    oracle_ratio = {}
    warm_scores_deepest = []
    worst, jac = 0.0, []
    t0 = time.time()
    for l in layers:
        K, V = _host(run["Kd"][l]), _host(run["Vd"][l])
        # warm-up: image mass (layer ratio) and, at the last warm-up step,
        # the deepest focal layer's scores; step 0 outputs
        if l in ratio_layers:
            masses = []
            for t in range(w):
                q = _host(run["Qd"][l][t])
                lens = st.lens(t)
                for b in range(B):
                    out, p = full_attention(q[b], K[b], V[b], int(lens[b, 1]), scale)
                    masses.append(image_mass(p, int(lens[b, 0])))
                    if t == 0 and 0 in rec:
                        worst = max(worst, check_out(rec[0]["outs"][l, b], out, wl.dtype,
                                                     f"warm-up t=0 l={l} b={b}"))
                    if t == w - 1 and l == deepest:
                        warm_scores_deepest.append(image_scores(p, int(lens[b, 0])))
            oracle_ratio[l] = float(np.mean(np.stack(masses)))
        # sampled pruned steps
        for t in sample_steps:
            if t < w:
                continue
            q = _host(run["Qd"][l][t])
            lens = st.lens(t)
            r = rec[t]
            for b in range(B):
                n, length = int(lens[b, 0]), int(lens[b, 1])
                if l in unused:
                    out, _ = full_attention(q[b], K[b], V[b], length, scale)
                elif l in focal:
                    out, p = full_attention(q[b], K[b], V[b], length, scale)
                    s = image_scores(p, n)
                    check_scores(r["scores"][focal.index(l), b, :n], s, f"scores t={t} l={l} b={b}")
                    c = int(r["cnts"][l + 1, b])
                    jac.append(check_set(r["sets"][l + 1, b, :c], s, kept_count(wl.tau, n),
                                         f"set t={t} l={l} b={b}"))
                elif l in nonfocal_sample:
                    c = int(r["cnts"][l, b])
                    out = sparse_attention(q[b], K[b], V[b], r["sets"][l, b, :c], n, length, scale)
                else:
                    continue
                worst = max(worst, check_out(r["outs"][l, b], out, wl.dtype, f"out t={t} l={l} b={b}"))
        del K, V
        log(f"[{wl.name}] layer {l} checked ({time.time() - t0:.0f}s)")
    # ratios and focal set
    gpu_r = np.asarray(run["ratios"])
    for l, r in oracle_ratio.items():
        assert abs(gpu_r[l] - r) < 1e-5, (l, gpu_r[l], r)
    if set(ratio_layers) == set(range(L)):
        want = [int(x) for x in choose_focal_layers([oracle_ratio[l] for l in range(L)], wl.num_focal)]
        assert focal == want, (focal, want)
    else:
        # sampled: the GPU's focal layers outrank every checked non-focal layer in the oracle too
        lowest_focal = min(oracle_ratio[l] for l in focal)
        for l, r in oracle_ratio.items():
            if l not in focal:
                assert r < lowest_focal, (l, r, lowest_focal)
    # warm start of the first pruned step
    if w in rec:
        for b in range(B):
            n = int(st.n_img[b])
            c = int(rec[w]["cnts"][0, b])
            jac.append(check_set(rec[w]["sets"][0, b, :c], warm_scores_deepest[b], kept_count(wl.tau, n),
                                 f"warm start b={b}"))
    # warm start of step t = set after the deepest focal layer of step t-1
    for t in sample_steps:
        if t - 1 in rec and t - 1 >= w:
            np.testing.assert_array_equal(rec[t]["sets"][0], rec[t - 1]["sets"][deepest + 1])
            np.testing.assert_array_equal(rec[t]["cnts"][0], rec[t - 1]["cnts"][deepest + 1])
    log(f"[{wl.name}] focal {focal}; worst out {worst:.3e}; mean Jaccard vs oracle sets {np.mean(jac):.3f}")


def _samples(wl):
    w, T = wl.warmup_steps, wl.steps
    mid = (w + T) // 2
    return sorted({0, w, w + 1, mid - 1, mid, T - 2, T - 1})


@pytest.mark.timeout(900)
def test_ragged_b16_full_size():
    wl = get_workload("7b-b16-ragged")
    run = run_sampled(wl, _samples(wl), True)
    check_sampled(run, _samples(wl), list(range(wl.num_layers)),
                  nonfocal_sample=[0, 7, 13, 27])


def _ranked_sample(run, extra):
    r = np.asarray(run["ratios"])
    order = list(np.argsort(-r, kind="stable"))
    C = len(run["focal"])
    return sorted(set(order[:C + 3]) | set(extra))


@pytest.mark.timeout(900)
def test_32b_b4_longpage_full_size():
    wl = get_workload("32b-b4-longpage")
    run = run_sampled(wl, _samples(wl), False)
    check_sampled(run, _samples(wl), _ranked_sample(run, [0, 20, 63]),
                  nonfocal_sample=[0, 31, 63])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tau,sigma", [(0.05, None), (0.2, None), (0.02, None), (0.1, None), (1.0, None),
                                       (0.05, 0.25), (0.05, 1.0)])
def test_72b_b8_full_size(tau, sigma):
    # the sweep's tau values (tau = 1: non-focal layers take the full pass)
    # and query-noise levels (sigma None: the default 0.5 and its seed)
    wl = get_workload("72b-b8-sweep", tau=tau) if sigma is None else \
        get_workload("72b-b8-sweep", tau=tau, sigma=sigma)
    run = run_sampled(wl, _samples(wl), False)
    check_sampled(run, _samples(wl), _ranked_sample(run, [0, 30, 79]),
                  nonfocal_sample=[0, 39, 79])
