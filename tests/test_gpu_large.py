"""GPU parity at the full sizes of the large workloads, on sampled steps.

The library runs every decode step of the real shape (the same handle
configuration and launch geometry the benchmark times); the oracle checks
sampled steps one by one, reading the exact device inputs back layer by
layer:
* every layer's warm-up image-attention ratio, so the focal set is checked
  exactly (Focal Layer Selection).  Only q.K and the softmax enter a ratio,
  and tau never enters the inputs, so the ratios of one input set (workload
  and seed) are computed once and shared by the tests that use it;
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
from oracle import (attention_probs, choose_focal_layers, full_attention, image_mass, image_scores,
                    kept_count, select_top, sparse_attention)
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


def run_sampled(wl, sample_steps):
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


# oracle image-attention ratio of every layer per input set (workload name,
# seed, query noise): tau does not enter the inputs, so the tests of a tau
# sweep share them
_RATIOS = {}


def oracle_ratios(run):
    """Mean warm-up image mass of every layer (over steps, sequences and
    heads), from the keys and queries the GPU consumed."""
    wl, st = run["wl"], run["st"]
    key = (wl.name, wl.seed, wl.sigma)
    if key in _RATIOS:
        return _RATIOS[key]
    L, B, w = wl.num_layers, wl.batch, wl.warmup_steps
    scale = 1.0 / math.sqrt(wl.head_dim)
    rows = int(max(st.lens(t)[:, 1].max() for t in range(w)))
    t0 = time.time()
    ratios = []
    for l in range(L):
        K = run["Kd"][l][:, :, :rows].float().cpu().numpy().astype(np.float64)
        masses = []
        for t in range(w):
            q = _host(run["Qd"][l][t])
            lens = st.lens(t)
            for b in range(B):
                p = attention_probs(q[b], K[b], slice(0, int(lens[b, 1])), scale)
                masses.append(image_mass(p, int(lens[b, 0])))
        ratios.append(float(np.mean(np.stack(masses))))
        del K
        if (l + 1) % 16 == 0:
            log(f"[{wl.name}] oracle ratios of {l + 1}/{L} layers ({time.time() - t0:.0f}s)")
    _RATIOS[key] = ratios
    return ratios


def check_focal_set(run):
    """C exact: the GPU's focal layers are the oracle's, picked from every
    layer's ratio; the ratios agree to 1e-5."""
    wl, focal = run["wl"], run["focal"]
    want_r = np.asarray(oracle_ratios(run))
    gpu_r = np.asarray(run["ratios"])
    worst = float(np.abs(gpu_r - want_r).max())
    assert worst < 1e-5, (int(np.argmax(np.abs(gpu_r - want_r))), worst)
    want = [int(x) for x in choose_focal_layers(want_r, wl.num_focal)]
    assert focal == want, (focal, want)
    ranked = np.sort(want_r)[::-1]
    C = wl.num_focal
    margin = ranked[C - 1] - ranked[C] if C < wl.num_layers else float("inf")
    log(f"[{wl.name}] C {focal} exact over all {wl.num_layers} layers; ratio margin between the |C|-th and "
        f"(|C|+1)-th layer {margin:.3e} ({margin / ranked[C - 1]:.2e} relative); worst ratio error {worst:.1e}")


def check_sampled(run, sample_steps, nonfocal_sample, warmup_out_layers):
    wl, st, rec, focal = run["wl"], run["st"], run["rec"], run["focal"]
    L, B, w = wl.num_layers, wl.batch, wl.warmup_steps
    scale = 1.0 / math.sqrt(wl.head_dim)
    deepest = max(focal)
    unused = unused_picks(focal, L)
    check_focal_set(run)
    layers = sorted(set(focal) | set(nonfocal_sample) | set(warmup_out_layers))
    warm_scores_deepest = []
    worst, jac = 0.0, []
    t0 = time.time()
    for l in layers:
        K, V = _host(run["Kd"][l]), _host(run["Vd"][l])
        # warm-up: step 0 outputs, and the deepest focal layer's scores at the
        # last warm-up step (they seed the first pruned step's kept set)
        for t in ([0] if l in warmup_out_layers and 0 in rec else []) + ([w - 1] if l == deepest else []):
            q = _host(run["Qd"][l][t])
            lens = st.lens(t)
            for b in range(B):
                out, p = full_attention(q[b], K[b], V[b], int(lens[b, 1]), scale)
                if t == 0:
                    worst = max(worst, check_out(rec[0]["outs"][l, b], out, wl.dtype, f"warm-up t=0 l={l} b={b}"))
                if t == w - 1:
                    warm_scores_deepest.append(image_scores(p, int(lens[b, 0])))
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
    run = run_sampled(wl, _samples(wl))
    check_sampled(run, _samples(wl), nonfocal_sample=[0, 7, 13, 27], warmup_out_layers=[0, 13, 27])


@pytest.mark.timeout(900)
def test_32b_b4_longpage_full_size():
    wl = get_workload("32b-b4-longpage")
    run = run_sampled(wl, _samples(wl))
    check_sampled(run, _samples(wl), nonfocal_sample=[0, 31, 63], warmup_out_layers=[0, 20, 63])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tau,sigma", [(0.05, None), (0.2, None), (0.02, None), (0.1, None), (1.0, None),
                                       (0.05, 0.25), (0.05, 1.0)])
def test_72b_b8_full_size(tau, sigma):
    # the sweep's tau values (tau = 1: non-focal layers take the full pass)
    # and query-noise levels (sigma None: the default 0.5 and its seed)
    wl = get_workload("72b-b8-sweep", tau=tau) if sigma is None else \
        get_workload("72b-b8-sweep", tau=tau, sigma=sigma)
    run = run_sampled(wl, _samples(wl))
    check_sampled(run, _samples(wl), nonfocal_sample=[0, 39, 79], warmup_out_layers=[0, 30, 79])
