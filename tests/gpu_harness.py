"""Shared GPU-test machinery: upload a synthetic workload, drive the library
through decode steps with recording, and check the records against the CPU
oracle (conditioned on the GPU's own kept sets where the method allows
several correct answers)."""

from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import dynamic_kv_cache_amd as fo
from oracle import (DecodeOracle, full_attention, image_scores, kept_count, select_top,
                    sparse_attention)
from workload import Generator, Workload, make_structure

# Output tolerances: fp32 inputs -> 1e-5 max-abs; bf16 inputs with fp32
# accumulation -> 2e-2 max-abs and 1e-2 relative L2.
TOL = {"f32": (1e-5, None), "bf16": (2e-2, 1e-2)}
# Kept sets may differ from the oracle's only on tokens whose oracle score is
# within this relative distance of the k-th largest oracle score.
SET_BAND = 1e-3


def unused_picks(focal, num_layers) -> set:
    """Focal layers whose pick the next (focal) layer replaces before any
    layer uses it: the library runs only their full attention (unless
    FASTOCR_SKIP_DEAD_PICKS=0), so they have outputs but no scores or set."""
    import os
    if os.environ.get("FASTOCR_SKIP_DEAD_PICKS", "1") == "0" or focal is None or len(focal) == 0:
        return set()
    f = set(int(x) for x in focal)
    return {l for l in f if l + 1 < num_layers and l + 1 in f}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Uploaded:
    wl: Workload
    st: object
    kv: List[tuple]  # host float32 (K, V) per layer
    q: List[np.ndarray]  # host float32 [T, B, Hq, d] per layer
    Kd: List[torch.Tensor]
    Vd: List[torch.Tensor]
    Qd: List[torch.Tensor]
    lens: torch.Tensor  # [T, B, 2] int32 device
    io_dtype: torch.dtype
    _kv64: Dict[int, tuple] = field(default_factory=dict)

    def kv64(self, l):
        if l not in self._kv64:
            k, v = self.kv[l]
            self._kv64[l] = (k.astype(np.float64), v.astype(np.float64))
        return self._kv64[l]


def upload(wl: Workload, steps: Optional[int] = None, dev="cuda:0") -> Uploaded:
    t0 = time.time()
    if steps is not None:
        wl = wl.with_overrides(steps=steps)
    st = make_structure(wl)
    gen = Generator(wl, st)
    io = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    kv, q, Kd, Vd, Qd = [], [], [], [], []
    for l in range(wl.num_layers):
        k, v = gen.layer_kv(l)
        ql = gen.layer_queries(l, K=k)
        kv.append((k, v))
        q.append(ql)
        Kd.append(torch.from_numpy(k).to(dev).to(io))
        Vd.append(torch.from_numpy(v).to(dev).to(io))
        Qd.append(torch.from_numpy(ql).to(dev).to(io))
    lens = torch.from_numpy(np.stack([st.lens(t) for t in range(wl.steps)])).to(dev)
    log(f"[upload] {wl.name}: L={wl.num_layers} B={wl.batch} S={st.max_seq_len} T={wl.steps} "
        f"in {time.time() - t0:.1f}s")
    return Uploaded(wl, st, kv, q, Kd, Vd, Qd, lens, io)


def make_config(up: Uploaded, mode="pruned", tau=None, **kw) -> fo.Config:
    wl, st = up.wl, up.st
    args = dict(num_layers=wl.num_layers, num_q_heads=wl.num_q_heads,
                num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, batch=wl.batch,
                max_seq_len=st.max_seq_len, max_img_tokens=int(st.n_img.max()),
                min_img_tokens=int(st.n_img.min()), max_text_tokens=int(st.n_prompt.max()) + wl.steps,
                tau=wl.tau if tau is None else tau,
                num_focal=wl.num_focal, warmup_steps=wl.warmup_steps, dtype=wl.dtype, mode=mode)
    args.update(kw)
    return fo.Config(**args)


@dataclass
class Records:
    focal: Optional[List[int]]
    outs: np.ndarray  # [T, L, B, Hq, d] float64
    sets: Optional[np.ndarray]  # [T, L+1, B, k_max]: before layer 0, after each layer
    cnts: Optional[np.ndarray]  # [T, L+1, B]
    scores: Optional[np.ndarray]  # [T, |C|, B, n_max]
    ratios: Optional[List[float]]
    status: int


def run(up: Uploaded, h: fo.Handle, steps: int, record_sets: bool = True) -> Records:
    wl = up.wl
    L, B, Hq, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim
    dev = up.Kd[0].device
    pruned = h.cfg.mode == "pruned"
    info = fo.fastocr_get_info(h)
    k_max = info["k_max"]
    n_max = h.cfg.max_img_tokens
    outs = torch.empty((steps, L, B, Hq, d), dtype=up.io_dtype, device=dev)
    sets = cnts = scores = None
    if pruned and record_sets:
        sets = torch.zeros((steps, L + 1, B, k_max), dtype=torch.int32, device=dev)
        cnts = torch.zeros((steps, L + 1, B), dtype=torch.int32, device=dev)
        scores = torch.zeros((steps, wl.num_focal, B, n_max), dtype=torch.float32, device=dev)
    focal = None
    ratios = None
    t0 = time.time()
    for t in range(steps):
        if pruned and t == wl.warmup_steps:
            focal = fo.fastocr_profile_warmup(h)
            ratios = fo.fastocr_get_layer_ratios(h)
        rec = pruned and record_sets and t >= wl.warmup_steps
        if rec:
            fo.fastocr_get_selection(h, sets[t, 0], cnts[t, 0])
        for l in range(L):
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], outs[t, l])
            if rec:
                fo.fastocr_get_selection(h, sets[t, l + 1], cnts[t, l + 1])
                if l in focal:
                    fo.fastocr_get_scores(h, scores[t, focal.index(l)])
        if (t + 1) % 256 == 0:
            torch.cuda.synchronize()
            log(f"[gpu] step {t + 1}/{steps} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    status = fo.fastocr_get_status(h)
    r = Records(focal=focal, outs=outs.float().cpu().numpy().astype(np.float64),
                sets=None if sets is None else sets.cpu().numpy(),
                cnts=None if cnts is None else cnts.cpu().numpy(),
                scores=None if scores is None else scores.cpu().numpy(),
                ratios=ratios, status=status)
    log(f"[gpu] ran {steps} steps in {time.time() - t0:.1f}s, status {status}")
    return r


def check_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str) -> float:
    max_abs_tol, rel_tol = TOL[dtype]
    err = float(np.abs(got - want).max()) if got.size else 0.0
    assert err <= max_abs_tol, f"{what}: max abs error {err:.3e} > {max_abs_tol}"
    if rel_tol is not None and got.size:
        rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
        assert rel <= rel_tol, f"{what}: relative L2 error {rel:.3e} > {rel_tol}"
    return err


def check_set(gpu: np.ndarray, s_oracle: np.ndarray, k: int, what: str) -> float:
    """Band rule; returns the Jaccard overlap with the oracle's own set."""
    assert len(gpu) == k, f"{what}: count {len(gpu)} != {k}"
    if k == 0:
        return 1.0
    assert np.all(np.diff(gpu) > 0), f"{what}: not strictly ascending"
    assert gpu[0] >= 0 and gpu[-1] < len(s_oracle), f"{what}: index out of range"
    ours = select_top(s_oracle, k)
    theta = np.sort(s_oracle)[::-1][k - 1]
    diff = set(int(j) for j in gpu) ^ set(int(j) for j in ours)
    for j in diff:
        assert abs(s_oracle[j] - theta) <= SET_BAND * theta, (
            f"{what}: token {j} (score {s_oracle[j]:.9g}) differs from the oracle set, "
            f"threshold {theta:.9g}")
    inter = len(set(int(j) for j in gpu) & set(int(j) for j in ours))
    return inter / (2 * k - inter)


def check_scores(got: np.ndarray, want: np.ndarray, what: str) -> None:
    top = float(want.max()) if want.size else 0.0
    err = np.abs(got - want)
    bad = err > (1e-4 * np.abs(want) + 1e-6 * top)
    assert not bad.any(), f"{what}: {int(bad.sum())} scores off, worst {float(err.max()):.3e}"


class Checker:
    """Replays the method on the CPU next to the GPU records."""

    def __init__(self, up: Uploaded, rec: Records, tau: Optional[float] = None, spans=None,
                 scale: Optional[float] = None):
        """spans: per sequence (start, count) of its image pages in up's
        (host) cache layout; the GPU ran on the image-first permuted cache."""
        self.up, self.rec = up, rec
        wl = up.wl
        self.tau = wl.tau if tau is None else tau
        self.scale = 1.0 / math.sqrt(wl.head_dim) if scale is None else scale
        self.oracle = DecodeOracle(num_layers=wl.num_layers, num_q_heads=wl.num_q_heads,
                                   num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, tau=self.tau,
                                   num_focal=wl.num_focal, warmup_steps=wl.warmup_steps, spans=spans,
                                   scale=scale)
        self.rows = (lambda b: None) if spans is None else (lambda b: self.oracle.image_rows[b])
        self.jaccard: List[float] = []
        self.worst_out = 0.0

    def q(self, l, t):
        return self.up.q[l][t].astype(np.float64)

    def warmup(self) -> None:
        """Run the oracle's warm-up, compare every warm-up output and C."""
        wl, up = self.up.wl, self.up
        for t in range(wl.warmup_steps):
            r = self.oracle.step(t, lambda l: self.q(l, t), up.kv64, up.st.lens(t))
            for l in range(wl.num_layers):
                self.worst_out = max(self.worst_out, check_out(
                    self.rec.outs[t, l], r.outs[l], wl.dtype, f"warm-up t={t} l={l}"))
        assert self.rec.focal == [int(x) for x in self.oracle.focal], (
            f"focal layers {self.rec.focal} != oracle {list(self.oracle.focal)}; "
            f"ratios gpu {self.rec.ratios} oracle {list(self.oracle.ratios)}")
        np.testing.assert_allclose(self.rec.ratios, self.oracle.ratios, rtol=0, atol=1e-5)
        # warm start of the first pruned step
        t = wl.warmup_steps
        if self.rec.sets is not None and t < self.rec.outs.shape[0]:
            deepest = int(self.oracle.focal.max())
            for b in range(wl.batch):
                n = int(up.st.n_img[b])
                c = int(self.rec.cnts[t, 0, b])
                self.jaccard.append(check_set(self.rec.sets[t, 0, b, :c],
                                              self.oracle.warm_scores[deepest][b],
                                              kept_count(self.tau, n), f"warm start b={b}"))

    def pruned_step(self, t: int) -> None:
        wl, up, rec = self.up.wl, self.up, self.rec
        lens = up.st.lens(t)
        focal = rec.focal
        unused = unused_picks(focal, wl.num_layers)
        for l in range(wl.num_layers):
            K, V = up.kv64(l)
            ql = self.q(l, t)
            for b in range(wl.batch):
                n, length = int(lens[b, 0]), int(lens[b, 1])
                if l in unused:
                    out, _ = full_attention(ql[b], K[b], V[b], length, self.scale)
                elif l in focal:
                    out, p = full_attention(ql[b], K[b], V[b], length, self.scale)
                    s = image_scores(p, n, self.rows(b))
                    slot = focal.index(l)
                    check_scores(rec.scores[t, slot, b, :n], s, f"scores t={t} l={l} b={b}")
                    c = int(rec.cnts[t, l + 1, b])
                    self.jaccard.append(check_set(rec.sets[t, l + 1, b, :c], s,
                                                  kept_count(self.tau, n), f"set t={t} l={l} b={b}"))
                else:
                    c = int(rec.cnts[t, l, b])
                    used = rec.sets[t, l, b, :c]
                    out = sparse_attention(ql[b], K[b], V[b], used, n, length, self.scale, self.rows(b))
                self.worst_out = max(self.worst_out, check_out(
                    rec.outs[t, l, b], out, wl.dtype, f"out t={t} l={l} b={b}"))
        # the warm start of step t+1 is the set after the deepest focal layer
        if t + 1 < rec.outs.shape[0]:
            deepest = max(focal)
            np.testing.assert_array_equal(rec.sets[t + 1, 0], rec.sets[t, deepest + 1])
            np.testing.assert_array_equal(rec.cnts[t + 1, 0], rec.cnts[t, deepest + 1])


def check_layer(up: Uploaded, t: int, l: int, out: np.ndarray, kind: str, tau: Optional[float] = None,
                used=None, picked=None, what: str = "") -> float:
    """One layer's output at step t against the oracle.

    kind: "full" (warm-up, FULL mode, or a focal layer whose pick is unused:
    full attention), "focal" (full attention; ``picked`` = (idx [B, k_max],
    cnt [B]) is the kept set after the layer, checked by the band rule
    against the oracle's scores) or "sparse" (attention over ``used`` =
    (idx, cnt), the set the GPU attended with, plus every text row).
    Returns the largest output error."""
    wl = up.wl
    tau = wl.tau if tau is None else tau
    scale = 1.0 / math.sqrt(wl.head_dim)
    lens = up.st.lens(t)
    K, V = up.kv64(l)
    q = up.q[l][t].astype(np.float64)
    worst = 0.0
    for b in range(wl.batch):
        n, length = int(lens[b, 0]), int(lens[b, 1])
        if kind in ("full", "focal"):
            want, p = full_attention(q[b], K[b], V[b], length, scale)
            if kind == "focal":
                idx, cnt = picked
                check_set(idx[b, :int(cnt[b])], image_scores(p, n), kept_count(tau, n),
                          f"{what} set t={t} l={l} b={b}")
        else:
            idx, cnt = used
            want = sparse_attention(q[b], K[b], V[b], idx[b, :int(cnt[b])], n, length, scale)
        worst = max(worst, check_out(out[b], want, wl.dtype, f"{what} out t={t} l={l} b={b}"))
    return worst
