"""GPU parity of the HIP library against the CPU oracle (through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import dynamic_kv_cache_amd as fo
from oracle import full_attention, kept_count, select_top, sparse_attention
from workload import get_workload

from gpu_harness import (Checker, check_layer, check_out, check_set, log, make_config, run, unused_picks,
                         upload)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------------------
# single-kernel checks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name,steps,valu", [("tiny-fp32", 6, False), ("7b-b1", 3, False),
                                             ("7b-b1", 3, True)])
def test_full_mode_matches_oracle(monkeypatch, name, steps, valu):
    # valu: the full split without MFMA (a measurement override)
    monkeypatch.setenv("FASTOCR_VALU_FULL", "1" if valu else "0")
    up = upload(get_workload(name), steps=steps)
    h = fo.fastocr_create(make_config(up, mode="full"))
    rec = run(up, h, steps)
    assert rec.status == 0
    scale = 1 / math.sqrt(up.wl.head_dim)
    worst = 0.0
    for t in range(steps):
        lens = up.st.lens(t)
        for l in range(up.wl.num_layers):
            K, V = up.kv64(l)
            for b in range(up.wl.batch):
                out, _ = full_attention(up.q[l][t][b].astype(np.float64), K[b], V[b],
                                        int(lens[b, 1]), scale)
                worst = max(worst, check_out(rec.outs[t, l, b], out, up.wl.dtype, f"t={t} l={l}"))
    log(f"[full] {name}: worst max-abs {worst:.3e}")


def _topk_case(rng, B, n_cap, tau):
    scores = np.zeros((B, n_cap), dtype=np.float32)
    ns = []
    for b in range(B):
        n = [0, 1, 7, n_cap, n_cap // 3, 1000, 64, 65][b % 8]
        n = min(n, n_cap)
        ns.append(n)
        kind = b % 5
        if kind == 0:  # continuous
            scores[b, :n] = rng.random(n).astype(np.float32) * 3
        elif kind == 1:  # heavy ties
            scores[b, :n] = (rng.integers(0, 5, n) / 4).astype(np.float32)
        elif kind == 2:  # all equal, zeros mixed in
            scores[b, :n] = np.float32(0.25)
            scores[b, : n // 2] = 0.0
        elif kind == 3:  # one narrow band: the leading digits do not separate the keys
            scores[b, :n] = (1.0 + rng.random(n) * 1e-4).astype(np.float32)
        else:  # head-summed softmax-like: a few large scores, a long tail
            scores[b, :n] = (rng.exponential(1.0, n) ** 3 / max(n, 1)).astype(np.float32)
    lens = np.stack([np.array(ns), np.array(ns) + 3], axis=1).astype(np.int32)
    return scores, lens


@pytest.mark.parametrize("tau", [0.02, 0.05, 0.1, 0.5, 1.0])
# row capacities for every keys-per-thread specialisation of the kernel:
# 1, 2, 4, 8, 16 in registers, and re-read from memory
@pytest.mark.parametrize("n_cap", [64, 2000, 4000, 6400, 16384, 70000])
def test_topk_bit_exact(tau, n_cap):
    rng = np.random.default_rng(int(tau * 1000) + n_cap)
    B = 10
    scores, lens = _topk_case(rng, B, n_cap, tau)
    k_stride = max(kept_count(tau, n_cap), 1)
    s_d = torch.from_numpy(scores).to(DEV)
    l_d = torch.from_numpy(lens).to(DEV)
    idx = torch.full((B, k_stride), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    fo.fastocr_select_topk(s_d, l_d, tau, idx, cnt)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        n = int(lens[b, 0])
        k = kept_count(tau, n)
        assert cnt[b] == k
        want = select_top(scores[b, :n].astype(np.float64), k)
        np.testing.assert_array_equal(idx[b, :k], want, err_msg=f"b={b} n={n} k={k}")


# kept-token pass variants (environment, expected plan): each pair's tiles
# dealt round-robin to the workgroups that fill one wave, merged by the merge
# kernel, rows loaded non-temporally, with the focal passes staging their
# logits in LDS; a few workgroups per pair (several rounds each), plain row
# loads, the focal passes storing their logits as they are computed; one
# workgroup per pair (no merge).  With batches of 4 (16 pairs) and 5 or 1
# (pair grids padded to a multiple of 8) every kept-token kernel form runs.
KEPT_VARIANTS = {
    "kept": ({"FASTOCR_FOCAL_STAGE": "1", "FASTOCR_STREAM_ROWS": "1"},
             dict(sparse_direct=0, focal_staged=1, stream_rows=1)),
    "kept-few-splits": ({"FASTOCR_SPARSE_ROWS": "1024", "FASTOCR_FOCAL_STAGE": "0", "FASTOCR_STREAM_ROWS": "0"},
                        dict(focal_staged=0, stream_rows=0)),
    "direct": ({"FASTOCR_SPARSE_ROWS": "16384"}, dict(sparse_direct=1)),
}
SPARSE_VARIANTS = pytest.mark.parametrize("rows", list(KEPT_VARIANTS), ids=list(KEPT_VARIANTS))


def _sparse_variant(monkeypatch, rows):
    monkeypatch.delenv("FASTOCR_SPARSE_ROWS", raising=False)
    monkeypatch.delenv("FASTOCR_FOCAL_STAGE", raising=False)
    monkeypatch.delenv("FASTOCR_STREAM_ROWS", raising=False)
    for k, v in KEPT_VARIANTS[rows][0].items():
        monkeypatch.setenv(k, v)


@SPARSE_VARIANTS
@pytest.mark.parametrize("tau", [0.05, 0.5])
def test_sparse_conditioned_on_injected_sets(monkeypatch, rows, tau):
    # tau = 0.5 gives a direct split many rounds
    _sparse_variant(monkeypatch, rows)
    up = upload(get_workload("7b-b1").with_overrides(num_layers=3, warmup_steps=1, num_focal=1, tau=tau),
                steps=3)
    h = fo.fastocr_create(make_config(up))
    info = fo.fastocr_get_info(h)
    for key, value in KEPT_VARIANTS[rows][1].items():
        assert info[key] == value, (rows, key, info)
    _check_injected_sets(up, h)


def _check_injected_sets(up, h):
    # one warm-up step, then layer 2 made the focal layer and two kept sets
    # injected in turn (a full one and one of 17 tokens): layers 0 and 1
    # attend with them, checked against the oracle's kept-token attention
    wl = up.wl
    for l in range(wl.num_layers):  # one warm-up step
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=up.io_dtype, device=DEV)
        fo.fastocr_attend(h, l, up.Qd[l][0], up.Kd[l], up.Vd[l], up.lens[0], out)
    fo.fastocr_set_focal_layers(h, [2])
    k_max = fo.fastocr_get_info(h)["k_max"]
    rng = np.random.default_rng(5)
    n = int(up.st.n_img[0])
    scale = 1 / math.sqrt(wl.head_dim)
    for t, k in [(1, k_max), (2, 17)]:
        sel = np.zeros((1, k_max), dtype=np.int32)
        chosen = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
        sel[0, :k] = chosen
        fo.fastocr_set_selection(h, torch.from_numpy(sel).to(DEV),
                                 torch.tensor([k], dtype=torch.int32, device=DEV))
        outs = []
        for l in range(wl.num_layers):
            out = torch.empty((1, wl.num_q_heads, wl.head_dim), dtype=up.io_dtype, device=DEV)
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out)
            outs.append(out)
        torch.cuda.synchronize()
        length = int(up.st.lens(t)[0, 1])
        for l in range(2):  # layers before the focal layer use the injected set
            K, V = up.kv64(l)
            want = sparse_attention(up.q[l][t][0].astype(np.float64), K[0], V[0], chosen, n, length,
                                    scale)
            check_out(outs[l].float().cpu().numpy()[0], want, wl.dtype, f"sparse t={t} l={l}")
    assert fo.fastocr_get_status(h) == 0


# The merges are instantiated per count of state slots a thread uses,
# ceil(states / lanes per output column) (8 lanes at head_dim 128, 16 at
# 64), and the general merge has its own path past 64 states: every count
# is forced through a rows-per-split override, found from the host-side
# launch plan for this device, and checked against the oracle.


def _rows_for_slots(monkeypatch, cfg, env, key, lanes, nv, step):
    # the largest override (a multiple of `step` rows) whose plan gives nv
    # slots per thread (nv = 0: more than 64 states), with more than one state
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in range(8192, 0, -step):
        monkeypatch.setenv(env, str(rows))
        n = fo.fastocr_plan_launch(cfg, ncu)[key]
        if n > 1 and (0 if n > 64 else -(-n // lanes)) == nv:
            return rows, n
    pytest.fail(f"no {env} gives {nv} slots")


GENERAL_MERGE_CASES = [(128, nv) for nv in range(9)] + [(64, nv) for nv in range(5)]


@pytest.mark.parametrize("d,nv", GENERAL_MERGE_CASES,
                         ids=[f"d{d}-slots{nv if nv else 'over64'}" for d, nv in GENERAL_MERGE_CASES])
def test_general_merge_slot_counts(monkeypatch, d, nv):
    up = upload(get_workload("7b-b1").with_overrides(num_layers=2, head_dim=d), steps=2)
    cfg = make_config(up, mode="full")
    rows, splits = _rows_for_slots(monkeypatch, cfg, "FASTOCR_FULL_ROWS", "full_max_splits",
                                   8 if d == 128 else 16, nv, 16)
    h = fo.fastocr_create(cfg)
    assert fo.fastocr_get_info(h)["full_max_splits"] == splits
    rec = run(up, h, 2)
    assert rec.status == 0
    scale = 1 / math.sqrt(d)
    for t in range(2):
        length = int(up.st.lens(t)[0, 1])
        for l in range(2):
            K, V = up.kv64(l)
            want, _ = full_attention(up.q[l][t][0].astype(np.float64), K[0], V[0], length, scale)
            check_out(rec.outs[t, l, 0], want, up.wl.dtype, f"{splits} splits of {rows} t={t} l={l}")


# a kept-token pass has at most 32 workgroups per pair: slots 1..4 at
# head_dim 128, 1..2 at 64
KEPT_MERGE_CASES = [(128, nv) for nv in range(1, 5)] + [(64, nv) for nv in range(1, 3)]


@pytest.mark.parametrize("d,nv", KEPT_MERGE_CASES, ids=[f"d{d}-slots{nv}" for d, nv in KEPT_MERGE_CASES])
def test_kept_merge_slot_counts(monkeypatch, d, nv):
    up = upload(get_workload("7b-b1").with_overrides(num_layers=3, warmup_steps=1, num_focal=1, head_dim=d),
                steps=3)
    cfg = make_config(up)
    _, P = _rows_for_slots(monkeypatch, cfg, "FASTOCR_SPARSE_ROWS", "sparse_max_splits",
                           8 if d == 128 else 16, nv, 1)
    h = fo.fastocr_create(cfg)
    assert fo.fastocr_get_info(h)["sparse_max_splits"] == P
    _check_injected_sets(up, h)


@SPARSE_VARIANTS
def test_tau_one_sparse_equals_full(monkeypatch, rows):
    # the kept-token kernels themselves (by default tau = 1 runs the full pass)
    _sparse_variant(monkeypatch, rows)
    monkeypatch.setenv("FASTOCR_KEPT_ALL_AS_FULL", "0")
    wl = get_workload("tiny-fp32").with_overrides(tau=1.0)
    up = upload(wl, steps=7)
    rec = run(up, fo.fastocr_create(make_config(up)), 7)
    full = run(up, fo.fastocr_create(make_config(up, mode="full")), 7)
    np.testing.assert_allclose(rec.outs, full.outs, rtol=0, atol=1e-5)


def test_tau_one_non_focal_layers_take_full_pass(monkeypatch):
    # tau = 1 keeps every image token, so non-focal layers run the full pass;
    # the focal layers still select (every index, ascending)
    monkeypatch.delenv("FASTOCR_KEPT_ALL_AS_FULL", raising=False)
    wl = get_workload("tiny-fp32").with_overrides(tau=1.0)
    up = upload(wl, steps=7)
    rec = run(up, fo.fastocr_create(make_config(up)), 7)
    full = run(up, fo.fastocr_create(make_config(up, mode="full")), 7)
    np.testing.assert_allclose(rec.outs, full.outs, rtol=0, atol=1e-5)
    assert rec.status == 0
    n = int(up.st.n_img[0])
    for t in range(wl.warmup_steps, 7):
        for l in rec.focal:
            assert rec.cnts[t, l + 1, 0] == n
            np.testing.assert_array_equal(rec.sets[t, l + 1, 0, :n], np.arange(n))


def test_lens_out_of_range_sets_flag():
    up = upload(get_workload("tiny-fp32"), steps=1)
    h = fo.fastocr_create(make_config(up, mode="full"))
    bad = up.lens[0].clone()
    bad[0, 1] = up.st.max_seq_len + 5
    out = torch.empty((1, up.wl.num_q_heads, up.wl.head_dim), dtype=up.io_dtype, device=DEV)
    fo.fastocr_attend(h, 0, up.Qd[0][0], up.Kd[0], up.Vd[0], bad, out)
    assert fo.fastocr_get_status(h) & fo.FLAG_LENS_CLAMPED


def test_text_beyond_declared_bound(monkeypatch):
    # max_text_tokens = 1 declares at most one text row; the sequence has 66.
    # The kept-token kernel deals whatever rows a pair has to its workgroups,
    # so every row is still attended: no flag, the oracle's output
    monkeypatch.delenv("FASTOCR_SPARSE_ROWS", raising=False)
    up = upload(get_workload("7b-b1").with_overrides(num_layers=2, warmup_steps=1, num_focal=1), steps=2)
    h = fo.fastocr_create(make_config(up, max_text_tokens=1))
    wl = up.wl
    out = torch.empty((1, wl.num_q_heads, wl.head_dim), dtype=up.io_dtype, device=DEV)
    for l in range(wl.num_layers):
        fo.fastocr_attend(h, l, up.Qd[l][0], up.Kd[l], up.Vd[l], up.lens[0], out)
    fo.fastocr_profile_warmup(h)
    assert fo.fastocr_get_status(h) == 0
    fo.fastocr_set_focal_layers(h, [1])
    k_max = fo.fastocr_get_info(h)["k_max"]
    sel = torch.zeros((1, k_max), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((1,), dtype=torch.int32, device=DEV)
    fo.fastocr_attend(h, 0, up.Qd[0][1], up.Kd[0], up.Vd[0], up.lens[1], out)  # non-focal
    fo.fastocr_get_selection(h, sel, cnt)
    torch.cuda.synchronize()
    assert fo.fastocr_get_status(h) == 0
    check_layer(up, 1, 0, out.float().cpu().numpy().astype(np.float64), "sparse",
                used=(sel.cpu().numpy(), cnt.cpu().numpy()), what="undeclared text")


def test_state_machine_errors():
    up = upload(get_workload("tiny-fp32"), steps=5)
    wl = up.wl
    h = fo.fastocr_create(make_config(up))
    out = torch.empty((1, wl.num_q_heads, wl.head_dim), dtype=up.io_dtype, device=DEV)
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_attend(h, 1, up.Qd[1][0], up.Kd[1], up.Vd[1], up.lens[0], out)
    assert e.value.code == fo.ERR_STATE
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_profile_warmup(h)
    assert e.value.code == fo.ERR_STATE
    for t in range(wl.warmup_steps):
        for l in range(wl.num_layers):
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out)
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_attend(h, 0, up.Qd[0][4], up.Kd[0], up.Vd[0], up.lens[4], out)
    assert e.value.code == fo.ERR_STATE
    assert len(fo.fastocr_profile_warmup(h)) == wl.num_focal
    fo.fastocr_attend(h, 0, up.Qd[0][4], up.Kd[0], up.Vd[0], up.lens[4], out)
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_attend(h, 0, up.Qd[0][4], up.Kd[0], up.Vd[0], up.lens[4], out)
    assert e.value.code == fo.ERR_STATE


# ---------------------------------------------------------------------------
# whole decode trajectories
# ---------------------------------------------------------------------------


def test_trajectory_tiny_all_steps():
    wl = get_workload("tiny-fp32")
    up = upload(wl)
    rec = run(up, fo.fastocr_create(make_config(up)), wl.steps)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, wl.steps):
        chk.pruned_step(t)
    log(f"[tiny] focal {rec.focal}, worst out {chk.worst_out:.2e}, "
        f"mean Jaccard {np.mean(chk.jaccard):.3f}")


@SPARSE_VARIANTS
def test_trajectory_ragged_small(monkeypatch, rows):
    _sparse_variant(monkeypatch, rows)
    wl = get_workload("7b-b16-ragged").with_overrides(
        batch=4, num_layers=6, focal_band=(2, 3), num_focal=2, warmup_steps=3,
        n_img_range=(100, 700), n_prompt=(5, 40))
    up = upload(wl, steps=12)
    rec = run(up, fo.fastocr_create(make_config(up)), 12)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, 12):
        chk.pruned_step(t)
    log(f"[ragged] n={up.st.n_img.tolist()} focal {rec.focal}, worst out {chk.worst_out:.2e}")


@SPARSE_VARIANTS
def test_trajectory_tiny_images(monkeypatch, rows):
    # sequences with 1-40 image tokens (k = 1 or 2) beside longer prompts:
    # kept-token passes that are mostly text, empty high splits
    _sparse_variant(monkeypatch, rows)
    wl = get_workload("7b-b16-ragged").with_overrides(
        batch=5, num_layers=4, focal_band=(1, 2), num_focal=1, warmup_steps=2,
        n_img_range=(1, 40), n_prompt=(1, 90))
    up = upload(wl, steps=7)
    rec = run(up, fo.fastocr_create(make_config(up)), 7)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, 7):
        chk.pruned_step(t)
    log(f"[tiny images] n={up.st.n_img.tolist()} focal {rec.focal}, worst out {chk.worst_out:.2e}")


@pytest.mark.parametrize("stream", ["0", "1"], ids=["plain-rows", "streamed-rows"])
@pytest.mark.parametrize("name,dtype,head_dim,steps", [
    ("tiny-fp32", "bf16", 64, None),    # bf16 kernels at d = 64
    ("tiny-fp32", "f32", 128, None),    # fp32 kernels at d = 128
    ("tiny-fp32", "f32", 64, None),     # fp32 kernels at d = 64
    ("7b-b1", "bf16", 64, 10),          # several splits per sequence at d = 64
])
def test_trajectory_other_dtype_and_head_dim(monkeypatch, name, dtype, head_dim, steps, stream):
    # every kept-token kernel form: both dtypes and head sizes, plain and
    # non-temporal row loads
    monkeypatch.setenv("FASTOCR_STREAM_ROWS", stream)
    wl = get_workload(name).with_overrides(dtype=dtype, head_dim=head_dim)
    if name == "7b-b1":
        wl = wl.with_overrides(num_layers=4, focal_band=(1, 2), num_focal=2, warmup_steps=2)
    up = upload(wl, steps=steps)
    T = up.wl.steps
    h = fo.fastocr_create(make_config(up))
    assert fo.fastocr_get_info(h)["stream_rows"] == int(stream)
    rec = run(up, h, T)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, T):
        chk.pruned_step(t)
    log(f"[{name} {dtype} d={head_dim} stream {stream}] focal {rec.focal}, worst out {chk.worst_out:.2e}")


def test_trajectory_layer0_focal():
    # Layer 0 is forced focal: the warm start is never used for attention.
    wl = get_workload("tiny-fp32").with_overrides(planted_layers=(0, 2))
    up = upload(wl)
    rec = run(up, fo.fastocr_create(make_config(up)), wl.steps)
    chk = Checker(up, rec)
    chk.warmup()
    assert rec.focal[0] == 0
    for t in range(wl.warmup_steps, wl.steps):
        chk.pruned_step(t)


def test_deterministic_replay():
    wl = get_workload("7b-b1").with_overrides(num_layers=6, focal_band=(2, 3), num_focal=2,
                                             warmup_steps=2)
    up = upload(wl, steps=10)
    a = run(up, fo.fastocr_create(make_config(up)), 10)
    b = run(up, fo.fastocr_create(make_config(up)), 10)
    np.testing.assert_array_equal(a.outs, b.outs)
    np.testing.assert_array_equal(a.sets, b.sets)
    np.testing.assert_array_equal(a.scores, b.scores)
    assert a.focal == b.focal and a.ratios == b.ratios


@pytest.fixture(scope="module")
def traj_7b():
    wl = get_workload("7b-b1")
    up = upload(wl)
    rec = run(up, fo.fastocr_create(make_config(up)), wl.steps)
    chk = Checker(up, rec)
    chk.warmup()
    log(f"[7b] focal {rec.focal} ratios {np.round(rec.ratios, 6).tolist()}")
    return up, rec, chk


@pytest.mark.parametrize("chunk", range(4))
def test_trajectory_7b_all_steps(traj_7b, chunk):
    up, rec, chk = traj_7b
    assert rec.status == 0
    w, T = up.wl.warmup_steps, up.wl.steps
    edges = np.linspace(w, T, 5).astype(int)
    for t in range(edges[chunk], edges[chunk + 1]):
        chk.pruned_step(t)
    log(f"[7b] steps {edges[chunk]}..{edges[chunk + 1] - 1} ok; worst out {chk.worst_out:.3e}, "
        f"mean Jaccard {np.mean(chk.jaccard):.3f}")


APPEND_CASES = {
    "tiny-full": ("tiny-fp32", dict(), "full", 6, {}),
    "tiny-pruned": ("tiny-fp32", dict(), "pruned", 7, {}),
    "7b-pruned": ("7b-b1", dict(num_layers=3, warmup_steps=1, num_focal=1), "pruned", 4, {}),
    "ragged-few-splits": ("7b-b16-ragged", dict(batch=4, num_layers=4, focal_band=(1, 2), num_focal=1,
                                                warmup_steps=2, n_img_range=(100, 700), n_prompt=(5, 40)),
                          "pruned", 5, {"FASTOCR_SPARSE_ROWS": "384"}),
    "ragged-direct": ("7b-b16-ragged", dict(batch=2, num_layers=4, focal_band=(1, 2), num_focal=1,
                                            warmup_steps=2, n_img_range=(100, 700), n_prompt=(5, 40)),
                      "pruned", 5, {"FASTOCR_SPARSE_ROWS": "16384"}),
}


@pytest.mark.parametrize("case", list(APPEND_CASES))
def test_attend_append_equals_prewritten_row(monkeypatch, case):
    # the current token's K/V given to fastocr_attend_append (its cache row
    # holding NaN before the call) gives the outputs of fastocr_attend on a
    # cache that already holds the row, bit for bit, and writes the row; the
    # appending handle's outputs, focal set and kept sets also match the
    # oracle (non-focal layers conditioned on the set the handle attended
    # with)
    from oracle import DecodeOracle
    name, over, mode, steps, env = APPEND_CASES[case]
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    wl = get_workload(name).with_overrides(**over)
    up = upload(wl, steps=steps)
    L, B, Hq, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim
    ha = fo.fastocr_create(make_config(up, mode=mode))
    hb = fo.fastocr_create(make_config(up, mode=mode))
    kb = [k.clone() for k in up.Kd]
    vb = [v.clone() for v in up.Vd]
    out_a = torch.empty((B, Hq, d), dtype=up.io_dtype, device=DEV)
    out_b = torch.empty_like(out_a)
    k_max = fo.fastocr_get_info(hb)["k_max"]
    sel = torch.zeros((B, k_max), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    orc = DecodeOracle(num_layers=L, num_q_heads=Hq, num_kv_heads=wl.num_kv_heads, head_dim=d, tau=wl.tau,
                       num_focal=wl.num_focal, warmup_steps=wl.warmup_steps)
    focal, worst = [], 0.0
    for t in range(steps):
        pruned = mode == "pruned" and t >= wl.warmup_steps
        if mode == "pruned" and t < wl.warmup_steps:
            orc.step(t, lambda l: up.q[l][t].astype(np.float64), up.kv64, up.st.lens(t))
        if mode == "pruned" and t == wl.warmup_steps:
            focal = fo.fastocr_profile_warmup(hb)
            assert fo.fastocr_profile_warmup(ha) == focal
            assert focal == [int(x) for x in orc.focal], (focal, list(orc.focal))
        unused = unused_picks(focal, L) if pruned else set()
        cur = up.st.lens(t)[:, 1] - 1
        for l in range(L):
            bi = torch.arange(B, device=DEV)
            ci = torch.from_numpy(cur.astype(np.int64)).to(DEV)
            k_new = up.Kd[l][bi, :, ci].contiguous()  # [B, Hkv, d]
            v_new = up.Vd[l][bi, :, ci].contiguous()
            kb[l][bi, :, ci] = float("nan")
            vb[l][bi, :, ci] = float("nan")
            kind = "sparse" if pruned and l not in focal else ("focal" if pruned and l not in unused else "full")
            if kind == "sparse":
                fo.fastocr_get_selection(hb, sel, cnt)  # the set this layer attends with
            fo.fastocr_attend(ha, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out_a)
            fo.fastocr_attend_append(hb, l, up.Qd[l][t], k_new, v_new, kb[l], vb[l], up.lens[t], out_b)
            if kind == "focal":
                fo.fastocr_get_selection(hb, sel, cnt)  # the set this layer picked
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b), f"step {t} layer {l}"
            s_np = (sel.cpu().numpy(), cnt.cpu().numpy())
            worst = max(worst, check_layer(up, t, l, out_b.float().cpu().numpy().astype(np.float64), kind,
                                           used=s_np, picked=s_np, what=f"append {case}"))
    for l in range(L):
        assert torch.equal(kb[l], up.Kd[l]) and torch.equal(vb[l], up.Vd[l]), f"layer {l} cache"
    assert fo.fastocr_get_status(ha) == 0 and fo.fastocr_get_status(hb) == 0
    log(f"[append] {case}: focal {focal}, worst out vs oracle {worst:.2e}")


# ---------------------------------------------------------------------------
# periodic re-selection of the focal layers
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name,over,R", [
    # planted strong layers {1, 3} -> {0, 2} at step 20; windows at steps
    # 0-3, 12-15, 24-27, 36-39
    ("tiny-fp32", dict(steps=40, drift=(20, (0, 2))), 8),
    # strong band 14-22 -> layers {3, 7, 11, 25} at step 20; windows at
    # steps 0-7, 20-27, 40-47
    ("7b-b1", dict(steps=50, drift=(20, (3, 7, 11, 25))), 12),
])
def test_reprofile_follows_drift(name, over, R):
    from oracle import DecodeOracle
    wl = get_workload(name).with_overrides(**over)
    up = upload(wl)
    L, B, Hq, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim
    h = fo.fastocr_create(make_config(up, reprofile_every=R))
    orc = DecodeOracle(num_layers=L, num_q_heads=Hq, num_kv_heads=wl.num_kv_heads, head_dim=d,
                       tau=wl.tau, num_focal=wl.num_focal, warmup_steps=wl.warmup_steps,
                       reprofile_every=R)
    scale = 1 / math.sqrt(d)
    k_max = fo.fastocr_get_info(h)["k_max"]
    sel = torch.zeros((B, k_max), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, d), dtype=up.io_dtype, device=DEV)
    picks, prev, worst, jac = [], None, 0.0, []
    for t in range(wl.steps):
        lens = up.st.lens(t)
        rec = orc.step(t, lambda l: up.q[l][t].astype(np.float64), up.kv64, lens)
        phase = fo.fastocr_get_info(h)["phase"]
        if t == wl.warmup_steps:
            assert phase == 1
            fo.fastocr_profile_warmup(h)
        assert (phase == 0) == (rec.phase == "warmup"), (t, phase, rec.phase)
        for l in range(L):
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out)
            got = out.float().cpu().numpy().astype(np.float64)
            what = f"t={t} l={l}"
            if l == 0 and rec.phase == "pruned":
                # a window that just ended was profiled by this call
                focal = fo.fastocr_get_focal_layers(h)
                assert focal == [int(x) for x in orc.focal], (t, focal, list(orc.focal))
                if prev.phase == "warmup":
                    picks.append((t, focal))
            if rec.phase == "warmup" or l in orc.focal:
                worst = max(worst, check_out(got, rec.outs[l], wl.dtype, what))
            if rec.phase == "pruned":
                fo.fastocr_get_selection(h, sel, cnt)
                c, s = cnt.cpu().numpy(), sel.cpu().numpy()
                for b in range(B):
                    n, length = int(lens[b, 0]), int(lens[b, 1])
                    k = kept_count(wl.tau, n)
                    if l in orc.focal:
                        if l not in unused_picks(orc.focal, L):
                            jac.append(check_set(s[b, :c[b]], rec.scores[l][b], k, f"set {what} b={b}"))
                    else:
                        if l == 0 and prev.phase == "warmup":
                            # warm start right after a (re-)profile: the
                            # window's last step at the deepest focal layer
                            jac.append(check_set(s[b, :c[b]], prev.scores[max(orc.focal)][b], k,
                                                 f"warm start {what} b={b}"))
                        want = sparse_attention(up.q[l][t][b].astype(np.float64), up.kv64(l)[0][b],
                                                up.kv64(l)[1][b], s[b, :c[b]], n, length, scale)
                        worst = max(worst, check_out(got[b], want, wl.dtype, f"{what} b={b}"))
        prev = rec
    want_picks = [(t, [int(x) for x in c]) for t, c in orc.profiles if t < wl.steps]
    assert picks == want_picks, (picks, want_picks)
    assert len(picks) >= 3 and picks[0][1] != picks[-1][1], picks  # the drift was followed
    assert fo.fastocr_get_info(h)["profiles"] == len(want_picks)
    assert fo.fastocr_get_status(h) == 0
    fo.fastocr_destroy(h)
    log(f"[reprofile] {name}: picks {picks}, worst out {worst:.2e}, mean Jaccard {np.mean(jac):.3f}")


def test_set_focal_layers_ends_window_then_reprofiles():
    # tiny fp32 page with re-selection after every R = 3 pruned steps.  The
    # first window is ended by fastocr_set_focal_layers with a set of our
    # choosing instead of the profiled one: the warm start is top-k of the
    # window's last-step scores at the deepest given layer, the pruned steps
    # run with that set, and the next window profiles itself at its end
    # (the oracle is conditioned the same way: its focal set and warm start
    # are replaced after its first window)
    from oracle import DecodeOracle
    R = 3
    wl = get_workload("tiny-fp32").with_overrides(steps=4 + R + 4 + 2)
    up = upload(wl)
    L, B, Hq, d, w = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim, wl.warmup_steps
    h = fo.fastocr_create(make_config(up, reprofile_every=R))
    orc = DecodeOracle(num_layers=L, num_q_heads=Hq, num_kv_heads=wl.num_kv_heads, head_dim=d, tau=wl.tau,
                       num_focal=wl.num_focal, warmup_steps=w, reprofile_every=R)
    k_max = fo.fastocr_get_info(h)["k_max"]
    sel = torch.zeros((B, k_max), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, d), dtype=up.io_dtype, device=DEV)
    chosen = [0, 2]  # the planted strong layers are {1, 3}
    with pytest.raises(fo.FastOCRError) as err:
        fo.fastocr_set_focal_layers(h, chosen)  # the window is not complete
    assert err.value.code == fo.ERR_STATE
    worst, focal = 0.0, None
    for t in range(wl.steps):
        lens = up.st.lens(t)
        rec = orc.step(t, lambda l: up.q[l][t].astype(np.float64), up.kv64, lens)
        if t == w - 1:
            # condition the oracle: C and the warm start come from `chosen`
            orc.focal = np.array(chosen)
            orc.f_last = [select_top(orc.warm_scores[max(chosen)][b], kept_count(wl.tau, int(lens[b, 0])))
                          for b in range(B)]
        if t == w:
            for bad in ([0, 1, 2], [1], [2, 2]):
                with pytest.raises(fo.FastOCRError) as err:
                    fo.fastocr_set_focal_layers(h, bad)
                assert err.value.code == fo.ERR_INVALID_ARG, bad
            fo.fastocr_set_focal_layers(h, chosen)
            info = fo.fastocr_get_info(h)
            assert info["profiles"] == 1 and info["phase"] == 2
            assert fo.fastocr_get_focal_layers(h) == chosen
            fo.fastocr_get_selection(h, sel, cnt)
            s_np, c_np = sel.cpu().numpy(), cnt.cpu().numpy()
            for b in range(B):
                n = int(lens[b, 0])
                check_set(s_np[b, :c_np[b]], orc.warm_scores[max(chosen)][b], kept_count(wl.tau, n),
                          f"warm start b={b}")
        for l in range(L):
            pruned = rec.phase == "pruned"
            focal_now = [int(x) for x in orc.focal] if orc.focal is not None else []
            kind = "sparse" if pruned and l not in focal_now else (
                "focal" if pruned and l not in unused_picks(focal_now, L) else "full")
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out)
            if l == 0 and pruned:
                focal = fo.fastocr_get_focal_layers(h)
                assert focal == focal_now, (t, focal, focal_now)
            # the set after the call: the one a non-focal layer attended with
            # (a layer-0 call that ends a window re-initialises it first) or
            # the one a focal layer picked
            fo.fastocr_get_selection(h, sel, cnt)
            torch.cuda.synchronize()
            s_np = (sel.cpu().numpy(), cnt.cpu().numpy())
            worst = max(worst, check_layer(up, t, l, out.float().cpu().numpy().astype(np.float64), kind,
                                           used=s_np, picked=s_np, what="set-then-reprofile"))
    # the second window (steps w+R .. w+R+w-1) was profiled by the GPU itself
    assert fo.fastocr_get_info(h)["profiles"] == 2
    assert focal == [int(x) for x in orc.profiles[-1][1]] != chosen, (focal, orc.profiles)
    assert fo.fastocr_get_status(h) == 0
    fo.fastocr_destroy(h)
    log(f"[set-focal] chosen {chosen} then re-picked {focal}; worst out {worst:.2e}")


# ---------------------------------------------------------------------------
# degenerate sequences and the largest head layouts the ABI accepts
# ---------------------------------------------------------------------------


def _small_ragged(**over):
    base = dict(batch=4, num_layers=4, focal_band=(1, 2), num_focal=2, warmup_steps=2,
                n_img_range=(30, 60), n_prompt=(30, 40))
    base.update(over)
    return get_workload("7b-b16-ragged").with_overrides(**base)


@pytest.mark.parametrize("mode", ["pruned", "full"])
def test_degenerate_sequences(mode):
    # one batch holding a normal sequence, a text-only one (no image
    # tokens), an empty one (len = 0: zero output, no image mass) and one
    # whose only text rows are the generated tokens
    steps = 6
    up = upload(_small_ragged(), steps=steps)
    st = up.st
    n = st.n_img.copy()
    p = st.n_prompt.copy()
    n[1], p[1] = 0, 30
    n[2] = 0
    p[3] = 0
    empty = np.array([False, False, True, False])

    def lens(t, n=n, p=p):
        out = np.stack([n, n + p + t + 1], axis=1).astype(np.int32)
        out[empty] = 0
        return out

    st.n_img = n
    st.lens = lens
    up.lens = torch.from_numpy(np.stack([lens(t) for t in range(steps)])).to(DEV)
    h = fo.fastocr_create(make_config(up, mode=mode))
    rec = run(up, h, steps)
    assert rec.status == 0
    assert np.all(rec.outs[:, :, 2] == 0.0)  # the empty sequence
    if mode == "full":
        scale = 1 / math.sqrt(up.wl.head_dim)
        for t in range(steps):
            for l in range(up.wl.num_layers):
                K, V = up.kv64(l)
                for b in range(up.wl.batch):
                    want, _ = full_attention(up.q[l][t][b].astype(np.float64), K[b], V[b],
                                             int(lens(t)[b, 1]), scale)
                    check_out(rec.outs[t, l, b], want, up.wl.dtype, f"t={t} l={l} b={b}")
        return
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(up.wl.warmup_steps, steps):
        chk.pruned_step(t)
    assert np.all(rec.cnts[up.wl.warmup_steps:, :, 1:3] == 0)  # no image tokens, nothing kept
    log(f"[degenerate] focal {rec.focal}, worst out {chk.worst_out:.2e}")


@pytest.mark.parametrize("hq,hkv,d,dtype", [
    (128, 8, 128, "bf16"),  # the most query heads, a group of 16
    (16, 1, 64, "f32"),     # one KV head serving a group of 16
])
def test_largest_head_layouts(hq, hkv, d, dtype):
    wl = _small_ragged(batch=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                       n_img_range=(200, 700))
    up = upload(wl, steps=6)
    rec = run(up, fo.fastocr_create(make_config(up)), 6)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, 6):
        chk.pruned_step(t)
    log(f"[heads {hq}/{hkv} d={d} {dtype}] focal {rec.focal}, worst out {chk.worst_out:.2e}")


# ---------------------------------------------------------------------------
# image tokens in several pages with text around them
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name,over,steps", [
    # two 8x8 pages behind 12 text tokens with 6 between them
    ("tiny-fp32", dict(batch=2, grid=(16, 8), pages=2, page_text=(12, 6), n_prompt=(38, 38)), None),
    # two 40x80 pages behind 20 text tokens with 12 between them, bf16
    ("7b-b1", dict(pages=2, page_text=(20, 12), n_prompt=(96, 96), num_layers=8, focal_band=(3, 5),
                   num_focal=2, warmup_steps=3), 12),
])
def test_multi_page_layout_packed(name, over, steps):
    import dataclasses
    wl = get_workload(name).with_overrides(**over)
    up = upload(wl, steps=steps)
    wl, st = up.wl, up.st
    B, S = wl.batch, st.max_seq_len
    maps = []
    for b in range(B):
        n, m = fo.fastocr_image_first_map(st.spans[b], S)
        assert n == int(st.n_img[b])
        maps.append(m)
    row_map = torch.tensor(maps, dtype=torch.int32, device=DEV)
    rows = torch.full((B,), S, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    Kp = [torch.empty_like(k) for k in up.Kd]
    Vp = [torch.empty_like(v) for v in up.Vd]
    for l in range(wl.num_layers):
        fo.fastocr_pack_rows(up.Kd[l], Kp[l], row_map, rows, status)
        fo.fastocr_pack_rows(up.Vd[l], Vp[l], row_map, rows, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    perm = torch.tensor(maps, dtype=torch.long, device=DEV)
    for l in range(wl.num_layers):  # a pure row gather: bit-exact
        for b in range(B):
            assert torch.equal(Kp[l][b], up.Kd[l][b][:, perm[b]]), (l, b)
            assert torch.equal(Vp[l][b], up.Vd[l][b][:, perm[b]]), (l, b)
    # the method on the packed cache against the oracle on the page layout
    packed = dataclasses.replace(up, Kd=Kp, Vd=Vp)
    T = wl.steps
    rec = run(packed, fo.fastocr_create(make_config(packed)), T)
    assert rec.status == 0
    chk = Checker(up, rec, spans=st.spans)
    chk.warmup()
    for t in range(wl.warmup_steps, T):
        chk.pruned_step(t)
    log(f"[pages] {name}: focal {rec.focal}, worst out {chk.worst_out:.2e}, "
        f"mean Jaccard {np.mean(chk.jaccard):.3f}")


def test_pack_rows_partial_and_clamped():
    # rows past rows_b are left alone; a map entry outside [0, S) is clamped
    # and flagged
    B, Hkv, S, d = 2, 3, 40, 64
    src = torch.randn((B, Hkv, S, d), device=DEV).to(torch.bfloat16)
    dst = torch.zeros_like(src)
    m = torch.arange(S, dtype=torch.int32, device=DEV).flip(0).repeat(B, 1).contiguous()
    m[1, 3] = S + 7
    rows = torch.tensor([S, 10], dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    fo.fastocr_pack_rows(src, dst, m, rows, status)
    torch.cuda.synchronize()
    assert torch.equal(dst[0], src[0].flip(1))
    want = src[1][:, m[1, :10].clamp(0, S - 1).long()]
    assert torch.equal(dst[1][:, :10], want)
    assert torch.count_nonzero(dst[1][:, 10:]) == 0
    assert int(status.item()) & fo.FLAG_INDEX_CLAMPED


# ---------------------------------------------------------------------------
# seeded random shapes within the ABI's limits
# ---------------------------------------------------------------------------


def _random_workload(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 5, 7, 8, 16]))
    L = int(rng.integers(2, 7))
    lo = int(rng.integers(1, 400))
    hi = lo + int(rng.integers(0, 900))
    plo = int(rng.integers(1, 60))
    nf = int(rng.integers(1, L))
    band_lo = int(rng.integers(0, L - nf + 1))
    return get_workload("7b-b16-ragged").with_overrides(
        batch=int(rng.integers(1, 7)), num_layers=L, num_q_heads=hkv * g, num_kv_heads=hkv,
        head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
        tau=float(rng.choice([0.02, 0.05, 0.1, 0.3, 0.7])), num_focal=nf,
        warmup_steps=int(rng.integers(1, 4)), focal_band=(band_lo, band_lo + nf - 1),
        n_img_range=(lo, hi), n_prompt=(plo, plo + int(rng.integers(0, 120))), seed=5000 + seed)


@SPARSE_VARIANTS
@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(monkeypatch, seed, rows):
    _sparse_variant(monkeypatch, rows)
    wl = _random_workload(seed)
    steps = wl.warmup_steps + 4
    up = upload(wl, steps=steps)
    log(f"[random {seed}] B={wl.batch} L={wl.num_layers} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"d={wl.head_dim} {wl.dtype} tau={wl.tau} n={up.st.n_img.tolist()}")
    rec = run(up, fo.fastocr_create(make_config(up)), steps)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, steps):
        chk.pruned_step(t)


@pytest.mark.parametrize("hq,hkv", [(28, 4), (40, 8), (64, 8), (8, 8)])
def test_valu_full_split_trajectory(monkeypatch, hq, hkv):
    # the VALU full split in warm-up steps (text mass -> focal set) and at
    # tau = 1 on non-focal layers, over a ragged batch
    monkeypatch.setenv("FASTOCR_VALU_FULL", "1")
    wl = _small_ragged(batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16",
                       n_img_range=(300, 1500), tau=1.0)
    up = upload(wl, steps=5)
    rec = run(up, fo.fastocr_create(make_config(up)), 5)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, 5):
        chk.pruned_step(t)
    log(f"[valu {hq}/{hkv}] focal {rec.focal}, worst out {chk.worst_out:.2e}")


# ---------------------------------------------------------------------------
# a captured step replayed as a HIP graph
# ---------------------------------------------------------------------------


def test_graph_replayed_steps_match_eager():
    # one pruned step captured as a graph (q and lens staged by copies, as
    # the benchmark does) and replayed step after step, with another
    # handle's eager steps and synchronisations in between: every replay's
    # outputs and kept set equal the eager step's bit for bit, and every
    # replayed output matches the oracle (focal layers: full attention, their
    # kept sets by the band rule; non-focal layers: attention over the set
    # they used, recorded by the eager handle)
    wl = get_workload("7b-b1").with_overrides(num_layers=6, focal_band=(2, 3), num_focal=2, warmup_steps=2)
    T = 10
    up = upload(wl, steps=T)
    L, B, Hq, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim
    stream = torch.cuda.Stream()
    ha = fo.fastocr_create(make_config(up), stream)
    hb = fo.fastocr_create(make_config(up), stream)
    io = up.io_dtype
    k_max = fo.fastocr_get_info(ha)["k_max"]
    rec_sel = torch.zeros((L, B, k_max), dtype=torch.int32, device=DEV)
    rec_cnt = torch.zeros((L, B), dtype=torch.int32, device=DEV)

    def eager(h, t, outs, focal=None):
        # with `focal`: record the set each non-focal layer attends with and
        # the set each focal layer picks
        for l in range(L):
            if focal is not None and l not in focal:
                fo.fastocr_get_selection(h, rec_sel[l], rec_cnt[l])
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], outs[l])
            if focal is not None and l in focal:
                fo.fastocr_get_selection(h, rec_sel[l], rec_cnt[l])

    scratch = torch.empty((L, B, Hq, d), dtype=io, device=DEV)
    with torch.cuda.stream(stream):
        for t in range(wl.warmup_steps):
            eager(ha, t, scratch)
            eager(hb, t, scratch)
    focal = fo.fastocr_profile_warmup(ha)
    assert fo.fastocr_profile_warmup(hb) == focal
    unused = unused_picks(focal, L)
    q_stage = torch.empty((L, B, Hq, d), dtype=io, device=DEV)
    lens_stage = torch.empty((B, 2), dtype=torch.int32, device=DEV)
    out_stage = torch.empty((L, B, Hq, d), dtype=io, device=DEV)
    sa, sb = (torch.zeros((B, k_max), dtype=torch.int32, device=DEV) for _ in range(2))
    ca, cb = (torch.zeros((B,), dtype=torch.int32, device=DEV) for _ in range(2))
    with torch.cuda.stream(stream):
        q_stage.copy_(torch.stack([up.Qd[l][wl.warmup_steps] for l in range(L)]))
        lens_stage.copy_(up.lens[wl.warmup_steps])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for l in range(L):
            fo.fastocr_attend(ha, l, q_stage[l], up.Kd[l], up.Vd[l], lens_stage, out_stage[l])
    torch.cuda.synchronize()
    out_b = torch.empty((L, B, Hq, d), dtype=io, device=DEV)
    worst = 0.0
    for t in range(wl.warmup_steps, T):
        with torch.cuda.stream(stream):
            q_stage.copy_(torch.stack([up.Qd[l][t] for l in range(L)]))
            lens_stage.copy_(up.lens[t])
            g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            eager(hb, t, out_b, focal)
        torch.cuda.synchronize()
        assert torch.equal(out_stage, out_b), f"step {t}"
        fo.fastocr_get_selection(ha, sa, ca)
        fo.fastocr_get_selection(hb, sb, cb)
        torch.cuda.synchronize()
        assert torch.equal(ca, cb) and torch.equal(sa, sb), f"kept set after step {t}"
        replayed = out_stage.float().cpu().numpy().astype(np.float64)
        rs, rc = rec_sel.cpu().numpy(), rec_cnt.cpu().numpy()
        for l in range(L):
            kind = "full" if l in unused else ("focal" if l in focal else "sparse")
            worst = max(worst, check_layer(up, t, l, replayed[l], kind, used=(rs[l], rc[l]),
                                           picked=(rs[l], rc[l]), what="replay"))
    assert fo.fastocr_get_status(ha) == 0 and fo.fastocr_get_status(hb) == 0
    log(f"[graph] focal {focal}, worst replayed out vs oracle {worst:.2e}")
    del g


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_unknown_bounds(seed):
    # min_img_tokens = max_text_tokens = 0: launches sized for the whole row
    # capacity (most kept-token splits and full-pass splits find no rows)
    wl = _random_workload(100 + seed)
    steps = wl.warmup_steps + 3
    up = upload(wl, steps=steps)
    rec = run(up, fo.fastocr_create(make_config(up, min_img_tokens=0, max_text_tokens=0)), steps)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, steps):
        chk.pruned_step(t)


@pytest.mark.parametrize("name,scale", [("tiny-fp32", 0.05), ("7b-b1", 0.2)])
def test_custom_logit_scale(name, scale):
    # sm_scale given instead of 1/sqrt(d)
    wl = get_workload(name)
    if name == "7b-b1":
        wl = wl.with_overrides(num_layers=4, focal_band=(1, 2), num_focal=2, warmup_steps=2)
    up = upload(wl, steps=8)
    rec = run(up, fo.fastocr_create(make_config(up, sm_scale=scale)), 8)
    assert rec.status == 0
    chk = Checker(up, rec, scale=scale)
    chk.warmup()
    for t in range(wl.warmup_steps, 8):
        chk.pruned_step(t)


@pytest.mark.parametrize("case", ["long-page", "wide-batch"])
def test_large_extents(case):
    # long-page: 40000 image tokens (the in-pipeline top-k beyond 16 keys per
    # thread re-reads its keys per pass); wide-batch: 64 sequences x 8 KV
    # heads (512 pairs per launch row)
    if case == "long-page":
        wl = get_workload("7b-b1").with_overrides(grid=(200, 200), num_layers=3, focal_band=(1, 1),
                                                  num_focal=1, warmup_steps=2, num_q_heads=8, num_kv_heads=1)
    else:
        wl = _small_ragged(batch=64, num_q_heads=32, num_kv_heads=8, n_img_range=(100, 300),
                           n_prompt=(10, 50), num_layers=3, focal_band=(1, 1), num_focal=1)
    up = upload(wl, steps=5)
    rec = run(up, fo.fastocr_create(make_config(up)), 5)
    assert rec.status == 0
    chk = Checker(up, rec)
    chk.warmup()
    for t in range(wl.warmup_steps, 5):
        chk.pruned_step(t)
    log(f"[{case}] focal {rec.focal}, worst out {chk.worst_out:.2e}")


# ---------------------------------------------------------------------------
# decode state moved to another handle between steps
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cut", [2, 4, 6, 10, 13])
def test_save_load_state_resumes_exactly(cut):
    # tiny page, 20 steps, re-selection every 4 pruned steps (windows at
    # steps 0-3, 8-11, 16-19): cuts mid-window, at the end of the first
    # window (before its profile), in pruned steps and mid re-selection
    wl = get_workload("tiny-fp32").with_overrides(steps=20, drift=(10, (0, 2)))
    up = upload(wl)
    L, B, Hq, d, T = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim, wl.steps
    cfg = make_config(up, reprofile_every=4)

    def step(h, t, out):
        info = fo.fastocr_get_info(h)
        if info["phase"] == 1 and info["profiles"] == 0:
            fo.fastocr_profile_warmup(h)
        for l in range(L):
            fo.fastocr_attend(h, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], out[l])

    ha = fo.fastocr_create(cfg)
    scratch = torch.empty((L, B, Hq, d), dtype=up.io_dtype, device=DEV)
    for t in range(cut):
        step(ha, t, scratch)
    blob = fo.fastocr_save_state(ha)
    hb = fo.fastocr_create(cfg)
    fo.fastocr_load_state(hb, blob)
    assert fo.fastocr_get_info(hb)["step"] == cut
    oa = torch.empty((T - cut, L, B, Hq, d), dtype=up.io_dtype, device=DEV)
    ob = torch.empty_like(oa)
    for t in range(cut, T):
        step(ha, t, oa[t - cut])
        step(hb, t, ob[t - cut])
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert fo.fastocr_get_focal_layers(ha) == fo.fastocr_get_focal_layers(hb)
    k_max = fo.fastocr_get_info(ha)["k_max"]
    sa, sb = (torch.zeros((B, k_max), dtype=torch.int32, device=DEV) for _ in range(2))
    ca, cb = (torch.zeros((B,), dtype=torch.int32, device=DEV) for _ in range(2))
    fo.fastocr_get_selection(ha, sa, ca)
    fo.fastocr_get_selection(hb, sb, cb)
    torch.cuda.synchronize()
    assert torch.equal(sa, sb) and torch.equal(ca, cb)
    assert fo.fastocr_get_info(ha)["profiles"] == fo.fastocr_get_info(hb)["profiles"]


def test_save_load_state_errors():
    wl = get_workload("tiny-fp32")
    up = upload(wl, steps=2)
    h = fo.fastocr_create(make_config(up))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=up.io_dtype, device=DEV)
    fo.fastocr_attend(h, 0, up.Qd[0][0], up.Kd[0], up.Vd[0], up.lens[0], out)
    with pytest.raises(fo.FastOCRError) as e:  # mid-step
        fo.fastocr_save_state(h)
    assert e.value.code == fo.ERR_STATE
    for l in range(1, wl.num_layers):
        fo.fastocr_attend(h, l, up.Qd[l][0], up.Kd[l], up.Vd[l], up.lens[0], out)
    blob = fo.fastocr_save_state(h)
    other = fo.fastocr_create(make_config(up, tau=0.2))  # another configuration
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_load_state(other, blob)
    assert e.value.code == fo.ERR_INVALID_ARG
    with pytest.raises(fo.FastOCRError) as e:  # truncated
        fo.fastocr_load_state(fo.fastocr_create(make_config(up)), blob[:100])
    assert e.value.code == fo.ERR_INVALID_ARG
    bad = bytearray(blob)
    bad[0] ^= 0xFF  # not a state blob
    with pytest.raises(fo.FastOCRError) as e:
        fo.fastocr_load_state(fo.fastocr_create(make_config(up)), bytes(bad))
    assert e.value.code == fo.ERR_INVALID_ARG


def test_trace_ranges_leave_results_unchanged(monkeypatch):
    # FASTOCR_TRACE=1 wraps every call in a named roctx range; outputs and
    # kept sets are bitwise those of an untraced run
    wl = get_workload("tiny-fp32")
    up = upload(wl)
    monkeypatch.setenv("FASTOCR_TRACE", "1")
    traced = run(up, fo.fastocr_create(make_config(up)), wl.steps)
    monkeypatch.setenv("FASTOCR_TRACE", "0")
    plain = run(up, fo.fastocr_create(make_config(up)), wl.steps)
    assert np.array_equal(traced.outs, plain.outs)
    assert np.array_equal(traced.sets, plain.sets) and np.array_equal(traced.cnts, plain.cnts)
    assert traced.focal == plain.focal


def test_hand_worked_trajectory_on_gpu():
    # the hand-worked trajectory of tests/golden/trajectory_two_focal.yaml
    # (exact rational outputs, sets and focal layers) run by the library in
    # fp32 with head_dim 64 (the fixture's 8-dimensional rows zero-padded)
    import os
    from fractions import Fraction

    import yaml
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "trajectory_two_focal.yaml")
    fx = yaml.safe_load(open(path))
    L, S, n, P, D = fx["layers"], fx["rows"], fx["n_img"], fx["prompt"], 64
    ex = fx["expect"]
    K = torch.zeros((1, 1, S, D), device=DEV)
    V = torch.zeros((1, 1, S, D), device=DEV)
    for j in range(S):
        K[0, 0, j, j] = 1.0
        V[0, 0, j, :3] = torch.tensor([j + 1, (j + 1) ** 2, 1.0])
    h = fo.fastocr_create(fo.Config(num_layers=L, num_q_heads=1, num_kv_heads=1, head_dim=D, batch=1,
                                    max_seq_len=S, max_img_tokens=n, tau=fx["tau"], num_focal=fx["num_focal"],
                                    warmup_steps=fx["warmup_steps"], dtype="f32", sm_scale=1.0))
    sel = torch.zeros((1, fo.fastocr_get_info(h)["k_max"]), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = torch.empty((1, 1, D), device=DEV)
    for t, per_layer in enumerate(fx["weights"]):
        length = n + P + t + 1
        if t == fx["warmup_steps"]:
            assert fo.fastocr_profile_warmup(h) == ex["focal"]
            ratios = fo.fastocr_get_layer_ratios(h)
            np.testing.assert_allclose(ratios, [float(Fraction(r)) for r in ex["ratios"]], rtol=0, atol=1e-6)
            fo.fastocr_get_selection(h, sel, cnt)
            assert sel[0, :int(cnt.item())].tolist() == ex["warm_start"][0]
        lens = torch.tensor([[n, length]], dtype=torch.int32, device=DEV)
        for l in range(L):
            q = torch.zeros((1, 1, D), device=DEV)
            q[0, 0, :length] = torch.log(torch.tensor(per_layer[l], dtype=torch.float64)).float()
            fo.fastocr_attend(h, l, q, K, V, lens, out)
            want = [float(Fraction(x)) for x in ex["outs"][t][l]]
            got = out[0, 0, :3].cpu().numpy()
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * max(1.0, max(abs(w) for w in want)))
            assert float(out[0, 0, 3:].abs().max()) == 0.0
            if t > 0:
                fo.fastocr_get_selection(h, sel, cnt)
                got_set = sel[0, :int(cnt.item())].tolist()
                focal_sets = ex["sets"][t - 1]
                used = ex["used_sets"][t - 1]
                if l in focal_sets:
                    assert got_set == focal_sets[l], (t, l, got_set)
                else:
                    assert got_set == used[l], (t, l, got_set)
    assert fo.fastocr_get_status(h) == 0
