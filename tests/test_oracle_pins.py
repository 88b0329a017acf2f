"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, a hand-worked fixture, an independent library routine
(torch's scaled_dot_product_attention on the CPU, float64) or brute-force
enumeration.  The tests run every pin; the mutation tests plant plausible
mistakes in the oracle (monkeypatched, CPU only) and check that some pin
catches each of them.
"""

import glob
import itertools
import math
import os

import numpy as np
import pytest
import torch
import yaml

import oracle.fastocr_oracle as ofo
from workload import Generator, get_workload, make_structure

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return yaml.safe_load(f)


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------


def sdpa_reference(q, K, V, mask_rows, scale):
    """torch SDPA (CPU, float64) with grouped KV heads expanded per query head.

    q [Hq, d], K/V [Hkv, S, d], mask_rows: boolean [S] of attended rows.
    """
    Hq, Hkv = q.shape[0], K.shape[0]
    g = Hq // Hkv
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, :, None, :]  # [1,Hq,1,d]
    kt = torch.from_numpy(np.asarray(K, dtype=np.float64)).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(np.asarray(V, dtype=np.float64)).repeat_interleave(g, dim=0)[None]
    m = torch.from_numpy(np.asarray(mask_rows, dtype=bool))[None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0, :, 0, :].numpy()


def sdpa_probs(q, K, mask_rows, scale):
    """Attention probabilities via the same library route: SDPA with V = I."""
    S = K.shape[1]
    Hkv = K.shape[0]
    eye = np.broadcast_to(np.eye(S), (Hkv, S, S)).copy()
    return sdpa_reference(q, K, eye, mask_rows, scale)


def brute_force_top(scores, k):
    """Lexicographically smallest sorted k-subset whose members all score at
    least as high as every non-member (= ties to the lower index)."""
    n = len(scores)
    for subset in itertools.combinations(range(n), k):  # lexicographic order
        inside = [scores[i] for i in subset]
        outside = [scores[i] for i in range(n) if i not in subset]
        if not inside or not outside or min(inside) >= max(outside):
            return list(subset)
    return []


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_golden_decode(name):
    fx = _load(name)
    q = np.array(fx["q"], dtype=np.float64)
    K = np.array(fx["keys"], dtype=np.float64)
    V = np.array(fx["values"], dtype=np.float64)
    n, length, scale = fx["n_img"], fx["length"], fx["scale"]
    ex = fx["expect"]
    out, p = ofo.full_attention(q, K, V, length, scale)
    np.testing.assert_allclose(p, ex["probs"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ex["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ofo.image_scores(p, n), ex["scores"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ofo.image_mass(p, n), ex["image_mass"], rtol=0, atol=1e-12)
    k = ofo.kept_count(fx["tau"], n)
    assert k == ex["kept"], (k, ex["kept"])
    sel = ofo.select_top(ofo.image_scores(p, n), k)
    assert list(sel) == ex["selected"], (list(sel), ex["selected"])
    sp = ofo.sparse_attention(q, K, V, sel, n, length, scale)
    np.testing.assert_allclose(sp, ex["sparse_out"], rtol=0, atol=1e-12)


def pin_golden_spans():
    fx = _load("decode_spans.yaml")
    q = np.array(fx["q"], dtype=np.float64)
    K = np.array(fx["keys"], dtype=np.float64)
    V = np.array(fx["values"], dtype=np.float64)
    length, scale = fx["length"], fx["scale"]
    ex = fx["expect"]
    rows = ofo.image_rows_of([tuple(sp) for sp in fx["spans"]])
    assert list(rows) == ex["image_rows"]
    n = len(rows)
    out, p = ofo.full_attention(q, K, V, length, scale)
    np.testing.assert_allclose(p, ex["probs"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ex["out"], rtol=0, atol=1e-12)
    s = ofo.image_scores(p, n, rows)
    np.testing.assert_allclose(s, ex["scores"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ofo.image_mass(p, n, rows), ex["image_mass"], rtol=0, atol=1e-12)
    k = ofo.kept_count(fx["tau"], n)
    assert k == ex["kept"]
    sel = ofo.select_top(s, k)
    assert list(sel) == ex["selected"]
    sp = ofo.sparse_attention(q, K, V, sel, n, length, scale, rows)
    np.testing.assert_allclose(sp, ex["sparse_out"], rtol=0, atol=1e-12)


def pin_golden_trajectory():
    """A hand-worked three-step trajectory (tests/golden/trajectory_two_focal.yaml)."""
    from fractions import Fraction
    fx = _load("trajectory_two_focal.yaml")
    L, S, n, P = fx["layers"], fx["rows"], fx["n_img"], fx["prompt"]
    ex = fx["expect"]
    frac = lambda x: float(Fraction(str(x)))  # noqa: E731
    K = np.eye(S)[None, None]  # key row j = e_j, d = S
    V = np.zeros((1, 1, S, S))
    for j in range(S):
        V[0, 0, j, :3] = (j + 1, (j + 1) ** 2, 1)
    orc = ofo.DecodeOracle(num_layers=L, num_q_heads=1, num_kv_heads=1, head_dim=S, tau=fx["tau"],
                           num_focal=fx["num_focal"], warmup_steps=fx["warmup_steps"], scale=1.0)
    for t, per_layer in enumerate(fx["weights"]):
        length = n + P + t + 1
        lens = np.array([[n, length]])

        def q_of(l, t=t, per_layer=per_layer):
            q = np.zeros((1, 1, S))
            a = per_layer[l]
            assert len(a) == length
            q[0, 0, :length] = np.log(np.asarray(a, dtype=np.float64))
            return q
        rec = orc.step(t, q_of, lambda l: (K, V), lens)
        for l in range(L):
            want = np.array([[frac(x) for x in ex["outs"][t][l]] + [0.0] * (S - 3)])
            np.testing.assert_allclose(rec.outs[l][0], want, rtol=0, atol=1e-12)
        if t == 0:
            assert list(orc.focal) == ex["focal"], orc.focal
            np.testing.assert_allclose(orc.ratios, [frac(r) for r in ex["ratios"]], rtol=0, atol=1e-12)
            continue
        assert [list(x) for x in rec.warm_start] == [ex["warm_start"][t - 1]]
        for l, sel in ex["sets"][t - 1].items():
            assert list(rec.sets[int(l)][0]) == sel, (t, l, rec.sets[int(l)][0])
        for l, sel in ex["used_sets"][t - 1].items():
            assert list(rec.used_sets[int(l)][0]) == sel, (t, l, rec.used_sets[int(l)][0])


def pin_kept_counts():
    fx = _load("selection_and_counts.yaml")
    for row in fx["kept"]:
        k = ofo.kept_count(row["tau"], row["n"])
        assert k == row["k"], (row, k)


def pin_golden_topk():
    fx = _load("selection_and_counts.yaml")["topk"]
    for case in fx["cases"]:
        got = list(ofo.select_top(np.array(fx["scores"]), case["k"]))
        assert got == case["selected"], (case, got)


def pin_golden_focal():
    fx = _load("selection_and_counts.yaml")["focal"]
    for case in fx["cases"]:
        got = list(ofo.choose_focal_layers(fx["ratios"], case["num_focal"]))
        assert got == case["layers"], (case, got)


def _rand_case(rng, Hq, Hkv, S, d):
    q = rng.standard_normal((Hq, d)) * 2.0
    K = rng.standard_normal((Hkv, S, d))
    V = rng.standard_normal((Hkv, S, d))
    return q, K, V


def pin_full_vs_sdpa():
    rng = np.random.default_rng(7)
    for Hq, Hkv, S, d in [(4, 2, 37, 16), (6, 3, 64, 8), (28, 4, 50, 32), (8, 8, 9, 4)]:
        q, K, V = _rand_case(rng, Hq, Hkv, S, d)
        length = S - 3
        scale = 1.0 / math.sqrt(d)
        mask = np.arange(S) < length
        out, p = ofo.full_attention(q, K, V, length, scale)
        np.testing.assert_allclose(out, sdpa_reference(q, K, V, mask, scale), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(p, sdpa_probs(q, K, mask, scale)[:, :length], rtol=1e-10, atol=1e-13)


def pin_sparse_vs_masked_sdpa():
    rng = np.random.default_rng(11)
    for Hq, Hkv, S, d, n in [(4, 2, 40, 16, 25), (6, 2, 30, 8, 10), (2, 1, 12, 4, 12)]:
        q, K, V = _rand_case(rng, Hq, Hkv, S, d)
        length = S - 2
        scale = 1.0 / math.sqrt(d)
        for trial in range(3):
            k = int(rng.integers(0, n + 1))
            sel = np.sort(rng.choice(n, size=k, replace=False))
            mask = np.zeros(S, dtype=bool)
            mask[sel] = True
            mask[n:length] = True
            got = ofo.sparse_attention(q, K, V, sel, n, length, scale)
            np.testing.assert_allclose(got, sdpa_reference(q, K, V, mask, scale), rtol=1e-10, atol=1e-12)


def pin_tau_one_is_full():
    rng = np.random.default_rng(3)
    q, K, V = _rand_case(rng, 4, 2, 30, 8)
    n, length, scale = 20, 28, 1 / math.sqrt(8)
    out, p = ofo.full_attention(q, K, V, length, scale)
    k = ofo.kept_count(1.0, n)
    assert k == n
    sel = ofo.select_top(ofo.image_scores(p, n), k)
    np.testing.assert_allclose(ofo.sparse_attention(q, K, V, sel, n, length, scale), out,
                               rtol=1e-12, atol=1e-13)


def pin_uniform_keys():
    # All keys equal => every attended row gets probability exactly 1/len,
    # the output is the mean value row, and each image token scores Hq/len.
    rng = np.random.default_rng(5)
    Hq, Hkv, S, d, n = 6, 2, 21, 8, 13
    q = rng.standard_normal((Hq, d))
    K = np.broadcast_to(rng.standard_normal(d), (Hkv, S, d)).copy()
    V = rng.standard_normal((Hkv, S, d))
    length = 19
    out, p = ofo.full_attention(q, K, V, length, 0.3)
    np.testing.assert_allclose(p, np.full((Hq, length), 1.0 / length), rtol=1e-13)
    for h in range(Hq):
        np.testing.assert_allclose(out[h], V[h // (Hq // Hkv), :length].mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ofo.image_scores(p, n), np.full(n, Hq / length), rtol=1e-13)


def pin_mass_identities():
    rng = np.random.default_rng(9)
    Hq, Hkv, S, d, n = 8, 2, 60, 16, 45
    q, K, V = _rand_case(rng, Hq, Hkv, S, d)
    _, p = ofo.full_attention(q, K, V, 55, 0.25)
    np.testing.assert_allclose(p.sum(axis=1), np.ones(Hq), rtol=0, atol=1e-12)
    text_mass = p[:, n:].sum(axis=1)
    total = ofo.image_scores(p, n).sum() + text_mass.sum()
    assert abs(total - Hq) < 1e-12, total
    np.testing.assert_allclose(ofo.image_mass(p, n) + text_mass, np.ones(Hq), atol=1e-12)


def pin_topk_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        scores = rng.integers(0, 4, size=n).astype(np.float64) / 4.0  # many ties
        for k in range(0, n + 1):
            got = list(ofo.select_top(scores, k))
            assert got == brute_force_top(list(scores), k), (scores, k, got)


def pin_focal_brute_force():
    rng = np.random.default_rng(17)
    for trial in range(200):
        L = int(rng.integers(1, 8))
        ratios = rng.integers(0, 3, size=L).astype(np.float64) / 3.0
        for c in range(1, L + 1):
            got = list(ofo.choose_focal_layers(ratios, c))
            assert got == brute_force_top(list(ratios), c), (ratios, c, got)


PINS = [
    pin_kept_counts, pin_golden_topk, pin_golden_focal, pin_full_vs_sdpa,
    pin_sparse_vs_masked_sdpa, pin_tau_one_is_full, pin_uniform_keys,
    pin_mass_identities, pin_topk_brute_force, pin_focal_brute_force, pin_golden_spans,
    pin_golden_trajectory,
] + [lambda name=n: pin_golden_decode(name) for n in
     ("decode_one_head.yaml", "decode_gqa_two_heads.yaml", "decode_gqa_map.yaml")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: getattr(f, "__name__", "golden"))
def test_pin(pin):
    pin()


@pytest.mark.parametrize("name", ["decode_one_head.yaml", "decode_gqa_two_heads.yaml",
                                  "decode_gqa_map.yaml"])
def test_golden_decode(name):
    pin_golden_decode(name)


def test_golden_files_cite_their_source():
    for path in glob.glob(os.path.join(GOLDEN, "*.yaml")):
        head = open(path).read().split("\n", 12)
        text = "\n".join(head)
        assert "FastOCR technical summary" in text or "Focal-Guided Pruning" in text, path


# ---------------------------------------------------------------------------
# whole-procedure properties
# ---------------------------------------------------------------------------


def _oracle_for(wl, **kw):
    return ofo.DecodeOracle(num_layers=wl.num_layers, num_q_heads=wl.num_q_heads,
                            num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, tau=wl.tau,
                            num_focal=wl.num_focal, warmup_steps=wl.warmup_steps, **kw)


def _tiny_inputs(wl):
    st = make_structure(wl)
    gen = Generator(wl, st)
    kv = [tuple(a.astype(np.float64) for a in gen.layer_kv(l)) for l in range(wl.num_layers)]
    qs = [gen.layer_queries(l, K=kv[l][0].astype(np.float32)).astype(np.float64)
          for l in range(wl.num_layers)]
    return st, kv, qs


def test_planted_focal_layers_recovered():
    wl = get_workload("tiny-fp32")
    st, kv, qs = _tiny_inputs(wl)
    orc = _oracle_for(wl)
    for t in range(wl.warmup_steps):
        orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
    assert list(orc.focal) == [1, 3], (orc.focal, orc.ratios)
    r = np.sort(orc.ratios)[::-1]
    assert (r[1] - r[2]) / r[1] > 0.02  # clear margin between focal and the rest


def test_csfr_fixed_point_under_stationary_inputs():
    # Stationary query and frozen cache: every step sees the same inputs, so
    # each focal layer re-picks the previous step's set and the warm start
    # equals the previous step's deepest-focal set (Cross-Step Fixation Reuse).
    wl = get_workload("tiny-fp32")
    st, kv, qs = _tiny_inputs(wl)
    orc = _oracle_for(wl)
    lens = st.lens(wl.warmup_steps)
    t_fix = wl.warmup_steps - 1
    recs = [orc.step(t, lambda l: qs[l][t_fix], lambda l: kv[l], lens)
            for t in range(wl.warmup_steps + 4)]
    pruned = recs[wl.warmup_steps:]
    deepest = int(orc.focal.max())
    for prev, cur in zip(pruned, pruned[1:]):
        for l in prev.sets:
            assert all(np.array_equal(a, b) for a, b in zip(prev.sets[l], cur.sets[l]))
        assert all(np.array_equal(a, b) for a, b in zip(cur.warm_start, prev.sets[deepest]))
        for a, b in zip(prev.outs, cur.outs):
            np.testing.assert_array_equal(a, b)
    # The warm start of the first pruned step is the pick from the last
    # warm-up step's scores at the deepest focal layer, which with stationary
    # inputs equals that layer's fresh pick.
    assert all(np.array_equal(a, b) for a, b in zip(pruned[0].warm_start, pruned[0].sets[deepest]))


def test_focal_layer_zero_ignores_warm_start():
    wl = get_workload("tiny-fp32")
    st, kv, qs = _tiny_inputs(wl)
    orc = _oracle_for(wl)
    for t in range(wl.warmup_steps):
        orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
    orc.focal = np.array([0, 3])
    t = wl.warmup_steps
    orc.f_last = [np.array([0, 1, 2])]
    a = orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
    orc.f_last = [np.arange(200, 226)]
    b = orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
    for x, y in zip(a.outs, b.outs):
        np.testing.assert_array_equal(x, y)


def test_no_eviction_token_reselected_later():
    # A 4x4 page read for 40 steps: the fixation window wraps around the
    # page, so tokens dropped from the set come back.  Nothing is evicted:
    # a re-selected token is attended with its original key/value row.
    wl = get_workload("tiny-fp32").with_overrides(grid=(4, 4), steps=40, num_layers=2,
                                                  planted_layers=(1,), num_focal=1,
                                                  warmup_steps=2, tau=0.25, window=(1, 1))
    st, kv, qs = _tiny_inputs(wl)
    orc = _oracle_for(wl)
    sets = []
    for t in range(wl.steps):
        rec = orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
        if rec.phase == "pruned":
            sets.append((t, set(int(j) for j in rec.sets[1][0])))
    back = False
    for (t1, s1), (t2, s2) in itertools.combinations(sets, 2):
        dropped = s1 - s2
        for t3, s3 in sets:
            if t3 > t2 and dropped & s3:
                back = True
                j = sorted(dropped & s3)[0]
                # Recompute the layer-0 output at t3 with SDPA over the set:
                # it reads row j from the untouched cache.
                rec_sel = sorted(s3)
                n, length = int(st.n_img[0]), int(st.lens(t3)[0, 1])
                mask = np.zeros(kv[0][0].shape[2], dtype=bool)
                mask[rec_sel] = True
                mask[n:length] = True
                want = sdpa_reference(qs[0][t3][0], kv[0][0][0], kv[0][1][0], mask,
                                      1 / math.sqrt(wl.head_dim))
                got = ofo.sparse_attention(qs[0][t3][0], kv[0][0][0], kv[0][1][0],
                                           rec_sel, n, length, 1 / math.sqrt(wl.head_dim))
                np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
                assert j in rec_sel
                break
        if back:
            break
    assert back, "expected some token to be dropped and selected again"


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by some pin
# ---------------------------------------------------------------------------



# ---------------------------------------------------------------------------
# periodic re-selection of the focal layers
# ---------------------------------------------------------------------------


def _drift_run(reprofile_every, oracle_cls=None):
    # tiny page read for 40 steps; the planted strong layers move from {1, 3}
    # to {0, 2} at step 20
    wl = get_workload("tiny-fp32").with_overrides(steps=40, drift=(20, (0, 2)))
    st, kv, qs = _tiny_inputs(wl)
    cls = oracle_cls or ofo.DecodeOracle
    orc = cls(num_layers=wl.num_layers, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
              head_dim=wl.head_dim, tau=wl.tau, num_focal=wl.num_focal,
              warmup_steps=wl.warmup_steps, reprofile_every=reprofile_every)
    recs = [orc.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t)) for t in range(wl.steps)]
    return wl, st, orc, recs


def test_reprofile_follows_planted_drift():
    # windows of w = 4 steps after every 8 pruned steps: steps 0-3, 12-15,
    # 24-27, 36-39; only the window after the drift sees the new layers
    wl, st, orc, recs = _drift_run(8)
    assert [r.phase for r in recs] == (["warmup"] * 4 + ["pruned"] * 8) * 3 + ["warmup"] * 4
    assert [(t, list(c)) for t, c in orc.profiles] == [(4, [1, 3]), (16, [1, 3]), (28, [0, 2]),
                                                       (40, [0, 2])]
    # each re-profile restarts the warm start from its window's last step
    for first in (16, 28):
        focal = [list(c) for t, c in orc.profiles if t == first][0]
        last = recs[first - 1]
        k = ofo.kept_count(wl.tau, int(st.n_img[0]))
        want = ofo.select_top(last.scores[max(focal)][0], k)
        np.testing.assert_array_equal(recs[first].warm_start[0], want)
    # without re-selection the drift is missed
    _, _, orc0, recs0 = _drift_run(0)
    assert [(t, list(c)) for t, c in orc0.profiles] == [(4, [1, 3])]
    assert all(r.phase == "pruned" for r in recs0[4:])


def test_reprofile_pin_catches_pooled_windows():
    # planted mistake: a re-profile that pools every window's statistics
    # instead of using its own window only
    class Pooled(ofo.DecodeOracle):
        def step(self, *a, **k):
            keep = {l: list(v) for l, v in self.mass.items()}
            rec = super().step(*a, **k)
            if self.window_pos == 0 and rec.phase == "pruned":
                self.mass = keep
            return rec

    with pytest.raises(AssertionError):
        _, _, orc, _ = _drift_run(8, oracle_cls=Pooled)
        assert [list(c) for _, c in orc.profiles][2] == [0, 2]



# ---------------------------------------------------------------------------
# image tokens in several spans (pages with text around them)
# ---------------------------------------------------------------------------


def _two_page_inputs():
    wl = get_workload("tiny-fp32").with_overrides(batch=2, grid=(16, 8), pages=2, page_text=(12, 6),
                                                  n_prompt=(38, 38))
    st, kv, qs = _tiny_inputs(wl)
    return wl, st, kv, qs


def _image_first(st, b, S):
    img = st.image_rows[b]
    return np.concatenate([img, np.setdiff1d(np.arange(S), img)])


def test_spans_attention_invariant_under_image_first_permutation():
    # softmax attention does not depend on key order: permuting the cache rows
    # image-first leaves outputs, probabilities per token, scores and masses
    # unchanged (closed form), and rows [0, n) of the permuted cache are the
    # image tokens in span order
    wl, st, kv, qs = _two_page_inputs()
    scale = 1 / math.sqrt(wl.head_dim)
    t = 3
    lens = st.lens(t)
    for b in range(wl.batch):
        n, length = int(lens[b, 0]), int(lens[b, 1])
        perm = _image_first(st, b, st.max_seq_len)
        K, V = kv[0][0][b], kv[0][1][b]
        o1, p1 = ofo.full_attention(qs[0][t][b], K, V, length, scale)
        o2, p2 = ofo.full_attention(qs[0][t][b], K[:, perm], V[:, perm], length, scale)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(p1[:, perm[:length]], p2, rtol=0, atol=1e-15)
        img = st.image_rows[b]
        np.testing.assert_allclose(ofo.image_scores(p1, n, img), ofo.image_scores(p2, n), rtol=1e-12)
        np.testing.assert_allclose(ofo.image_mass(p1, n, img), ofo.image_mass(p2, n), rtol=1e-12)
        sel = np.array([0, 5, 70, 127])
        s1 = ofo.sparse_attention(qs[0][t][b], K, V, sel, n, length, scale, img)
        s2 = ofo.sparse_attention(qs[0][t][b], K[:, perm], V[:, perm], sel, n, length, scale)
        np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-12)


def test_spans_sparse_matches_masked_sdpa():
    import torch
    wl, st, kv, qs = _two_page_inputs()
    scale = 1 / math.sqrt(wl.head_dim)
    t, b = 5, 1
    n, length = (int(x) for x in st.lens(t)[b])
    img = st.image_rows[b]
    sel = np.array([1, 2, 63, 64, 100])
    allowed = np.zeros(length, dtype=bool)
    allowed[img[sel]] = True
    text = np.ones(length, dtype=bool)
    text[img] = False
    allowed |= text
    q = torch.from_numpy(qs[1][t][b])[:, None, :]  # [Hq, 1, d]
    g = wl.num_q_heads // wl.num_kv_heads
    K = torch.from_numpy(kv[1][0][b][:, :length]).repeat_interleave(g, dim=0)
    V = torch.from_numpy(kv[1][1][b][:, :length]).repeat_interleave(g, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(
        q, K, V, attn_mask=torch.from_numpy(allowed)[None, None, :], scale=scale)[:, 0].numpy()
    got = ofo.sparse_attention(qs[1][t][b], kv[1][0][b], kv[1][1][b], sel, n, length, scale, img)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_spans_trajectory_equals_image_first_trajectory():
    # the whole procedure on the page layout (image tokens at their span
    # rows) equals the procedure on the image-first permuted cache
    wl, st, kv, qs = _two_page_inputs()
    S = st.max_seq_len
    perms = [_image_first(st, b, S) for b in range(wl.batch)]
    kv_p = [(np.stack([k[b][:, perms[b]] for b in range(wl.batch)]),
             np.stack([v[b][:, perms[b]] for b in range(wl.batch)])) for k, v in kv]
    a = _oracle_for(wl, spans=st.spans)
    p = _oracle_for(wl)
    for t in range(wl.steps):
        ra = a.step(t, lambda l: qs[l][t], lambda l: kv[l], st.lens(t))
        rp = p.step(t, lambda l: qs[l][t], lambda l: kv_p[l], st.lens(t))
        for x, y in zip(ra.outs, rp.outs):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
        for l in ra.sets:
            assert all(np.array_equal(u, v) for u, v in zip(ra.sets[l], rp.sets[l]))
    assert list(a.focal) == list(p.focal) == [1, 3]


def _mut_gqa_modulo(h, Hq, Hkv):
    return h % Hkv


def _mut_ties_high(scores, k):
    idx = np.arange(len(scores))
    order = np.lexsort((-idx, -np.asarray(scores, dtype=np.float64)))
    return np.sort(order[:k])


def _mut_floor(tau, n):
    return 0 if n <= 0 else int(min(max(math.floor(tau * n), 1), n))


def _mut_mean_scores(p, n, image_rows=None):
    return (p[:, :n] if image_rows is None else p[:, image_rows]).mean(axis=0)


def _mut_drop_current(q, K, V, selected, n, length, scale, image_rows=None):
    sel = np.sort(np.asarray(selected, dtype=np.int64))
    if image_rows is None:
        rows = np.concatenate([sel, np.arange(n, length - 1, dtype=np.int64)])
    else:
        text = np.setdiff1d(np.arange(length - 1, dtype=np.int64), image_rows)
        rows = np.concatenate([np.asarray(image_rows)[sel], text])
    p = ofo.attention_probs(q, K, rows, scale)
    return ofo._weighted_values(p, V, rows)


def _mut_focal_ascending(ratios, c):
    r = np.asarray(ratios, dtype=np.float64)
    return np.sort(np.lexsort((np.arange(len(r)), r))[:c])


def _mut_no_scale(q, K, V, length, scale):
    rows = slice(0, int(length))
    p = ofo.attention_probs(q, K, rows, 1.0)
    return ofo._weighted_values(p, V, rows), p


def _mut_transposed_values(p, V, rows):
    out = np.zeros((p.shape[0], V.shape[2]))
    Hkv = V.shape[0]
    for h in range(p.shape[0]):
        vv = np.asarray(V[ofo.kv_head_of(h, p.shape[0], Hkv)][rows])
        out[h] = (p[h] @ vv[::-1]) if vv.shape[0] > 1 else p[h] @ vv
    return out


MUTATIONS = {
    "gqa_modulo": ("kv_head_of", _mut_gqa_modulo),
    "ties_to_higher_index": ("select_top", _mut_ties_high),
    "k_floor": ("kept_count", _mut_floor),
    "score_mean_over_heads": ("image_scores", _mut_mean_scores),
    "sparse_drops_current_token": ("sparse_attention", _mut_drop_current),
    "focal_lowest_ratio": ("choose_focal_layers", _mut_focal_ascending),
    "missing_logit_scale": ("full_attention", _mut_no_scale),
    "values_rows_reversed": ("_weighted_values", _mut_transposed_values),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(ofo, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(getattr(pin, "__name__", "golden"))
    assert caught, f"no pin caught the planted mistake {mutation}"


class _ProcedureMistake(ofo.DecodeOracle):
    """The pruned step with one planted mistake in the procedure:
    'stale'  non-focal layers keep the step's warm start instead of the
             latest focal pick;
    'first'  the next step starts from the first focal layer's pick, not the
             deepest one's;
    'fixed'  every step starts from the set picked at profile time."""

    bug = None

    def step(self, t, q_of, kv_of, lens):
        if self.window_pos is not None or self.full_mode:
            rec = super().step(t, q_of, kv_of, lens)
            self._profiled = [s.copy() for s in self.f_last] if self.window_pos is None else None
            return rec
        lens = np.asarray(lens)
        rec = ofo.StepRecord(t=t, phase="pruned")
        start = self._profiled if self.bug == "fixed" else self.f_last
        current = [s.copy() for s in start]
        rec.warm_start = [s.copy() for s in current]
        first = None
        for l in range(self.L):
            q, (K, V) = q_of(l), kv_of(l)
            out = np.zeros((lens.shape[0], self.Hq, self.d))
            if l in set(int(c) for c in self.focal):
                rec.sets[l] = []
                for b in range(lens.shape[0]):
                    n, length = int(lens[b, 0]), int(lens[b, 1])
                    out[b], p = ofo.full_attention(q[b], K[b], V[b], length, self.scale)
                    current[b] = ofo.select_top(ofo.image_scores(p, n), ofo.kept_count(self.tau, n))
                    rec.sets[l].append(current[b].copy())
                if first is None:
                    first = [c.copy() for c in current]
            else:
                use = rec.warm_start if self.bug == "stale" else current
                rec.used_sets[l] = [c.copy() for c in use]
                for b in range(lens.shape[0]):
                    n, length = int(lens[b, 0]), int(lens[b, 1])
                    out[b] = ofo.sparse_attention(q[b], K[b], V[b], use[b], n, length, self.scale)
            rec.outs.append(out)
        self.f_last = first if self.bug == "first" else current
        return rec


@pytest.mark.parametrize("bug", ["stale", "first", "fixed"])
def test_trajectory_pin_catches_procedure_mistakes(bug, monkeypatch):
    cls = type(f"Mistake_{bug}", (_ProcedureMistake,), {"bug": bug})
    monkeypatch.setattr(ofo, "DecodeOracle", cls)
    with pytest.raises(AssertionError):
        pin_golden_trajectory()


def test_procedure_mistake_harness_without_mistake_passes(monkeypatch):
    # the mutated step with no mistake planted reproduces the oracle
    monkeypatch.setattr(ofo, "DecodeOracle", type("NoMistake", (_ProcedureMistake,), {"bug": None}))
    pin_golden_trajectory()
