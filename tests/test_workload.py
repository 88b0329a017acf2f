"""Checks of the seeded synthetic workload generator (CPU only)."""

import numpy as np
import pytest
import torch

from workload import (WORKLOADS, Generator, bf16_bits, bf16_round, bits_to_f32, get_workload,
                      make_structure)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -0.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x), want)
    np.testing.assert_array_equal(bits_to_f32(bf16_bits(x)), want)


@pytest.mark.parametrize("name", ["tiny-fp32", "7b-b1", "7b-b16-ragged", "32b-b4-longpage",
                                  "72b-b8-sweep"])
def test_structure_shapes(name):
    wl = WORKLOADS[name]
    st = make_structure(wl)
    assert st.centre.shape == (wl.steps, wl.batch)
    assert st.alpha.shape == (wl.num_layers,)
    assert np.all(st.centre < st.n_img[None, :])
    lens0 = st.lens(0)
    assert np.all(lens0[:, 1] == st.n_img + st.n_prompt + 1)
    assert st.max_seq_len == int(np.max(st.n_img + st.n_prompt)) + wl.steps
    if wl.n_img_range is not None:
        assert np.all((st.n_img >= wl.n_img_range[0]) & (st.n_img <= wl.n_img_range[1]))
        assert np.all(st.grid_w * st.grid_h >= st.n_img)
    if wl.focal_band is not None:
        lo, hi = wl.focal_band
        assert np.all(st.alpha[lo:hi + 1] == wl.alpha_hi)
        rest = np.r_[st.alpha[:lo], st.alpha[hi + 1:]]
        assert np.all((rest >= 0.3) & (rest <= 1.0))


def test_named_sizes():
    st = make_structure(WORKLOADS["7b-b1"])
    assert int(st.n_img[0]) == 6400 and int(st.n_prompt[0]) == 64 and st.max_seq_len == 7488
    st = make_structure(WORKLOADS["32b-b4-longpage"])
    assert st.max_seq_len == 16384 + 128 + 4096
    assert WORKLOADS["32b-b4-longpage"].focal_band == (32, 50)
    assert WORKLOADS["72b-b8-sweep"].focal_band == (40, 62)


def test_window_and_trajectory():
    wl = WORKLOADS["tiny-fp32"]
    st = make_structure(wl)
    # centre advances one cell per step from cell 0 for a single sequence
    assert list(st.centre[:, 0]) == list(range(wl.steps))
    # 3x3 window clipped at the top-left corner: rows 0..1, cols 0..1
    assert list(st.windows[0][0]) == [0, 1, 16, 17]
    assert list(st.windows[0][5]) == [4, 5, 6, 20, 21, 22]
    wl3 = WORKLOADS["32b-b4-longpage"]
    st3 = make_structure(wl3)
    W = 128
    for b in range(wl3.batch):
        c = st3.centre[:, b]
        for t in range(1, wl3.steps):
            if t % 128 == 0:
                assert c[t] // W == (c[t - 1] // W + 1) % 128
            else:
                assert c[t] == (c[t - 1] + 1) % 16384


def test_generator_deterministic_and_moments():
    wl = get_workload("tiny-fp32")
    g1, g2 = Generator(wl), Generator(wl)
    K1, V1 = g1.layer_kv(2)
    K2, V2 = g2.layer_kv(2)
    np.testing.assert_array_equal(K1, K2)
    np.testing.assert_array_equal(V1, V2)
    assert abs(K1.mean()) < 0.02 and abs(K1.std() - 1) < 0.02
    q_all = g1.layer_queries(2)
    q_some = g2.layer_queries(2, steps=[3, 7])
    np.testing.assert_array_equal(q_all[[3, 7]], q_some)
    # query = alpha * window-mean key + sigma * noise
    st = g1.st
    mean_key = K1[0, 0, st.windows[0][3]].mean(axis=0)
    resid = q_all[3, 0, 0] - st.alpha[2] * mean_key
    assert abs(resid.std() - wl.sigma) < 0.15


def test_bf16_workload_values_are_representable():
    wl = get_workload("7b-b1").with_overrides(num_layers=1, steps=4)
    g = Generator(wl)
    K, V = g.layer_kv(0)
    np.testing.assert_array_equal(bf16_round(K[:, :, :64]), K[:, :, :64])
    q = g.layer_queries(0, K=K)
    np.testing.assert_array_equal(bf16_round(q), q)
