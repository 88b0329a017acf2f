"""The C ABI library on the CPU: load, exported symbols, host logic and
argument validation.  No kernel is launched here."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import dynamic_kv_cache_amd as fo
from dynamic_kv_cache_amd import _abi
from oracle import choose_focal_layers, kept_count

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fastocr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fastocr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fo.lib()
    names = declared_functions()
    assert len(names) >= 18, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in fastocr.h but not exported"
    assert set(names) == set(n for n, _, _ in _abi.SIGNATURES)


def test_struct_layouts_match_header(tmp_path):
    # the header compiled by the host C compiler gives every field's offset
    # and each struct's size; the ctypes mirrors must agree
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"fastocr_config": _abi.Config, "fastocr_info": _abi.Info, "fastocr_timing": _abi.Timing}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "fastocr.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    include = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-I", include, "-o", str(exe), str(src)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, value = line.split()
        got[(cname, field)] = int(value)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


@pytest.mark.parametrize("tau", [0.02, 0.05, 0.1, 0.2, 0.25, 0.3, 1 / 3, 0.5, 0.7, 1.0])
def test_kept_count_matches_oracle(tau):
    for n in list(range(0, 300)) + [2048, 6400, 8192, 12800, 16384, 65536]:
        assert fo.fastocr_kept_count(tau, n) == kept_count(tau, n), (tau, n)


def test_kept_count_rejects_bad_tau():
    for tau in (0.0, -0.1, 1.5, float("nan")):
        assert fo.fastocr_kept_count(tau, 10) == fo.ERR_INVALID_ARG


def test_choose_focal_layers_matches_oracle():
    rng = np.random.default_rng(1)
    for trial in range(500):
        L = int(rng.integers(1, 40))
        r = rng.integers(0, 5, size=L) / 5.0 if trial % 2 else rng.random(L)
        c = int(rng.integers(1, L + 1))
        assert fo.fastocr_choose_focal_layers(list(r), c) == list(choose_focal_layers(r, c))


def _cfg(**kw):
    base = dict(num_layers=4, num_q_heads=4, num_kv_heads=2, head_dim=64, batch=1, max_seq_len=304,
                max_img_tokens=256, tau=0.1, num_focal=2, warmup_steps=4, dtype="f32")
    base.update(kw)
    return fo.Config(**base).to_c()


BAD = [
    dict(head_dim=96), dict(num_q_heads=5), dict(num_q_heads=34, num_kv_heads=2),
    dict(num_q_heads=136, num_kv_heads=17), dict(tau=0.0), dict(tau=1.01), dict(num_focal=0),
    dict(num_focal=5), dict(warmup_steps=0), dict(max_img_tokens=305), dict(batch=0),
    dict(max_seq_len=0), dict(num_layers=0), dict(sm_scale=-1.0), dict(min_img_tokens=300),
    dict(max_text_tokens=-1), dict(max_text_tokens=305), dict(batch=32768),
    dict(reprofile_every=-1),
]


@pytest.mark.parametrize("bad", BAD, ids=[str(b) for b in BAD])
def test_create_rejects_bad_config(bad):
    c = _cfg(**bad)
    out = ctypes.c_void_p(0)
    assert fo.lib().fastocr_create(ctypes.byref(c), None, ctypes.byref(out)) == fo.ERR_INVALID_ARG
    assert not out.value


def test_null_arguments():
    lib = fo.lib()
    out = ctypes.c_void_p(0)
    assert lib.fastocr_create(None, None, ctypes.byref(out)) == fo.ERR_INVALID_ARG
    c = _cfg()
    assert lib.fastocr_create(ctypes.byref(c), None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_attend(None, 0, None, None, None, None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_profile_warmup(None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_get_focal_layers(None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_state_bytes(None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_save_state(None, None, 0) == fo.ERR_INVALID_ARG
    assert lib.fastocr_load_state(None, None, 0) == fo.ERR_INVALID_ARG
    assert lib.fastocr_destroy(None) == fo.OK
    assert lib.fastocr_select_topk(None, 4, None, 1, 0.5, None, 4, None, None) == fo.ERR_INVALID_ARG


def test_create_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    c = _cfg()
    out = ctypes.c_void_p(0)
    assert fo.lib().fastocr_create(ctypes.byref(c), None, ctypes.byref(out)) == fo.ERR_HIP
    assert not out.value


def test_error_strings():
    for code in (fo.OK, fo.ERR_INVALID_ARG, fo.ERR_STATE, fo.ERR_HIP, fo.ERR_OOM, 7):
        assert isinstance(fo.fastocr_error_string(code), str)


def test_image_first_map_matches_definition():
    # image rows ascending, then every other row ascending
    from oracle import image_rows_of
    rng = np.random.default_rng(3)
    for trial in range(300):
        rows = int(rng.integers(1, 200))
        cuts = np.sort(rng.choice(rows + 1, size=min(2 * int(rng.integers(0, 5)), rows + 1 - rows % 2 - 1),
                                  replace=False))
        spans = [(int(a), int(b - a)) for a, b in zip(cuts[0::2], cuts[1::2])]
        n, m = fo.fastocr_image_first_map(spans, rows)
        img = image_rows_of(spans)
        want = np.concatenate([img, np.setdiff1d(np.arange(rows), img)])
        assert n == len(img) and m == list(want), (spans, rows)


def test_image_first_map_rejects_bad_spans():
    for spans, rows in [([(5, 4), (2, 1)], 20), ([(0, 5), (4, 2)], 20), ([(18, 4)], 20), ([(3, -1)], 20)]:
        with pytest.raises(fo.FastOCRError):
            fo.fastocr_image_first_map(spans, rows)


def test_pack_rows_rejects_bad_arguments():
    lib = fo.lib()
    i32 = ctypes.c_void_p(0x2000)
    # null pointers, bad head_dim, overlapping buffers (the pointers are
    # checked on the host and never dereferenced)
    assert lib.fastocr_pack_rows(None, None, None, None, 1, 1, 8, 64, 1, None, None) == fo.ERR_INVALID_ARG
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100000 + 512)
    assert lib.fastocr_pack_rows(a, b, i32, i32, 1, 1, 8, 64, 1, None, None) == fo.ERR_INVALID_ARG
    c = ctypes.c_void_p(0x200000)
    assert lib.fastocr_pack_rows(a, c, i32, i32, 1, 1, 8, 96, 1, None, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_pack_rows(a, c, i32, i32, 1, 1, 8, 64, 7, None, None) == fo.ERR_INVALID_ARG


def _plan(num_cu=256, **kw):
    base = dict(num_layers=4, num_q_heads=4, num_kv_heads=2, head_dim=64, batch=1, max_seq_len=304,
                max_img_tokens=256, tau=0.1, num_focal=2, warmup_steps=4, dtype="f32")
    base.update(kw)
    return fo.fastocr_plan_launch(fo.Config(**base), num_cu)


@pytest.mark.parametrize("bad", BAD, ids=[str(b) for b in BAD])
def test_plan_rejects_what_create_rejects(bad):
    with pytest.raises(fo.FastOCRError):
        _plan(**bad)


def test_plan_launch_null_and_cu_count():
    lib = fo.lib()
    c = _cfg()
    info = fo._abi.Info()
    assert lib.fastocr_plan_launch(None, 256, ctypes.byref(info)) == fo.ERR_INVALID_ARG
    assert lib.fastocr_plan_launch(ctypes.byref(c), 256, None) == fo.ERR_INVALID_ARG
    assert lib.fastocr_plan_launch(ctypes.byref(c), 0, ctypes.byref(info)) == fo.ERR_INVALID_ARG


MAX_MERGE_STATES = 1024  # merge states per head one merge workgroup holds in LDS
MAX_KEPT_SPLITS = 32     # workgroups per (sequence, KV head) pair of a kept-token pass


def _check_plan(info, S):
    assert info["full_max_splits"] * info["full_rows_per_split"] >= S
    assert info["full_max_splits"] <= MAX_MERGE_STATES
    assert 1 <= info["sparse_max_splits"] <= MAX_KEPT_SPLITS
    assert info["sparse_direct"] == (info["sparse_max_splits"] == 1)


def test_plan_multi_million_rows_stays_within_merge_capacity():
    # full passes of millions of rows grow their splits, and kept-token
    # passes their rows per workgroup, so the merge never sees more states
    # than its LDS holds
    for S in (2_200_000, 3_000_000, 8_000_000):
        info = _plan(num_layers=2, num_q_heads=16, num_kv_heads=8, head_dim=128, batch=1, max_seq_len=S,
                     max_img_tokens=S // 2, tau=0.05, num_focal=1, warmup_steps=1, dtype="bf16")
        _check_plan(info, S)
        assert info["sparse_max_splits"] * info["sparse_rows_per_split"] >= info["k_max"] + S - S // 2


def test_plan_random_configs_within_kernel_limits():
    rng = np.random.default_rng(11)
    for _ in range(400):
        hkv = int(rng.integers(1, 9))
        g = int(rng.integers(1, 17))
        S = int(rng.integers(1, 3_000_000))
        n = int(rng.integers(0, S + 1))
        nmin = int(rng.integers(0, n + 1))
        text = int(rng.integers(0, S + 1))
        info = _plan(num_cu=int(rng.choice([80, 256, 304])), num_layers=2, num_q_heads=hkv * min(g, 128 // hkv),
                     num_kv_heads=hkv, head_dim=int(rng.choice([64, 128])), batch=int(rng.integers(1, 65)),
                     max_seq_len=S, max_img_tokens=n, min_img_tokens=nmin, max_text_tokens=text,
                     tau=float(rng.uniform(0.01, 1.0)), num_focal=1, warmup_steps=1)
        _check_plan(info, S)


def test_plan_of_benchmark_workloads():
    # kept-token passes: each pair's tiles dealt to the workgroups that fill
    # one wave of resident workgroups (3 per CU), at most one per 16-row tile
    # at the longest text and at most 32
    def plan(**kw):
        base = dict(num_layers=80, num_q_heads=64, num_kv_heads=8, head_dim=128, batch=8, max_seq_len=14976,
                    max_img_tokens=12800, min_img_tokens=12800, max_text_tokens=128 + 2048, tau=0.05,
                    num_focal=8, warmup_steps=8, dtype="bf16")
        base.update(kw)
        return _plan(**base)
    b1 = plan(num_layers=28, num_q_heads=28, num_kv_heads=4, batch=1, max_seq_len=7488, max_img_tokens=6400,
              min_img_tokens=6400, max_text_tokens=64 + 1024, num_focal=4)
    assert b1["k_max"] == 320 and b1["sparse_max_splits"] == 32
    w8 = plan()
    assert w8["k_max"] == 640 and w8["sparse_max_splits"] == 3 * 256 // 64
    b4 = plan(num_layers=64, num_q_heads=40, num_kv_heads=8, batch=4, max_seq_len=20608, max_img_tokens=16384,
              min_img_tokens=16384, max_text_tokens=128 + 4096, num_focal=6)
    assert b4["k_max"] == 820 and b4["sparse_max_splits"] == 3 * 256 // 32
    t2 = plan(tau=0.2)
    assert t2["k_max"] == 2560 and t2["sparse_max_splits"] == 12
    for info in (b1, w8, b4, t2):
        _check_plan(info, info["full_max_splits"] * info["full_rows_per_split"])
    # focal passes stage their logits at 1920- and 1408-row splits, not at
    # B=1's 128-row splits
    assert (b1["focal_staged"], w8["focal_staged"], b4["focal_staged"], t2["focal_staged"]) == (0, 1, 1, 1)
    # kept-token passes stream their rows (non-temporal loads) when a step's
    # kept rows exceed the 256 MiB last-level cache: not at B=1 (69 MB)
    assert (b1["stream_rows"], w8["stream_rows"], b4["stream_rows"], t2["stream_rows"]) == (0, 1, 1, 1)


LAST_LEVEL_CACHE_BYTES = 256 << 20


@pytest.mark.parametrize("env", [None, "0", "1"])
def test_plan_kept_row_streaming(monkeypatch, env):
    # pruned handles load kept-token rows non-temporally when the non-focal
    # layers' kept rows at the longest text (k_max image rows + the text
    # bound) exceed the last-level cache; FASTOCR_STREAM_ROWS overrides; full
    # handles run no kept-token pass
    if env is None:
        monkeypatch.delenv("FASTOCR_STREAM_ROWS", raising=False)
    else:
        monkeypatch.setenv("FASTOCR_STREAM_ROWS", env)
    rng = np.random.default_rng(13)
    seen = set()
    for _ in range(300):
        hkv = int(rng.integers(1, 9))
        S = int(rng.integers(16, 40_000))
        n_img = int(rng.integers(1, S + 1))
        min_img = int(rng.integers(0, n_img + 1))
        max_text = int(rng.choice([0, int(rng.integers(1, S + 1))]))
        L = int(rng.integers(2, 81))
        C = int(rng.integers(1, L + 1))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "f32"]))
        mode = str(rng.choice(["pruned", "full"]))
        B = int(rng.integers(1, 33))
        info = _plan(num_layers=L, num_q_heads=hkv * 2, num_kv_heads=hkv, head_dim=d,
                     batch=B, max_seq_len=S, max_img_tokens=n_img, min_img_tokens=min_img,
                     max_text_tokens=max_text, tau=0.05, num_focal=C, warmup_steps=1, dtype=dtype, mode=mode)
        rows = S
        if min_img > 0:
            rows = min(rows, info["k_max"] + S - min_img)
        if max_text > 0:
            rows = min(rows, info["k_max"] + max_text)
        step_bytes = (L - C) * B * hkv * rows * 2 * d * (2 if dtype == "bf16" else 4)
        want = mode == "pruned" and {None: step_bytes > LAST_LEVEL_CACHE_BYTES, "0": False, "1": True}[env]
        assert info["stream_rows"] == int(want), (info, step_bytes)
        seen.add(want)
    assert seen == ({False} if env == "0" else {True, False})


LOGIT_STAGE_FLOATS = 8 * (2048 + 16)  # LDS floats a focal pass stages a split's logits in
LOGIT_STAGE_MIN_ROWS = 512               # rows per split from which it stages them by default


@pytest.mark.parametrize("env", [None, "0", "1"])
def test_plan_focal_logit_staging(monkeypatch, env):
    # a focal pass stages its split's image-token logits in LDS only when the
    # group's heads x (rows per split + 16 padding) fit; by default only for
    # splits of at least 512 rows; FASTOCR_FOCAL_STAGE=0 never, =1 whenever
    # they fit
    if env is None:
        monkeypatch.delenv("FASTOCR_FOCAL_STAGE", raising=False)
    else:
        monkeypatch.setenv("FASTOCR_FOCAL_STAGE", env)
    rng = np.random.default_rng(12)
    seen = set()
    for _ in range(300):
        hkv = int(rng.integers(1, 9))
        g = int(rng.integers(1, 17))
        S = int(rng.integers(1, 200_000))
        info = _plan(num_cu=int(rng.choice([80, 256])), num_layers=2, num_q_heads=hkv * min(g, 128 // hkv),
                     num_kv_heads=hkv, head_dim=128, batch=int(rng.integers(1, 65)), max_seq_len=S,
                     max_img_tokens=int(rng.integers(0, S + 1)), tau=0.05, num_focal=1, warmup_steps=1,
                     dtype="bf16")
        R = info["full_rows_per_split"]
        fits = min(g, 128 // hkv) * (R + 16) <= LOGIT_STAGE_FLOATS
        want = fits and {None: R >= LOGIT_STAGE_MIN_ROWS, "0": False, "1": True}[env]
        assert info["focal_staged"] == int(want), info
        seen.add(want)
    assert seen == ({False} if env == "0" else {True, False})


def test_set_focal_layers_null_handle():
    lib = fo.lib()
    arr = (ctypes.c_int32 * 2)(1, 3)
    assert lib.fastocr_set_focal_layers(None, arr, 2) == fo.ERR_INVALID_ARG
