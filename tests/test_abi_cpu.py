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
