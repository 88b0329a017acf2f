"""Host-side logic of bench.py (no GPU): kernel classes from demangled names,
counter summaries with the copy-kernel calibration, the digest gate on
committed traffic figures, and the one-GPU guard."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("name,cls", [
    ("void fastocr::split_attn_kernel<unsigned short, 128, 0, 4, 2, false>(fastocr::SplitParams)", "full_split"),
    ("void fastocr::split_attn_kernel<unsigned short, 128, 1, 4, 2, true>(fastocr::SplitParams)", "focal_split"),
    ("void fastocr::kept_attn_kernel<unsigned short, 128, 4, 2, false>(fastocr::SplitParams)", "sparse_split"),
    ("void fastocr::merge_kernel<unsigned short, 128>(fastocr::MergeParams)", "merge"),
    ("void fastocr::kept_merge_kernel<float, 64, true>(fastocr::MergeParams)", "merge"),
    ("fastocr::topk_kernel(fastocr::TopkParams)", "topk"),
    ("void at::native::elementwise_kernel<128, 4>(int)", None),
])
def test_kernel_class(name, cls):
    assert bench.kernel_class(name) == cls


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_pmc_summary_scales_by_calibration(tmp_path, capsys):
    cal = bench.CAL_BYTES // 1024
    fetch = tmp_path / "fetch"
    write = tmp_path / "write"
    fetch.mkdir()
    write.mkdir()
    split = "void fastocr::split_attn_kernel<unsigned short, 128, 2, 4, 2>(fastocr::SplitParams)"
    add = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<long>>"
    # FETCH_SIZE counts half of the calibration copy, WRITE_SIZE all of it
    _counter_csv(fetch / "run_counter_collection.csv", [
        {"Kernel_Name": add, "Counter_Name": "FETCH_SIZE", "Counter_Value": cal / 2},
        {"Kernel_Name": split, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": split, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
    ])
    _counter_csv(write / "run_counter_collection.csv", [
        {"Kernel_Name": add, "Counter_Name": "WRITE_SIZE", "Counter_Value": cal},
        {"Kernel_Name": split, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
    ])
    log = tmp_path / "run.log"
    log.write_text('[bench] noise\n{"value": 1.0, "alg_bytes_per_launch_run": {"sparse_split": 4321}}\n')
    bench.pmc_summary([str(fetch), str(write), str(log)])
    out = capsys.readouterr().out
    vals = dict(line.split("#")[0].split(":", 1) for line in out.splitlines() if ":" in line)
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    assert float(vals["calibration_FETCH_SIZE"]) == pytest.approx(2.0)
    assert float(vals["calibration_WRITE_SIZE"]) == pytest.approx(1.0)
    # (mean 200 KiB fetched x 2 + 10 KiB written) per launch
    assert float(vals["sparse_split.hbm_bytes_per_launch"]) == pytest.approx((200 * 2 + 10) * 1024, rel=1e-6)
    assert vals["library_source_sha256_16"] == bench.library_source_digest()
    assert int(vals["sparse_split.run_alg_bytes_per_launch"]) == 4321


def test_read_traffic_requires_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    text = ("# header: with a colon\nlibrary_source_sha256_16: {}\nsparse_split.hbm_bytes_per_launch: 1234  # note\n"
            "sparse_split.run_alg_bytes_per_launch: 1200  # rows\n")
    (prof / "pmc_w.txt").write_text(text.format(bench.library_source_digest()))
    assert bench.read_traffic("sparse_split", "w") == (1234.0, 1200.0)
    assert bench.read_traffic("merge", "w") == (None, None)
    assert bench.read_traffic("sparse_split", "other") == (None, None)
    (prof / "pmc_w.txt").write_text(text.format("0" * 16))
    assert bench.read_traffic("sparse_split", "w") == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("workload,shard", [("72b-b8-sweep", 3), ("7b-b1", 8), ("32b-b4-longpage", 0)])
def test_tp_shard_must_divide_the_heads(workload, shard):
    # a tensor-parallel rank's share needs a whole number of KV and query heads
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload,
                        "--tp-shard", str(shard)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "must divide" in r.stderr, r.stderr
