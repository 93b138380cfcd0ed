"""Host logic of the HBM traffic summary (no GPU).

`bench.py --summarize-traffic` reduces two rocprofv3 --pmc passes over
`bench.py --profile-pass` to bytes per launch of the one-row GEMV.  The
profile pass also launches the multi-row streaming GEMV, the matrix-core
kernels and the prefill GEMM, so the summary must key on the one-row
instantiation alone and scale by the calibration copy.  These tests feed it
counter tables of the layout rocprofv3 writes.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
M1 = "void gq::(anonymous namespace)::gemv_stream_kernel<1, 2, 256, false, false, false>(x)"
M1_512 = "void gq::(anonymous namespace)::gemv_stream_kernel<1, 2, 512, false, false, false>(x)"
MULTI = ["void gq::(anonymous namespace)::gemv_stream_kernel<%d, 2, 256, false, false, false>(x)" % m
         for m in (2, 3, 4)]
M8 = "void gq::(anonymous namespace)::gemv_mfma_stream_kernel<8, 8, 2, false, false, false>(x)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(x)"


def write_pass(d, counter, per_shape_kib, calib_kib, extra_kib=1.0e6):
    """Three decode steps (one-row GEMV per projection), then multi-row and
    matrix-core calls that must be ignored, then the calibration copy."""
    os.makedirs(d)
    rows, i = [], 0
    order = synth.SHAPE_ORDER
    for _ in range(3):
        for nm in order:
            name = M1_512 if nm == "down" else M1
            rows.append((i, name, counter, per_shape_kib[nm]))
            i += 1
    # as many multi-row calls as one-row ones: a filter that let them in would
    # move every shape's median
    for name in MULTI + [M8]:
        for nm in order:
            rows.append((i, name, counter, extra_kib))
            i += 1
    rows.append((i, NEG, counter, calib_kib))
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(FIELDS)
        w.writerows(rows)


def run_summary(tmp_path, fetch_kib, write_kib, calib_fetch, calib_write):
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    write_pass(fd, "FETCH_SIZE", fetch_kib, calib_fetch)
    write_pass(wd, "WRITE_SIZE", write_kib, calib_write)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-traffic", fd, wd],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout)


def test_summary_keys_on_the_one_row_kernel_and_calibrates(tmp_path):
    calib_bytes = bench.CALIB_BYTES
    # counters as this GPU reports them: FETCH_SIZE counts one KiB per 2 KiB
    # moved (2048 bytes per counted KiB), WRITE_SIZE one per KiB
    calib_fetch = calib_bytes / 2048.0
    calib_write = calib_bytes / 1024.0
    fetch = {nm: 1000.0 * (j + 1) for j, nm in enumerate(synth.SHAPE_ORDER)}
    write = {nm: 3.0 * (j + 1) for j, nm in enumerate(synth.SHAPE_ORDER)}
    out = run_summary(tmp_path, fetch, write, calib_fetch, calib_write)
    assert out["FETCH_SIZE"]["scale_bytes_per_KiB"] == pytest.approx(2048.0)
    assert out["WRITE_SIZE"]["scale_bytes_per_KiB"] == pytest.approx(1024.0)
    for nm in synth.SHAPE_ORDER:
        want = fetch[nm] * 2048.0 + write[nm] * 1024.0
        assert out["hbm_bytes_per_launch"][nm] == pytest.approx(want)
        n, k = synth.LLAMA3_8B_SHAPES[nm]
        assert out["algorithmic_bytes_per_launch"][nm] == bench.gemv_bytes(n, k, bench.G)
    assert out["mean_hbm_bytes_per_launch"] == pytest.approx(
        sum(out["hbm_bytes_per_launch"].values()) / len(synth.SHAPE_ORDER))
    assert out["source_sha256_16"] == bench.source_digest()


def test_summary_rejects_a_pass_without_calibration(tmp_path):
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    fetch = {nm: 1.0 for nm in synth.SHAPE_ORDER}
    write_pass(fd, "FETCH_SIZE", fetch, 1.0)
    write_pass(wd, "WRITE_SIZE", fetch, 1.0)
    # drop the calibration rows of the write pass
    p = os.path.join(wd, "run_counter_collection.csv")
    with open(p) as f:
        rows = [r for r in csv.reader(f) if "neg_kernel" not in r[1]]
    with open(p, "w", newline="") as f:
        csv.writer(f).writerows(rows)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-traffic", fd, wd],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "WRITE_SIZE" in (r.stderr + r.stdout)
