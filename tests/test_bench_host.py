"""Host-side checks of bench.py's bookkeeping: the one-GPU guard, the
comment-free source digest that keys the traffic records, and the turning of
two rocprofv3 counter runs into a traffic record.  No GPU is used."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = bench.ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--variant", "--storage", "--workload",
                 "--dims", "--size-sweep", "--march-sweep", "--variant-table", "--traffic"):
        assert flag in r.stdout, flag


def test_strip_comments_ignores_comments_and_layout_only():
    src = 'int a = 1; // one\n/* block\n comment */ float s = "x // y"; char c = \'/\';\n'
    assert bench.strip_comments(src) == 'int a = 1; float s = "x // y"; char c = \'/\';'
    # a comment-only or layout-only edit leaves the text the digest sees unchanged
    edited = src.replace("// one", "// another remark").replace("int a", "int   a")
    assert bench.strip_comments(edited) == bench.strip_comments(src)
    # a code edit does not
    assert bench.strip_comments(src.replace("1;", "2;")) != bench.strip_comments(src)


def test_digest_follows_the_kernel_sources(tmp_path, monkeypatch):
    d0 = bench.kernel_source_digest("tb3")
    fake = tmp_path / "repo"
    csrc = fake / "stencil_dual_update_amd" / "csrc"
    csrc.mkdir(parents=True)
    real = os.path.join(ROOT, "stencil_dual_update_amd", "csrc")
    for name in bench.KERNELS["tb3"][1]:
        with open(os.path.join(real, name)) as f:
            (csrc / name).write_text(f.read())
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.kernel_source_digest("tb3") == d0
    k = csrc / "tv_fgp_tb3_kernel.hpp"
    k.write_text("// a new leading comment\n" + k.read_text())
    assert bench.kernel_source_digest("tb3") == d0
    k.write_text(k.read_text() + "\nstatic int extra_symbol;\n")
    assert bench.kernel_source_digest("tb3") != d0


def _write_counter_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, value) in enumerate(rows, 1):
            # two counter lines per dispatch (as for a counter summed over
            # instances), which the reader adds up
            for half in (value / 2, value / 2):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": 1,
                            "Counter_Name": "X", "Counter_Value": half})


def test_traffic_record_from_two_counter_runs(tmp_path, monkeypatch):
    # FETCH reads half the bytes of the 1 GiB copy (scale 2), WRITE all of
    # them (scale 1); torch's earlier copies of other sizes must be ignored
    copy_fetch, copy_write = 524288.0, 1048576.0
    kern_fetch, kern_write = 2.5e6, 3.0e6
    fetch = [("__amd_rocclr_copyBuffer", 1.0e6)] * 3 + [("void tvfgp::tb3_kernel<int>", kern_fetch)] * 5 \
        + [("__amd_rocclr_copyBuffer", copy_fetch)] * 23
    write = [("__amd_rocclr_copyBuffer", 7.0e5)] * 3 + [("void tvfgp::tb3_kernel<int>", kern_write)] * 5 \
        + [("__amd_rocclr_copyBuffer", copy_write)] * 23
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counter_csv(fcsv, fetch)
    _write_counter_csv(wcsv, write)
    out = tmp_path / "traffic_tb3_512.json"
    monkeypatch.setattr(bench, "traffic_file", lambda v: str(out))
    bench.write_traffic(str(fcsv), str(wcsv), "tb3")
    rec = json.loads(out.read_text())
    assert rec["fetch"]["scale"] == pytest.approx(2.0)
    assert rec["write"]["scale"] == pytest.approx(1.0)
    assert rec["fetch"]["dispatches"] == 5
    assert rec["hbm_read_bytes_per_launch"] == round(kern_fetch * 2 * 1024)
    assert rec["hbm_write_bytes_per_launch"] == round(kern_write * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 52 * 512 ** 3
    assert rec["kernel_source_sha256"] == bench.kernel_source_digest("tb3")
    # reported while the sources match, withheld once they differ
    assert bench.measured_traffic("tb3", 3) == rec["hbm_bytes_per_launch"]
    assert bench.measured_traffic("tb3", 2) is None
    rec["kernel_source_sha256"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic("tb3", 3) is None


def test_committed_traffic_records_are_consistent():
    for variant in ("tb3", "tb2", "fused"):
        with open(bench.traffic_file(variant)) as f:
            rec = json.load(f)
        assert rec["variant"] == variant
        assert rec["hbm_bytes_per_launch"] == (rec["hbm_read_bytes_per_launch"]
                                              + rec["hbm_write_bytes_per_launch"])
        # at least the compulsory bytes move, and the writes are the six
        # output volumes to within 1%
        assert rec["hbm_bytes_per_launch"] >= 0.99 * rec["algorithmic_bytes_per_launch"]
        assert abs(rec["volumes_written"] - 6.0) < 0.06
