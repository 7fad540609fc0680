"""bench.py's command line on the CPU: it runs on one GPU only and says so for
any other --gpus before it touches torch or the GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_counted_traffic_is_keyed_to_the_gemm_sources(tmp_path):
    # The bench reports the counted HBM bytes of its dominant kernel only while
    # the GEMM sources hash to the value recorded beside the counters; an edit
    # to those sources turns the figure into null until the counters are retaken.
    import json
    import shutil
    b = _bench_module()
    rec = json.load(open(b.TRAFFIC_FILE))
    name, entry = next(iter(rec["kernels"].items()))
    assert b.measured_traffic(name) == entry["hbm_bytes_per_launch"]
    assert b.measured_traffic("no_such_kernel") is None
    for f in b.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)
    b.ROOT = str(tmp_path)
    assert b.measured_traffic(name) == entry["hbm_bytes_per_launch"]  # same bytes, same hash
    with open(tmp_path / b.KERNEL_SOURCES[0], "a") as fh:
        fh.write("\n")
    assert b.measured_traffic(name) is None
