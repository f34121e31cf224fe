"""bench.py's command line, CPU only: the one-GPU contract is checked before
any GPU work starts."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""      # no JSON line


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_records_follow_the_kernel_sources(tmp_path):
    """The committed HBM-traffic records are used only while the forward
    kernel's sources are the ones they were measured on."""
    bench = _bench_module()
    for wl in ("full_causal_8k", "local", "long", "flex_block_causal"):
        t = bench.traffic_from_profiles(wl)
        assert t is not None and t > 0, f"{wl}: record missing or stale"
    changed = tmp_path / "common.h"
    changed.write_bytes(open(bench.KERNEL_SRCS[1], "rb").read() + b"\n// changed\n")
    bench.KERNEL_SRCS = [bench.KERNEL_SRCS[0], str(changed)]
    assert bench.traffic_from_profiles("full_causal_8k") is None
