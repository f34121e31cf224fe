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
    """A committed HBM-traffic record is used only while the forward kernel's
    sources are the ones it was measured on (a synthetic record here)."""
    import json
    bench = _bench_module()
    srcs = []
    for name, text in (("inkattn.hip", b"// kernel\n"), ("common.h", b"// shared\n")):
        f = tmp_path / name
        f.write_bytes(text)
        srcs.append(str(f))
    bench.KERNEL_SRCS = srcs
    bench.ROOT = str(tmp_path)
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_source_sha256": bench.kernel_source_sha256(), "hbm_bytes_per_launch": 12345}
    (tmp_path / "profiles" / "traffic_attn_fwd_kernel_wl.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("wl") == 12345
    assert bench.traffic_from_profiles("other") is None          # no record
    (tmp_path / "common.h").write_bytes(b"// shared, changed\n")
    assert bench.traffic_from_profiles("wl") is None              # either source changed
