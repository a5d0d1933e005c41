"""bench.py's host-side contract, checked without a GPU: it refuses more than
one GPU before touching the device, and roofline.traffic comes from the
committed counter summary only while the kernel sources still hash to the
digest recorded there."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""        # no JSON line for a refused run


def test_traffic_record_follows_the_source_digest(monkeypatch):
    b = _bench()
    wl = "qwen06b_head_bf16_2048x1024x151936"
    fwd = b.traffic_from_profiles(wl, "fwd_gemm")
    bwd = b.traffic_from_profiles(wl, "bwd_gemm")
    if fwd is None:
        # the sources changed since the counters were taken: both kinds void
        assert bwd is None
    else:
        # algorithmic bytes per launch bound the counters from below: the
        # forward reads W and H once (315 MB), a backward launch about 69 MB
        assert isinstance(fwd, int) and isinstance(bwd, int)
        assert fwd > 315_000_000 and bwd > 69_000_000
    # pretend the sources match: the record is read
    rec_digest = None
    for line in open(os.path.join(ROOT, "profiles",
                                  "fused_ce_gemms_bf16_2048x1024x151936_hbm_traffic.md")):
        if line.startswith("traffic: "):
            rec_digest = line.split('"sources_sha256": "')[1].split('"')[0]
    monkeypatch.setattr(b, "kernel_sources_sha256", lambda: rec_digest)
    assert b.traffic_from_profiles(wl, "bwd_gemm") > 69_000_000
    assert b.traffic_from_profiles("no_such_workload", "fwd_gemm") is None
    assert b.traffic_from_profiles(wl, "no_such_kind") is None
    # any change to the kernel sources voids the record
    monkeypatch.setattr(b, "kernel_sources_sha256", lambda: "0" * 64)
    assert b.traffic_from_profiles(wl, "bwd_gemm") is None
