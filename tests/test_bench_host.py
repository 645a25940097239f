"""Host-side checks of bench.py that need no GPU: the one-GPU refusal and the
traffic-summary reader (counter figures are dropped once the kernel sources
they were taken on change)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_reader_rejects_other_sources():
    m = _bench_module()
    # the qmv summary does not describe the GEMM source, nor a missing summary anything
    assert m.measured_traffic("qmv_affine_m1", ["qmm.hip"]) is None
    assert m.measured_traffic("no_such_summary", ["qmv.hip"]) is None


def test_algorithmic_bytes_of_the_decode_shapes():
    m = _bench_module()
    # codes K/2 + bf16 scale and bias per 64-group + x + y, per [N, K] matrix
    assert m.affine_bytes(25600, 5120) == 73_789_440
    assert m.affine_bytes(5120, 25600) == 73_789_440
    # MXFP4: codes + one E8M0 byte per 32 + x + y
    assert m.fp4_bytes(5760, 2880, 32) == 5760 * 1440 + 5760 * 90 + 2 * 2880 + 2 * 5760
