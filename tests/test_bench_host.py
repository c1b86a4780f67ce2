"""Host-side checks of bench.py that need no GPU: the one-GPU refusal and the
kernel-source hash that ties committed counters to the source they were
taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_kernel_source_hash_ignores_comments(tmp_path):
    import bench
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block */\n")
    b.write_text("int f(int x) {   return x + 1; }\n")
    assert bench.kernel_source_sha(str(a)) == bench.kernel_source_sha(str(b))
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_sha(str(a)) != bench.kernel_source_sha(str(b))


def test_also_measured_configurations_exist():
    import bench
    import workloads
    for label, wname, backward, bits, cold in bench.ALSO:
        assert wname in workloads.WORKLOADS, label
        assert bits in (0, 4, 8)
