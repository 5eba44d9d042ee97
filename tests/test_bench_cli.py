"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message and a nonzero status before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def _load_bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_committed_traffic_follows_the_kernel_sources(tmp_path):
    """The stored PMC traffic is reported only while the kernel file and every
    header it includes are the ones the counters were taken on."""
    import shutil
    bench = _load_bench()
    names = ("up_cols_llama7b_relu2_b1_traffic.md", "gather_sel_llama7b_relu2_b1_traffic.md")
    for n in names:
        assert bench.committed_traffic(n, 64) is not None, n   # the committed profiles match
        assert bench.committed_traffic(n, 0) is None, n        # counted on padded rows only
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "sparse_activation_amd" / "csrc"
    csrc.mkdir(parents=True)
    for n in names:
        shutil.copy(os.path.join(ROOT, "profiles", n), tmp_path / "profiles" / n)
    for f in bench.GEMV_SOURCES:
        shutil.copy(os.path.join(ROOT, "sparse_activation_amd", "csrc", f), csrc / f)
    bench.ROOT = str(tmp_path)
    assert bench.committed_traffic(names[0], 64) is not None
    for f in bench.GEMV_SOURCES:   # an edit of any one of them voids the stored figure
        orig = (csrc / f).read_bytes()
        (csrc / f).write_bytes(orig + b"\n")
        assert bench.committed_traffic(names[0], 64) is None, f
        (csrc / f).write_bytes(orig)
    assert bench.committed_traffic(names[0], 64) is not None
