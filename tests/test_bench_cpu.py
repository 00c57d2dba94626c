"""Host logic of bench.py, on the CPU: the one-GPU contract and the rule that
the reported HBM traffic comes only from a counter summary taken on the
current kernel source."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_from_a_summary_of_the_current_source(tmp_path):
    bench = _bench_module()
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "softmax_attention_ut_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("// kernel v1\n")
    sha = hashlib.sha256(b"// kernel v1\n").hexdigest()[:16]
    (tmp_path / "profiles" / "k.md").write_text(
        f"# k\n\ntraffic_bytes_per_launch: 123456789\nkernel_source_sha256_16: {sha}\n")
    bench.ROOT = str(tmp_path)
    assert bench._traffic("k.md", "k.hip") == 123456789.0
    # the kernel changed since the counters were taken: no traffic figure
    (src / "k.hip").write_text("// kernel v2\n")
    assert bench._traffic("k.md", "k.hip") is None
    # no summary at all
    assert bench._traffic("missing.md", "k.hip") is None


def test_flop_model_terms_by_enumeration():
    """The carry term counts one d x d product per (query chunk, chunk it is
    carried through): chunks a-1 .. 1 for query chunk a (the walk ends at
    chunk 0, through which nothing is carried)."""
    bench = _bench_module()
    C = 64
    for N in (1, 2, 5, 11):
        L = N * C
        for d in (64, 128):
            f = bench.flop_model(1, 1, L, d)
            carries = sum(max(a - 1, 0) for a in range(N))
            per = 2.0 * d * d * C
            eff = 2.0 * L * L * d
            want = eff + carries * per - N * C * C * d    # the own-chunk Q K^T is the prepare stage's
            assert abs(f["scan"] - want) <= 1e-9 * want, (N, d)
            assert f["eff"] == eff
