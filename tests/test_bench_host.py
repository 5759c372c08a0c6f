"""Host-side checks of bench.py (no GPU): the one-GPU guard, the digest that
ties committed counter summaries to the kernel sources, and the rule that a
summary taken on other sources reports no traffic."""
import importlib.util
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_digest_ignores_comments_and_layout_but_not_code(tmp_path):
    bench = _bench()
    srcs = []
    for p in bench.KERNEL_SOURCES:
        q = tmp_path / p.name
        q.write_text(p.read_text())
        srcs.append(q)
    bench.KERNEL_SOURCES = srcs
    d0 = bench.kernel_digest()
    srcs[0].write_text("// a new comment line\n" + srcs[0].read_text().replace("\n", "\n\n", 3))
    assert bench.kernel_digest() == d0
    srcs[0].write_text(srcs[0].read_text() + "\nstatic int extra_symbol;\n")
    assert bench.kernel_digest() != d0


def test_traffic_is_null_for_a_summary_of_other_sources(tmp_path):
    bench = _bench()
    (tmp_path / "profiles").mkdir()
    digest = bench.kernel_digest()
    good = f"kernel_sources_sha256_16: {digest}\nhbm_bytes_per_launch: 1234.0\n"
    (tmp_path / "profiles" / "attn_fwd_traffic_x.txt").write_text(good)
    stale = good.replace(digest, "0" * 16)
    (tmp_path / "profiles" / "attn_fwd_traffic_y.txt").write_text(stale)
    bench.ROOT = tmp_path
    assert bench.measured_traffic("x") == 1234.0
    assert bench.measured_traffic("y") is None
    assert bench.measured_traffic("z") is None
