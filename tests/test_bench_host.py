"""Host logic of bench.py, on the CPU: the refusal of more than one GPU,
the kernel-source hash that gates the committed HBM-counter figure, and the
reading of that figure from a counter summary."""
import os
import subprocess
import sys

import bench

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def _hash_of(tmp_path, texts, monkeypatch):
    paths = []
    for i, t in enumerate(texts):
        p = tmp_path / f"src{i}.hip"
        p.write_text(t)
        paths.append(str(p))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", paths)
    return bench.kernel_source_hash()


def test_kernel_hash_ignores_comments_and_layout_not_code(tmp_path, monkeypatch):
    base = ["int f(int x) { return x + 1; }  // add one\n", "/* header */ #define K 4\n"]
    h = _hash_of(tmp_path, base, monkeypatch)
    recommented = ["// a new comment\nint f(int x) {\n    return x + 1;\n}\n", "/* other\n header */\n#define K 4\n"]
    assert _hash_of(tmp_path, recommented, monkeypatch) == h
    assert _hash_of(tmp_path, ["int f(int x) { return x + 2; }\n", base[1]], monkeypatch) != h
    assert _hash_of(tmp_path, [base[0], "#define K 8\n"], monkeypatch) != h


def test_counter_figure_only_for_the_recorded_kernel(tmp_path, monkeypatch):
    prof = tmp_path / "counters.md"
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(prof))
    assert bench.counters_from_profile() is None  # no summary
    current = bench.kernel_source_hash()
    prof.write_text(f"# summary\n\n- kernel_source_sha256_16: {current}\n- hbm_bytes_per_dispatch: 7516208717\n")
    assert bench.counters_from_profile() == 7516208717.0
    prof.write_text("- kernel_source_sha256_16: 0123456789abcdef\n- hbm_bytes_per_dispatch: 7516208717\n")
    assert bench.counters_from_profile() is None  # taken on other kernel sources
    prof.write_text(f"- kernel_source_sha256_16: {current}\n")
    assert bench.counters_from_profile() is None  # no figure


def test_committed_counter_summary_matches_the_current_kernel():
    """The summary under profiles/ was taken on the kernel sources in the
    tree, so bench.py reports roofline.traffic from it."""
    v = bench.counters_from_profile()
    assert v is not None and abs(v / (28 * (1 << 28)) - 1) < 0.01
