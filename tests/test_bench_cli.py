"""Host-side checks of bench.py's command line (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profiling_modes_are_listed():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--profile-gate", "--profile-rows", "--profile-mlp", "--profile-trellis"):
        assert flag in r.stdout


def test_profile_rows_outside_the_choices_is_rejected():
    r = _run("--profile-gate", "1", "--profile-rows", "3")
    assert r.returncode != 0
    assert "invalid choice" in r.stderr


def test_source_hash_is_stable_and_short():
    sys.path.insert(0, ROOT)
    import bench
    h1, h2 = bench.src_hash(), bench.src_hash()
    assert h1 == h2 and len(h1) == 16
    int(h1, 16)
