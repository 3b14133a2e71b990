"""bench.py on the CPU: it runs on one GPU only and says so; the kernel source
hash and the committed counter records it reads are consistent."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_distributed_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The hash that ties a counter record to the kernel sources stays the
    same when only comments or whitespace change, and changes with code."""
    import shutil
    b = _bench_module()
    ref = b.kernel_source_sha()
    csrc = tmp_path / "rmsnorm_linear_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "rmsnorm_linear_amd", "csrc"), csrc,
                    ignore=shutil.ignore_patterns("*.so", "*.o"))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.kernel_source_sha() == ref
    f = csrc / "decode.hip"
    text = f.read_text()
    f.write_text("// a comment\n/* a block\n   comment */\n" + text.replace("\n", "\n\n", 5))
    assert b.kernel_source_sha() == ref
    f.write_text(text + "\nstatic const int fn_hash_probe = 1;\n")
    assert b.kernel_source_sha() != ref


def test_committed_counter_records_match_the_kernel_sources():
    """Every committed counter record was taken on the current kernel
    sources, names a summary that exists, and its HBM bytes are the sum of
    the scaled fetch and write bytes."""
    import glob
    import json
    b = _bench_module()
    sha = b.kernel_source_sha()
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert paths
    for p in paths:
        with open(p) as f:
            t = json.load(f)
        name = os.path.basename(p)
        assert t["kernel_src_sha"] == sha, f"{name}: counters taken on other kernel sources"
        assert os.path.exists(os.path.join(ROOT, t["summary"])), name
        assert t["fetch_bytes_per_launch"] > 0 and t["write_bytes_per_launch"] > 0, name
        assert abs(t["hbm_bytes_per_launch"] - t["fetch_bytes_per_launch"] - t["write_bytes_per_launch"]) \
            <= 1e-9 * t["hbm_bytes_per_launch"], name
        assert t["hbm_bytes_per_launch"] >= 0.9 * t["algorithmic_bytes"], name


def test_kernel_source_hash_covers_every_library_source():
    """Every source file of the library (kernels and the C ABI layer that
    picks tiles and passes) feeds the hash, so a change to any of them
    invalidates the committed counter records."""
    import glob
    b = _bench_module()
    files = sorted(os.path.basename(p) for ext in ("*.hip", "*.cpp", "*.hpp")
                   for p in glob.glob(os.path.join(ROOT, "rmsnorm_linear_amd", "csrc", ext)))
    assert sorted(b.KERNEL_SOURCES) == files
