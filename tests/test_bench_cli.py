"""bench.py's command line on a machine without a GPU: more than one GPU is refused
with a message before anything touches a device, the help text lists the
measurement modes, and the committed byte counters belong to the current kernel."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "8", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 8" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = run("--gpus", "1", env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE=2" in r.stderr


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--config", "--commit", "--fold", "--overlap", "--offload",
                 "--gather", "--flush-mall", "--cpu-seconds", "--calibrate-copy", "--graph",
                 "--unfused"):
        assert flag in r.stdout


def test_graph_mode_needs_the_device_commit():
    r = run("--graph", "4", "--commit", "host")
    assert r.returncode == 2
    assert "--graph" in r.stderr


def test_committed_counters_match_the_kernel():
    """The byte counters in profiles/traffic.json were taken on the step kernel as
    it is now (their code hash matches), for every workload's default launch, so
    the bench line carries measured traffic; each profile summary names the same
    hash."""
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    for name in ("llama70b", "llama7b", "gpt2s", "ragged"):
        t = bench.measured_traffic(name, "tiled")
        assert t is not None, f"{name}: counters taken on another kernel (hash {h})"
        with open(os.path.join(ROOT, "profiles", f"fused_step_{name}.md")) as f:
            assert h in f.read(), name


def test_fetch_profile_matches_the_kernel():
    """profiles/gather_gpt2s.md was taken on the stage-3 fetch kernel as it is now:
    it names the sha256[:16] of gather_kernels.hip with comments and whitespace
    removed."""
    import hashlib
    import re
    with open(os.path.join(ROOT, "zero_partitioned_optimizer_amd", "csrc", "gather_kernels.hip")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    h = hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]
    with open(os.path.join(ROOT, "profiles", "gather_gpt2s.md")) as f:
        assert h in f.read()
