"""CPU checks of bench.py's command line: more than one GPU is refused with a
message before anything touches a GPU, and so is a launch with WORLD_SIZE > 1
(as torch.distributed.run would start it); and the HBM traffic the roofline
reports is taken from a counter summary only while that summary names the
hash of the kernel source being measured."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_distributed_launch_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr


def _bench_module(monkeypatch, root):
    import importlib
    sys.path.insert(0, ROOT)
    bench = importlib.import_module("bench")
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench


def _fake_tree(tmp_path, kernel_text):
    csrc = tmp_path / "rope_joint_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "attn_fwd.hip").write_text(kernel_text)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def test_recorded_traffic_needs_the_current_kernel_hash(tmp_path, monkeypatch):
    """The roofline's HBM traffic comes from the committed counter summary only
    while it names the hash of the kernel source that bench.py measures; comment
    and blank-line edits do not change that hash, code edits do."""
    code = "int a; // one\n\n/* block\n comment */ int b;\n"
    root = _fake_tree(tmp_path, code)
    bench = _bench_module(monkeypatch, root)
    h = bench.kernel_source_hash()
    prof = root / "profiles" / "attn_fwd_wl_traffic.md"
    assert bench.recorded_traffic("wl") is None                     # no summary
    prof.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 24.5e9\n")
    assert bench.recorded_traffic("wl") == 24.5e9
    (root / "rope_joint_attention_amd" / "csrc" / "attn_fwd.hip").write_text(
        "int a;   // other words\n/* x */ int b;\n\n")
    assert bench.kernel_source_hash() == h                         # comments only
    assert bench.recorded_traffic("wl") == 24.5e9
    (root / "rope_joint_attention_amd" / "csrc" / "attn_fwd.hip").write_text("int a; int c;\n")
    assert bench.kernel_source_hash() != h
    assert bench.recorded_traffic("wl") is None                     # stale counters
