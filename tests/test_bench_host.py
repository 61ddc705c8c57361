"""The benchmark's host-side logic, without a GPU: the one-GPU refusal, the
source hash that keeps committed counter figures tied to the kernel they were
taken on, the traffic lookup, and the CPU baseline's sample and JSON object."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("/* header */\nint f(int x)\n{\n    return x + 1;\n}\n// end\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash(str(a)) == bench.source_hash(str(b))
    assert bench.source_hash(str(a)) != bench.source_hash(str(c))


def _traffic_file(path, workload, sha, value):
    path.write_text(f"# counters\nworkload = {workload}\nk_gemm_sha256_16 = {sha}\n"
                    f"traffic_bytes_per_launch = {value}\n")


def test_traffic_is_reported_only_for_the_kernel_it_was_taken_on(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    tf = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "GEMM_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.read_traffic("qkv4096") is None                 # no file
    _traffic_file(tf, "qkv4096", bench.source_hash(str(src)), 12345.0)
    assert bench.read_traffic("qkv4096") == 12345.0
    assert bench.read_traffic("down11008") is None               # another workload
    src.write_text("// a comment\n__global__ void k() {}\n")
    assert bench.read_traffic("qkv4096") == 12345.0              # comment-only edit
    src.write_text("__global__ void k() { int a = 1; }\n")
    assert bench.read_traffic("qkv4096") is None                 # the kernel changed
    _traffic_file(tf, "qkv4096", bench.source_hash(str(src)), "n/a")
    assert bench.read_traffic("qkv4096") is None                 # unreadable figure


def test_committed_traffic_summary_names_its_kernel_and_command():
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    assert kv["workload"] == "qkv4096"
    assert len(kv["k_gemm_sha256_16"]) == 16
    assert float(kv["traffic_bytes_per_launch"]) > 0
    assert "rocprofv3" in open(bench.TRAFFIC_FILE).read()


def test_cpu_baseline_on_a_bounded_sample(orc):
    import workloads as W
    wl = W.WORKLOADS["tiny"]
    inp = W.generate(wl)
    s = bench.cpu_layer_sample(inp, wl, budget_s=5.0, threads=2)
    assert s["tokens"] == wl.M == s["of_tokens"] and s["tops"] > 0
    out = bench.cpu_baseline([("tiny", s)], threads=2)
    assert out["kind"] == "oracle" and out["unit"] == "TOP/s" and out["cores"] == 2
    assert out["value"] == s["tops"] and "tiny" in out["sample"] and "tiny" in out["workloads"]


def test_cpu_sample_stops_at_its_budget(orc):
    """A zero budget still runs one round of blocks and scales it to the batch."""
    import workloads as W
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl)
    s = bench.cpu_layer_sample(inp, wl, budget_s=0.0, threads=2)
    assert s["tokens"] == 128 and s["of_tokens"] == 2048
    assert s["layer_s_per_batch"] >= s["layer_s"] * 15
