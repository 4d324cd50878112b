"""bench.py's contract on the host: the refusal of more than one GPU, the
algorithmic byte / flop counts it divides by, and the rule that committed
HBM traffic counters only count while the kernel they measured is unchanged."""
import importlib.util
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_by_hand():
    b = _bench()

    class Cfg:
        T, d, f, E, k, S, dtype = 16, 2880, 2880, 32, 4, 0, "bf16"

    counts = [2] * 29 + [0] * 3  # 29 active experts
    ac = b.alg_counts(Cfg, counts)
    R = 16 * 4
    assert ac["active"] == 29 and ac["R"] == R
    w_gu = 29 * 2 * 2880 * 2880 * 2
    assert ac["gate_up_bytes"] == w_gu + 16 * 2880 * 2 + R * 2880 * 2
    assert ac["gate_up_bytes"] == 962611200  # the decode workload's figure
    assert ac["down_bytes"] == 29 * 2880 * 2880 * 2 + 2 * R * 2880 * 2
    assert ac["gate_up_flops"] == 4 * 2880 * 2880 * R
    assert ac["layer_flops"] == 2 * 16 * 2880 * 32 + 6 * 2880 * 2880 * R

    class Cfg5(Cfg):
        T, d, f, E, k, S = 4096, 7168, 2048, 256, 8, 1

    ac5 = b.alg_counts(Cfg5, [128] * 256 + [4096])
    assert ac5["active"] == 257 and ac5["R"] == 4096 * 8 + 4096


def test_traffic_only_while_the_kernel_is_unchanged(tmp_path, monkeypatch):
    b = _bench()
    h = hashlib.sha256()
    for path in b.GEMM_SRCS:
        h.update(open(path, "rb").read())
    src_hash = h.hexdigest()[:16]
    assert b.gemm_src_hash() == src_hash
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"w": {"bytes_per_launch": 123,
                                    "gemm_src_sha256_16": src_hash}}))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tf))
    assert b.load_traffic("w") == 123
    assert b.load_traffic("no_such_workload") is None
    # a change to any of the kernel's sources invalidates the stored counters
    orig = tuple(b.GEMM_SRCS)
    for i in range(len(orig)):
        src = tmp_path / f"src{i}"
        src.write_bytes(open(orig[i], "rb").read() + b"\n// changed\n")
        monkeypatch.setattr(b, "GEMM_SRCS",
                            tuple(str(src) if j == i else p for j, p in enumerate(orig)))
        assert b.load_traffic("w") is None
    monkeypatch.setattr(b, "GEMM_SRCS", orig)
    assert b.load_traffic("w") == 123
    # the committed file parses and names the kernel it was taken on
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for ent in data.values():
        assert ent["bytes_per_launch"] > 0 and len(ent["gemm_src_sha256_16"]) == 16

