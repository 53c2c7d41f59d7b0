"""bench.py's host-side contract, on the CPU: one GPU only (a request of
several exits with status 2 and says why, before touching a device), and the
pure helpers that turn measurements into the JSON line."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = _bench(env=env)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def _import_bench():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    return bench


def test_expected_tau_closed_form():
    """E[tau] = sum_{j<=K} p^j = (1 - p^(K+1)) / (1 - p); at p = 0.7, K = 8 the
    3.1988 the bench line reports beside the realized tau."""
    bench = _import_bench()
    for p in (0.0, 0.3, 0.7, 0.95):
        for K in (0, 1, 8, 15):
            want = K + 1 if p == 1.0 else (1 - p ** (K + 1)) / (1 - p)
            assert abs(bench.expected_tau(p, K) - want) < 1e-12
    assert bench.expected_tau(1.0, 8) == 9.0
    assert abs(bench.expected_tau(0.7, 8) - 3.1988) < 1e-4


def test_encoder_flops_of_a_large_v3_window():
    """Per 30 s window of the large-v3 encoder: stem 17.69 GFLOP (two width-3
    convolutions, 3000 and 1500 frames), per block QKV 14.75, attention 11.52,
    output 4.92, fc1 and fc2 19.66 GFLOP each; 2.274 TFLOP in all."""
    bench = _import_bench()
    from synthetic import ENC_LARGE_V3
    f = bench.encoder_flops(ENC_LARGE_V3, 1)
    L = ENC_LARGE_V3.n_layers
    assert abs(f["stem"] / 1e9 - 17.69) < 0.01
    for k, g in (("qkv", 14.75), ("attn", 11.52), ("oproj", 4.92), ("fc1", 19.66), ("fc2", 19.66)):
        assert abs(f[k] / L / 1e9 - g) < 0.01, k
    assert abs(sum(f.values()) / 1e12 - 2.274) < 0.001
    f32 = bench.encoder_flops(ENC_LARGE_V3, 32)
    assert all(f32[k] == 32 * f[k] for k in f)


def test_traffic_is_reported_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    """A stored HBM-traffic figure is used only while the kernel sources hash
    to the value it was taken with."""
    import json
    bench = _import_bench()
    wl = "large-v3-verify-b32-greedy"
    h = bench.kernel_source_hash(wl)
    (tmp_path / "profiles").mkdir()
    entries = [{"workload": wl, "kind": "cross_attn", "source_hash": h, "hbm_bytes_per_launch": 2.5e8},
               {"workload": wl, "kind": "qkv", "source_hash": "0" * 16, "hbm_bytes_per_launch": 2e7}]
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(entries))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_of(wl, "cross_attn") == 2.5e8
    assert bench.traffic_of(wl, "qkv") is None           # taken from other sources
    assert bench.traffic_of(wl, "fc1") is None           # never taken
    assert bench.traffic_of("large-v3-verify-b1", "cross_attn") is None
