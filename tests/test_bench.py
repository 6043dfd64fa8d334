"""bench.py's host-side contract: the algorithmic flop count and the
source-hash gate on the committed traffic figures (CPU only; the one-GPU
refusal is tested with the ABI)."""

import importlib.util
import json
import os

from software_pipelined_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_flops_count_visible_pairs_only():
    full = I.AttnConfig("t", 2, 3, 5, 64, False, seed=1)
    causal = I.AttnConfig("t", 2, 3, 5, 64, True, seed=1)
    assert full.flops() == 4 * 2 * 3 * 64 * 5 * 5
    assert causal.flops() == 4 * 2 * 3 * 64 * (5 * 6 // 2)
    # the headline workload: 2 x 16 heads of 16384^2 pairs at d = 128
    assert I.HEADLINE.flops() == 4 * 2 * 16 * 128 * 16384 * 16384 == 4398046511104


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    bench = load_bench()
    rec = {"w": {"kernel_source_sha256_16": "0123456789abcdef", "hbm_bytes_per_launch": 12345}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("w") == 12345
    assert bench.measured_traffic("other") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.measured_traffic("w") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("w") is None


def test_committed_traffic_record_is_consistent():
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for name, ent in rec.items():
        cal = ent["copy_calibration"]
        # the calibration copy moves copy_bytes in and out; the scales map the counters to bytes
        assert abs(cal["fetch_size_kb"] * 1024 * cal["fetch_scale"] - cal["copy_bytes"]) < 1e-6 * cal["copy_bytes"]
        assert abs(cal["write_size_kb"] * 1024 * cal["write_scale"] - cal["copy_bytes"]) < 1e-6 * cal["copy_bytes"]
        hbm = ent["fetch_size_kb_per_launch"] * 1024 * cal["fetch_scale"] + \
            ent["write_size_kb_per_launch"] * 1024 * cal["write_scale"]
        assert abs(hbm - ent["hbm_bytes_per_launch"]) <= 1
        cfg = {c.name: c for c in I.CONFIGS}[name]
        n = cfg.B * cfg.H * cfg.N
        assert ent["compulsory_bytes_per_launch"] == 3 * n * cfg.d * 2 + n * cfg.d * 4 + n * 4
        assert ent["hbm_bytes_per_launch"] >= ent["compulsory_bytes_per_launch"]


def test_other_rows_algorithmic_counts():
    """The work and byte counts the other bench modes divide by, against
    brute-force counts on small shapes."""
    # ChunkScan: causal pairs inside each chunk, ragged last chunk included
    cs = I.ChunkScanConfig("t", 2, 70, 3, 64, 32, seed=1)
    brute = sum(1 for s in range(cs.S) for k in range(cs.S) if k // cs.L == s // cs.L and k <= s)
    assert cs.pairs() == brute
    assert cs.flops() == 2 * cs.B * cs.H * cs.P * brute
    nc = 3
    assert cs.hbm_bytes() == (2 * 2 * 70 * 3 * 64 + 2 * 2 * nc * 32 * 32 + 2 * 4 * 2 * 3 * nc * 32
                              + 4 * 2 * 70 * 3 * 64)
    # backward: five contractions over the visible pairs, 2.5x the forward's two
    for cfg in I.CONFIGS:
        assert 2 * I.bwd_flops(cfg) == 5 * cfg.flops()
    # decoding: q, k, v read once in bf16, out and lse written once in fp32
    dc = I.DecodeConfig("t", 3, 4, 2, 100, 64, seed=1)
    assert dc.kv_bytes() == 2 * (3 * 4 * 2 * 64 + 2 * 3 * 4 * 100 * 64) + 4 * 3 * 4 * 2 * 65
    assert dc.flops() == 4 * 3 * 4 * 2 * 100 * 64
    # MLA: q and the shared cache read once, out (512 wide) and lse written once
    m = I.MlaConfig("t", 2, 64, 10, seed=1)
    assert m.hbm_bytes() == 2 * (2 * 64 * 576 + 2 * 10 * 576) + 4 * 2 * 64 * 513
    assert m.flops() == 2 * 2 * 64 * 10 * (576 + 512)

