"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop counts
its roofline figures divide by, the counter-summary guard, and the one-GPU rule."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_bytes_k3_shape():
    # q, k, v, out bf16 (4 x 256 B) + log_alpha fp32 (512 B) + beta (4 B) per
    # token-head, plus the initial and final state (2 x 64 KB) per head
    assert bench.prefill_bytes(32768, 96, 128, 1) == 32768 * 96 * 1540 + 2 * 96 * 65536
    assert bench.prefill_bytes(32768, 96, 128, 1) == 4_857_004_032
    # one gate per token-head instead of 128
    assert bench.prefill_bytes(10, 2, 128, 1, gate_width=1) == 10 * 2 * (1024 + 4 + 4) + \
        2 * 2 * 65536


def test_decode_bytes_b256():
    assert bench.decode_bytes(256, 96, 128) == 24576 * (2 * 65536 + 1540)
    assert bench.decode_bytes(256, 96, 128) == 3_259_072_512


def test_backward_bytes_and_flops_per_token_head():
    assert bench.bwd_bytes(1, 1, 128, 0) == 2824
    assert bench.bwd_bytes(32768, 96, 128, 1) == 32768 * 96 * 2824 + 3 * 96 * 65536
    # 18 d^2 + 448 d flop per token-head at d = 128
    assert 18 * 128 * 128 + 448 * 128 == 352_256


def test_traffic_summary_is_read_when_its_hash_matches(tmp_path):
    doc = json.load(open(bench.TRAFFIC_FILE))
    doc["kernel_source_sha256"] = bench.source_digest()
    p = tmp_path / "t.json"
    p.write_text(json.dumps(doc))
    assert bench.measured_traffic(str(p)) == doc["hbm_bytes_per_launch"]


def test_traffic_summary_of_other_sources_is_ignored(tmp_path):
    doc = json.load(open(bench.TRAFFIC_FILE))
    doc["kernel_source_sha256"] = "0" * 64
    p = tmp_path / "t.json"
    p.write_text(json.dumps(doc))
    assert bench.measured_traffic(str(p)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json")) is None


def test_source_digest_is_per_kernel():
    a = bench.source_digest()
    assert a == bench.source_digest()
    assert a != bench.source_digest(bench.DECODE_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
