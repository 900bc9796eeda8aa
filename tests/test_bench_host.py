"""Host-side pieces of bench.py (no GPU): the algorithmic byte and FLOP
counts behind the roofline figures, the source-hash gate on measured traffic,
and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_launch():
    # per (sequence, head): state 2 x 65,536 + conv state 2 x 2,304 + q, k, v, z 1,024 + g 512 + beta 4 + out 256
    per = 2 * 65536 + 2 * 2304 + 1024 + 512 + 4 + 256
    assert per == 137476
    # plus conv weights (32 heads x 384 channels x 4 taps fp32), the norm weight and the slot ids
    assert bench.decode_bytes_per_launch(64, 32, 128, 128) == 64 * 32 * per + 32 * 384 * 16 + 128 * 4 + 64 * 4
    assert bench.decode_bytes_per_launch(64, 32, 128, 128) == 281748224
    assert bench.decode_bytes_per_launch(64, 32, 128, 128, state_bytes=2) == 147530496


def test_prefill_work_per_token_head():
    assert bench.prefill_flops_per_token_head(128, 128) == 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128) + 64 * 64 // 3
    assert bench.prefill_flops_per_token_head(128, 128) == 140629
    assert bench.prefill_bytes_per_token_head(128, 128) == 1796


def test_measured_traffic_is_gated_by_the_kernel_source(tmp_path):
    sha = bench.source_sha(bench.DECODE_SOURCES)
    good, bad = tmp_path / "good.json", tmp_path / "bad.json"
    good.write_text(json.dumps({"kernel_source_sha": sha, "traffic_bytes_per_launch": 123}))
    bad.write_text(json.dumps({"kernel_source_sha": "0" * 16, "traffic_bytes_per_launch": 123}))
    assert bench.measured_traffic(str(good), bench.DECODE_SOURCES) == 123
    assert bench.measured_traffic(str(bad), bench.DECODE_SOURCES) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), bench.DECODE_SOURCES) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
