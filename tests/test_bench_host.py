"""Host logic of bench.py, on the CPU: the algorithmic byte accounting of the
decode and append lines, the counter file's source-hash check, and the
refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_per_unit():
    # units: certified, key fallback, value fallback, both; per unit 8 B of
    # statistics, keys 8,192 codes + 128 scale bytes or 16,384 fp16 bytes,
    # values 4,096 code bytes + 512 scale bytes or 16,384 fp16 bytes
    mask = np.array([[[0, 1, 2, 3]]], np.uint8)
    units = (8 + 8320 + 4608) + (8 + 16384 + 4608) + (8 + 8320 + 16384) + (8 + 16384 + 16384)
    B, Hq = 1, 4
    assert bench.decode_bytes(mask, B, Hq) == units + 2 * B * Hq * 256  # q read and out written


def test_append_bytes_per_token_head():
    # 512 fp16 K and V bytes read; 128 key codes, 2 key-scale bytes, 64 value-code
    # bytes, 8 value-scale bytes written; 8 bytes of block statistics (one per
    # token for a one-token append)
    assert bench.append_bytes(2, 8, 3) == 2 * 8 * 3 * (512 + 128 + 2 + 64 + 8 + 8)


def test_counters_are_used_only_for_the_same_sources(tmp_path):
    h = bench.kernel_source_hash()
    good = tmp_path / "good.json"
    good.write_text(json.dumps({"kernel_source_hash": h, "hbm_bytes_per_launch": 123456}))
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123456}))
    assert bench.traffic_from_counters(str(good)) == 123456.0
    assert bench.traffic_from_counters(str(stale)) is None
    assert bench.traffic_from_counters(str(tmp_path / "absent.json")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
