"""bench.py's algorithmic byte counts, which every reported GB/s and
roofline fraction divides by, against the closed forms of the layouts, and
its one-GPU contract. No GPU."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("name,kv_bytes,append_bytes", [
    # 8-bit codes with one fp32 scale per (token, head) for K and for V:
    # 2 (128 + 4); append: bf16 K and V in (2 * 128 * 2) + that, per head,
    # plus the 8-byte slot
    ("llama3_70b", 2 * (128 + 4), 8 * (2 * 128 * 2 + 264) + 8),
    ("llama3_8b", 2 * (128 + 4), 6216),
    # 4-bit codes, fp32 scale + uint8 zero point per 32-element group
    ("int4_long", 2 * (64 + 4 * 5), 8 * (512 + 168) + 8),
    # per-channel INT8 keys (a scale per channel per 16-token block) and
    # per-token INT8 values
    ("mixed", 128 + 128 * 4 / 16 + 128 + 4, 8 * (512 + 292) + 8),
    # 16-bit passthrough: no metadata
    ("llama3_70b_bf16", 2 * 128 * 2, 8 * (512 + 512) + 8),
])
def test_algorithmic_bytes(name, kv_bytes, append_bytes):
    w = workloads.get(name)
    assert bench.kv_bytes_per_token_head(w) == kv_bytes
    assert bench.append_bytes_per_token(w) == append_bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
