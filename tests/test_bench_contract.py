"""The bench's contract on the CPU: it refuses more than one GPU, and the
algorithmic bytes it divides by a launch's duration are the per-unit sums the
design states, worked out here by hand for each fixed-budget workload."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import configs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


# per unit and step: K and V rows (B slots), the policy's metadata, q, k, v
# read (3 d s), token t's K/V row written, the float32 output (4 d)
@pytest.mark.parametrize("name,units,expect", [
    # OPT-30B H2O: 408 x 256 x 2 + 408 x 12 + (768 + 512 + 512) = 215,584 B
    ("opt30b_decode_h2o", 1792, 215584),
    # 4-bit slots: rows of 64 code bytes + 4 scales = 80 B:
    # 408 x 80 x 2 + 408 x 12 + (768 + 160 + 512) = 71,616 B
    ("opt30b_decode_h2o_q4", 1792, 71616),
    # OPT-6.7B layer, fp16: 102 x 256 x 2 + 102 x 12 + 1,792 = 55,240 B
    ("opt6.7b_layer_h2o", 2048, 55240),
    # persistence: 64-bit history read + written and the position, 20 B a slot
    ("opt30b_decode_persist", 1792, 408 * 512 + 408 * 20 + 1792),
    # HashEvict, 32-bit sketches: 4096 x 512 + 4096 x (4 + 4) + 1,792 + 4
    ("hashevict_lsh", 512, 4096 * 512 + 4096 * 8 + 1792 + 4),
])
def test_algorithmic_bytes_per_launch(name, units, expect):
    w = configs.get(name)
    assert w.units_per_layer == units
    assert bench.decode_bytes_per_layer_step(w) == units * expect


def test_headline_launch_bytes():
    assert bench.decode_bytes_per_layer_step(configs.get("opt30b_decode_h2o")) == 386_326_528
