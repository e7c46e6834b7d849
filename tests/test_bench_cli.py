"""CPU tier of the benchmark's command line: more than one GPU is refused before anything runs,
the roofline peaks and the algorithmic-work formula hold what they state."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from block_diffusion_lm_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_published_peaks():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.BF16_PEAK_TFLOPS == 2500.0


def test_attention_units_of_the_long_workload():
    w = I.WORKLOADS["long"]
    lens = I.prefix_lengths(w)
    fl, kv, qb = bench.attn_units(w, lens, np.ones(w.B, bool))
    n = 65536 + 16
    assert fl == 4 * 4 * 32 * 16 * n * 128            # 4 flops per (query row, key, dim): a MAC in QK and in PV
    assert kv == 4 * 2 * 2 * n * 128 * 2              # K and V rows of 2 KV heads, bf16
    assert qb == 4 * 16 * 32 * 128 * 2
    # intensity = query rows per KV head (S * Hq / Hkv = 256) flops per K/V byte
    assert fl / kv == 256
    fl1, kv1, _ = bench.attn_units(w, lens, np.array([True, False, False, False]))
    assert fl1 * 4 == fl and kv1 * 4 == kv
