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


def test_code_hash_ignores_comments_only(tmp_path):
    """The counter summary is tied to the kernel's code: comment and blank-line edits keep the
    hash, a code change alters it."""
    import bench
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {  // doubles\n  return 2 * x;\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// header comment\n\nint f(int x) {  // twice x\n\n  return 2 * x;   \n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return 3 * x;\n}\n")
    assert bench.code_sha256(str(a)) == bench.code_sha256(str(b))
    assert bench.code_sha256(str(a)) != bench.code_sha256(str(c))


def test_per_step_kernel_medians():
    # two traced calls of a three-step loop: loop_init, then split / merge / reduce / commit per step
    T, recs = 3, []
    for call in range(2):
        recs.append(("loop_init", 0.004))
        for t in range(T):
            recs += [("attn_split", 0.070 + 0.001 * t + 0.002 * call), ("attn_merge", 0.007),
                     ("vocab_reduce", 0.009 - 0.001 * t), ("commit", 0.005)]
    got = bench.per_step_kernel_us(recs, T)
    assert got["attn_split"] == [71.0, 72.0, 73.0]     # median of the two calls at each step
    assert got["vocab_reduce"] == [9.0, 8.0, 7.0]
    assert got["commit"] == [5.0, 5.0, 5.0]
    assert "loop_init" not in got
    # a kernel launched a number of times that does not split into steps is left out
    cut = bench.per_step_kernel_us(recs[:-2], T)    # the last reduction and commit missing
    assert "vocab_reduce" not in cut and "commit" not in cut
    assert cut["attn_merge"] == [7.0, 7.0, 7.0]
