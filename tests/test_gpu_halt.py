"""GPU parity of adaptive loop halting (bd_loop_halt) against the float64 oracle through the C ABI.

rel: the kernel sums squares in float32 in a fixed order (per-thread chains of at most a few
hundred terms, a 64-lane butterfly, four waves, then at most a few hundred slices in order), so
each sum of nonnegative terms carries a relative error below k * 2^-24 with k < 1000; the square
roots halve it and the quotient adds an ulp: rel within RTOL of the oracle. halt: bit-exact
wherever the oracle's rel is farther than that from epsilon (both decide in float32 there)."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import bf16_f64, dev, dev_bf16

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def to_dev(x, bf16):
    return dev_bf16(x) if bf16 else dev(x)


def to_f64(x, bf16):
    return bf16_f64(x) if bf16 else np.asarray(x, np.float64)


def check(rel, halt, ref_rel, ref_halt, eps, what):
    fin = np.isfinite(ref_rel)
    assert np.array_equal(np.isfinite(rel), fin), f"{what}: finiteness differs"
    assert np.all(rel[~fin] == ref_rel[~fin]), what
    np.testing.assert_allclose(rel[fin], ref_rel[fin], rtol=RTOL, atol=0, err_msg=what)
    assert np.all(rel[ref_rel == 0] == 0), what
    clear = ~np.isfinite(ref_rel) | (np.abs(ref_rel - eps) > 2 * RTOL * eps)
    assert np.array_equal(halt[clear], ref_halt[clear]), f"{what}: halt {halt} vs {ref_halt}"


CASES = [
    # name, B, n, bf16, scales, zero_prev, same, eps, iteration, max_iter
    ("bf16-one-slice", 6, 3000, True, [1e-1, 3e-3, 1e-3, 3e-4, 1e-2, 0.5], (), (), 2e-3, 2, 8),
    ("bf16-ragged-slices", 5, 100000, True, [2e-3, 5e-3, 1e-3, 1e-2, 4e-3], (), (), 4e-3, 3, 12),
    ("f32-degenerate", 6, 4100, False, [1e-2, 1e-5, 1e-3, 1e-2, 0.0, 1e-1], (1, 4), (2,), 5e-3, 1, 4),
    ("f32-budget", 3, 20000, False, [1e-1, 1e-1, 1e-1], (), (), 1e-3, 4, 4),
    ("bf16-eps0", 4, 8, True, [1e-1, 0.0, 2.0, 1e-2], (3,), (1,), 0.0, 1, 3),
    ("one-seq-many-slices", 1, 1 << 20, True, [6e-3], (), (), 5e-3, 1, 8),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_halt_matches_oracle(case):
    name, B, n, bf16, scales, zp, same, eps, it, mx = case
    print(f"[halt] {name} B={B} n={n} bf16={bf16}", flush=True)
    hp, hc = I.loop_states(700 + CASES.index(case), B, n, scales, bf16, zp, same)
    r = bd.loop_halt(to_dev(hp, bf16), to_dev(hc, bf16), it, eps, mx)
    torch.cuda.synchronize()
    ref_rel, ref_halt = O.loop_halt(to_f64(hp, bf16), to_f64(hc, bf16), eps, it, mx)
    check(r["rel"].cpu().numpy().astype(np.float64), r["halt"].cpu().numpy(), ref_rel, ref_halt, eps, name)


def test_halt_degenerate_values():
    hp, hc = I.loop_states(790, 4, 64, [1e-1, 0.0, 1.0, 0.0], False, zero_prev=(2, 3), same=(1, 3))
    r = bd.loop_halt(dev(hp), dev(hc), 1, 1e-3, 5)
    rel = r["rel"].cpu().numpy()
    halt = r["halt"].cpu().numpy()
    assert rel[1] == 0 and halt[1] == 1            # no change
    assert np.isposinf(rel[2]) and halt[2] == 0     # change from a zero state
    assert rel[3] == 0 and halt[3] == 1             # both zero
    r2 = bd.loop_halt(dev(hp), dev(hc), 5, 1e-3, 5, want_rel=False)
    assert r2["rel"] is None and np.all(r2["halt"].cpu().numpy() == 1)   # budget reached


def test_halt_full_size_sampled():
    """32 sequences x 1024 positions x 4096 hidden units (bf16), the size the bench times; the
    oracle checks a sample of sequences one by one."""
    B, n = 32, 1024 * 4096
    scales = np.geomspace(1e-4, 1e-1, B)
    print(f"[halt] full B={B} n={n}", flush=True)
    hp, hc = I.loop_states(799, B, n, scales, True)
    r = bd.loop_halt(dev_bf16(hp), dev_bf16(hc), 3, 2e-3, 12)
    torch.cuda.synchronize()
    rel = r["rel"].cpu().numpy().astype(np.float64)
    halt = r["halt"].cpu().numpy()
    for b in (0, 9, 17, 31):
        ref_rel, ref_halt = O.loop_halt(bf16_f64(hp[b:b + 1]), bf16_f64(hc[b:b + 1]), 2e-3, 3, 12)
        check(rel[b:b + 1], halt[b:b + 1], ref_rel, ref_halt, 2e-3, f"seq {b}")
