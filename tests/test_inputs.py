"""The seeded input generator: determinism, bf16 rounding, the planted structure, and the
margin check on every official seed (no commit decision may sit inside float32 rounding)."""
import numpy as np
import pytest

from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O


def test_bf16_round_to_nearest_even_patterns():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)           # bf16 spacing at 1.0
    cases = {
        one: 0x3F80,
        one + ulp / 2: 0x3F80,            # exact tie -> even (mantissa ...0)
        one + ulp + ulp / 2: 0x3F82,      # exact tie -> even (round up to ...2)
        one + ulp / 2 + np.float32(2.0 ** -20): 0x3F81,   # just above the tie -> up
        np.float32(-2.5): 0xC020,
        np.float32(3.0e38): 0x7F62,
        np.float32(0.0): 0x0000,
    }
    got = I.f32_to_bf16_bits(np.array(list(cases.keys()), dtype=np.float32))
    np.testing.assert_array_equal(got, np.array(list(cases.values()), dtype=np.uint16))
    back = I.bf16_bits_to_f32(got)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(back), got)


def test_deterministic_and_distinct_streams():
    w = I.WORKLOADS["tiny"]
    a = I.attn_inputs(w)
    b = I.attn_inputs(w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["q"][0, 0], a["k_blk"][0, 0, :2].reshape(-1)[: a["q"].shape[-1]])
    np.testing.assert_array_equal(I.logits(w), I.logits(w))
    s1 = I.attn_inputs(I.WORKLOADS["tiny"], step=1, cache=False)
    assert not np.array_equal(s1["q"], a["q"])


def test_shapes_and_statistics():
    w = I.WORKLOADS["tiny"]
    a = I.attn_inputs(w)
    assert a["q"].shape == (1, 16, 8, 64) and a["k_cache"].shape == (1, 2, 256, 64)
    x = I.bf16_bits_to_f32(a["k_cache"]).astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    lg = I.logits(w)
    assert lg.dtype == np.float32 and lg.shape == (16, 4096)
    assert abs(lg.std() - 2.0) < 0.02
    m = I.initial_mask(w)
    assert m.sum() == 8


def test_ragged_lengths_and_zero_tail():
    w = I.small_workload(B=5, prefix_len=(3, 40), wid=7)
    lens = I.prefix_lengths(w)
    assert lens.min() >= 3 and lens.max() <= 40
    a = I.attn_inputs(w)
    for b in range(5):
        assert np.all(a["k_cache"][b, :, lens[b]:] == 0)
        assert np.any(a["k_cache"][b, :, : lens[b]] != 0)
    lb = I.prefix_lengths(I.WORKLOADS["stress_b"])
    assert lb.min() >= 1024 and lb.max() <= 32768 and len(set(lb.tolist())) > 8


def test_mask_fraction_rule():
    w = I.WORKLOADS["batched16"]
    m = I.initial_mask(w).reshape(w.B, w.S)
    counts = m.sum(axis=1)
    assert counts.min() >= 4 and counts.max() <= 16 and len(set(counts.tolist())) > 3


def test_planted_peaks_ties_and_fallback_pair():
    w = I.small_workload(B=4, S=8, V=3000, logits_dtype="bf16", sigma=3.0, ties=True, mask_rule="frac", wid=9)
    x = I.bf16_bits_to_f32(I.logits(w)).astype(np.float64)
    mask = I.initial_mask(w).reshape(4, 8)
    # peaked rows: max is 8 above the rest (rows of sequence 0 carry no peak)
    gaps = []
    for r in range(8, 32):
        srt = np.sort(x[r])[::-1]
        gaps.append(srt[0] - srt[1])
    assert sum(g > 7 for g in gaps) >= 6
    # exact ties exist
    ntie = sum(int((x[r] == x[r].max()).sum() >= 2) for r in range(32))
    assert ntie >= 4
    # fallback pair in sequence 0: first and last masked rows are identical
    ms = np.flatnonzero(mask[0])
    if ms.size >= 2:
        np.testing.assert_array_equal(x[ms[0]], x[ms[-1]])


def test_additive_peak_recipe_is_distinct():
    w = I.WORKLOADS["tiny"]
    w2 = I.small_workload(B=1, S=16, V=4096, peaks=True, wid=0)
    a = I.logits(w2)
    b = I.logits(w2, additive_peaks=True)
    assert not np.array_equal(a, b)


def _check_no_near_ties(w, steps=1):
    dec = O.bf16_to_f64 if w.logits_dtype == "bf16" else None
    mask = I.initial_mask(w)
    tokens = np.zeros(w.B * w.S, np.int32)
    for t in range(steps):
        if not mask.any():
            break
        lg = I.logits(w, step=t)
        ca = steps > 1 and t == steps - 1
        p, a = O.confidences(lg, mask, dec)
        nt = O.near_ties(p, mask, w.S, w.gamma, True, ca)
        assert not nt, f"{w.name} step {t}: near-ties {nt[:5]}"
        mask, tokens, _ = O.commit(p, a, mask, tokens, w.S, w.gamma, True, ca)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["tiny", "decode", "batched16", "batched32", "stress_a", "stress_b", "long"])
def test_official_seeds_have_no_near_ties(name):
    w = I.WORKLOADS[name]
    _check_no_near_ties(w, steps=w.T)
