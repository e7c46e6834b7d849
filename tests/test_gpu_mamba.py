"""GPU parity of bd_mamba_block_scan (the block-local bidirectional Mamba scan) against the
float64 oracle, through the C ABI.

The output y is bf16 and, unlike an attention output, not bounded by the values' magnitude (a sum
of up to N + 2 S products): every element must lie within 2^-8 of |ref| (the bf16 rounding of the
result, half an ulp being at most 2^-8 relative) plus 2e-3 absolute (float32 sums of a few hundred
terms of magnitude ~1 and the float32 exponentials, with a wide margin), and the relative L2 error
of the tensor and of every output row must stay below 1e-2. The boundary state h_out is float32 computed from float32 products (the closed form
of the recurrence on float32 MFMA, exponentials by expf): it must match the oracle's float64
recurrence to 1e-4 of its largest magnitude (derivation: 2^-24 per product and sum over at most
N + S terms, and a few ulp of the decay factors, far below that bound)."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import RTOL_L2, dev, dev_bf16, guarded, guards_intact, host_f64

pytestmark = pytest.mark.gpu


def f64(side):
    return {"x": O.bf16_to_f64(side["x"]), "dt": side["dt"].astype(np.float64),
            "Bm": O.bf16_to_f64(side["Bm"]), "Cm": O.bf16_to_f64(side["Cm"])}


def run_gpu(inp, active=None, want_h_out=True):
    def dside(sd):
        return (dev_bf16(sd["x"]), dev(sd["dt"]), dev_bf16(sd["Bm"]), dev_bf16(sd["Cm"]))
    h0 = dev(inp["h0"])
    h0_before = h0.clone()
    y, h_out = bd.mamba_block_scan(h0, dside(inp["fwd"]), dside(inp["rev"]), dev(inp["fwd"]["A"]), dev(inp["rev"]["A"]),
                                   dev(inp["D"]), active=None if active is None else dev(active), want_h_out=want_h_out)
    torch.cuda.synchronize()
    assert torch.equal(h0, h0_before), "h0 was written"
    return y, h_out


Y_RTOL = 2.0 ** -8
Y_ATOL = 2e-3


def assert_y_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (Y_RTOL * np.abs(ref) + Y_ATOL)
    worst = np.unravel_index(int(np.argmax(excess)), got.shape)
    assert excess[worst] <= 0, f"{what}: at {worst} got {got[worst]:.6g} ref {ref[worst]:.6g}"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= RTOL_L2, f"{what}: rel-L2 {rel:.3e}"
    d = (got - ref).reshape(-1, got.shape[-1])
    row_rel = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1), 1e-30)
    assert row_rel.max() <= RTOL_L2, f"{what}: row {int(np.argmax(row_rel))} rel-L2 {row_rel.max():.3e}"


def check(inp, y, h_out, active=None):
    ref_y, ref_h = O.mamba_block_scan(inp["h0"].astype(np.float64), f64(inp["fwd"]), f64(inp["rev"]),
                                      inp["fwd"]["A"].astype(np.float64), inp["rev"]["A"].astype(np.float64),
                                      inp["D"].astype(np.float64))
    sel = slice(None) if active is None else (np.asarray(active) == 1)
    assert_y_close(host_f64(y)[sel], ref_y[sel], "mamba y")
    if h_out is not None:
        got = h_out.cpu().numpy().astype(np.float64)[sel]
        err = np.abs(got - ref_h[sel]).max()
        assert err <= 1e-4 * np.abs(ref_h[sel]).max(), f"h_out max-abs {err:.3e}"


CASES = [
    # name, B, S, H, G, N
    ("S16-N128", 2, 16, 8, 2, 128),
    ("S1", 3, 1, 4, 1, 128),
    ("S17-padded", 2, 17, 4, 4, 128),
    ("S32-N64", 2, 32, 6, 3, 64),
    ("S5-N64-G1", 1, 5, 8, 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mamba_matches_oracle(case):
    name, B, S, H, G, N = case
    inp = I.mamba_inputs(500 + CASES.index(case), B, S, H, G, N)
    print(f"[mamba] {name}", flush=True)
    y, h_out = run_gpu(inp)
    check(inp, y, h_out)


def test_mamba_full_size():
    """The measured shape: 32 sequences x 64 heads x P 64, N 128, 8 groups, S 16."""
    inp = I.mamba_inputs(510, 32, 16, 64, 8, 128)
    print("[mamba] full size", flush=True)
    y, h_out = run_gpu(inp)
    check(inp, y, h_out)


def test_mamba_inactive_sequences_and_no_h_out():
    inp = I.mamba_inputs(511, 3, 16, 4, 2, 128)
    act = np.array([1, 0, 1], np.uint8)

    def dside(sd):
        return (dev_bf16(sd["x"]), dev(sd["dt"]), dev_bf16(sd["Bm"]), dev_bf16(sd["Cm"]))
    big, y, gd = guarded((3, 16, 4, 64), torch.bfloat16)
    hbig, h_out, hg = guarded((3, 4, 128, 64), torch.float32)
    b0, hb0 = big.clone(), hbig.clone()
    bd.mamba_block_scan(dev(inp["h0"]), dside(inp["fwd"]), dside(inp["rev"]), dev(inp["fwd"]["A"]), dev(inp["rev"]["A"]),
                        dev(inp["D"]), active=dev(act), y=y, h_out=h_out)
    torch.cuda.synchronize()
    assert guards_intact(big, gd, y.numel(), b0) and guards_intact(hbig, hg, h_out.numel(), hb0)
    assert torch.equal(y[1].view(torch.int16), b0[gd:gd + y.numel()].view(y.shape)[1].view(torch.int16))
    assert torch.equal(h_out[1].view(torch.int32), hb0[hg:hg + h_out.numel()].view(h_out.shape)[1].view(torch.int32))
    check(inp, y, h_out, active=act)
    y2, none = run_gpu(inp, want_h_out=False)
    assert none is None
    sel = torch.from_numpy(act == 1).cuda()
    assert torch.equal(y2[sel].view(torch.int16), y[sel].view(torch.int16))


@pytest.mark.parametrize("B", [40, 70], ids=["ballot-40", "direct-70"])
def test_mamba_scattered_active_sequences(B):
    """A scattered active mask: up to 64 sequences the work-groups take the active ones in order
    (one ballot per wave), beyond that they map directly; active sequences match the oracle,
    retired ones keep y and h_out as they were."""
    inp = I.mamba_inputs(520 + B, B, 16, 8, 2, 64)
    act = (np.random.default_rng(521 + B).random(B) < 0.35).astype(np.uint8)
    act[0], act[-1] = 0, 1

    def dside(sd):
        return (dev_bf16(sd["x"]), dev(sd["dt"]), dev_bf16(sd["Bm"]), dev_bf16(sd["Cm"]))
    y = torch.full((B, 16, 8, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    h_out = torch.full((B, 8, 64, 64), -7.0, dtype=torch.float32, device="cuda")
    y0, h0c = y.clone(), h_out.clone()
    print(f"[mamba] scattered active B={B} active={int(act.sum())}", flush=True)
    bd.mamba_block_scan(dev(inp["h0"]), dside(inp["fwd"]), dside(inp["rev"]), dev(inp["fwd"]["A"]), dev(inp["rev"]["A"]),
                        dev(inp["D"]), active=dev(act), y=y, h_out=h_out)
    torch.cuda.synchronize()
    off = torch.from_numpy(act == 0).cuda()
    assert torch.equal(y[off].view(torch.int16), y0[off].view(torch.int16))
    assert torch.equal(h_out[off], h0c[off])
    check(inp, y, h_out, active=act)


def test_mamba_in_place_state_update():
    """h_out = h0: the cache entry advanced in place gives the out-of-place results bit for bit."""
    inp = I.mamba_inputs(514, 4, 16, 16, 4, 128)
    y_ref, h_ref = run_gpu(inp)

    def dside(sd):
        return (dev_bf16(sd["x"]), dev(sd["dt"]), dev_bf16(sd["Bm"]), dev_bf16(sd["Cm"]))
    h = dev(inp["h0"])
    y, h_out = bd.mamba_block_scan(h, dside(inp["fwd"]), dside(inp["rev"]), dev(inp["fwd"]["A"]), dev(inp["rev"]["A"]),
                                   dev(inp["D"]), h_out=h)
    torch.cuda.synchronize()
    assert h_out.data_ptr() == h.data_ptr()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(h.view(torch.int32), h_ref.view(torch.int32))


def test_mamba_committed_block_chains():
    """Two blocks in a row: the second starts from the h_out of the first (the cache entry after a
    commit), and matches the oracle's whole-sequence scan of both blocks."""
    B, S, H, G, N = 2, 16, 4, 2, 128
    i1 = I.mamba_inputs(512, B, S, H, G, N)
    i2 = I.mamba_inputs(513, B, S, H, G, N)
    i2["h0"] = np.zeros_like(i2["h0"])
    for k in ("A",):
        i2["fwd"][k], i2["rev"][k] = i1["fwd"][k], i1["rev"][k]
    i2["D"] = i1["D"]
    _, h1 = run_gpu(i1)
    i2g = dict(i2, h0=h1.cpu().numpy())
    y2, _ = run_gpu(i2g)
    seq = {side: {k: np.concatenate([f64(i1[side])[k], f64(i2[side])[k]], axis=1) for k in ("x", "dt", "Bm", "Cm")}
           for side in ("fwd", "rev")}
    ys, _ = O.mamba_sequence(seq["fwd"], seq["rev"], i1["fwd"]["A"].astype(np.float64),
                             i1["rev"]["A"].astype(np.float64), i1["D"].astype(np.float64), S,
                             h_init=i1["h0"].astype(np.float64))
    assert_y_close(host_f64(y2), ys[:, S:], "second block")
