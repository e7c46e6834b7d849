"""Pins of the oracle's block-local bidirectional Mamba scan (BDLM Mamba-H) against things other
than itself.

The page fixes the structure, not the recurrence: completed prefix blocks keep the forward scan's
boundary state, the reverse scan runs inside the active block only, and the cached prefix state is
a function of the clean prefix alone. Pins: a pure-Python scalar brute force on tiny shapes; the
closed (matrix) form of the same linear recurrences, written with decay matrices instead of a
scan; closed forms (no decay, no input, one position); and the page's three properties -- the
state at the block start is the cached boundary state, prefix outputs and boundary states do not
depend on the active block, the reverse scan sees nothing outside the block.
``test_planted_mistakes_are_caught`` swaps in plausible slips and checks that a pin fails."""
import math

import numpy as np
import pytest

from oracle import bd_oracle as O


def inputs(B=2, S=4, H=4, G=2, N=5, P=3, seed=0, L=None):
    """Random float64 inputs of one block (or of a sequence of L positions)."""
    rng = np.random.default_rng(seed)
    n = S if L is None else L

    def side():
        return {"x": rng.standard_normal((B, n, H, P)), "dt": rng.uniform(0.05, 1.2, (B, n, H)),
                "Bm": rng.standard_normal((B, n, G, N)), "Cm": rng.standard_normal((B, n, G, N))}
    return {"h0": rng.standard_normal((B, H, N, P)), "fwd": side(), "rev": side(),
            "A": -rng.uniform(0.2, 2.0, H), "A_r": -rng.uniform(0.2, 2.0, H), "D": rng.standard_normal(H)}


def run(c):
    return O.mamba_block_scan(c["h0"], c["fwd"], c["rev"], c["A"], c["A_r"], c["D"])


def test_mamba_scalar_brute_force():
    """Every state element and output as scalar Python arithmetic, position by position."""
    c = inputs(B=1, S=3, H=2, G=1, N=2, P=2, seed=1)
    y, h_out = run(c)
    f, r = c["fwd"], c["rev"]
    for h in range(2):
        F = [[float(c["h0"][0, h, n, p]) for p in range(2)] for n in range(2)]
        yy = [[0.0, 0.0] for _ in range(3)]
        for s in range(3):
            a = math.exp(float(f["dt"][0, s, h]) * float(c["A"][h]))
            for n in range(2):
                for p in range(2):
                    F[n][p] = a * F[n][p] + float(f["dt"][0, s, h]) * float(f["Bm"][0, s, 0, n]) * float(f["x"][0, s, h, p])
            for p in range(2):
                yy[s][p] += sum(float(f["Cm"][0, s, 0, n]) * F[n][p] for n in range(2))
        for n in range(2):
            for p in range(2):
                assert abs(h_out[0, h, n, p] - F[n][p]) < 1e-12
        R = [[0.0, 0.0] for _ in range(2)]
        for s in (2, 1, 0):
            a = math.exp(float(r["dt"][0, s, h]) * float(c["A_r"][h]))
            for n in range(2):
                for p in range(2):
                    R[n][p] = a * R[n][p] + float(r["dt"][0, s, h]) * float(r["Bm"][0, s, 0, n]) * float(r["x"][0, s, h, p])
            for p in range(2):
                yy[s][p] += sum(float(r["Cm"][0, s, 0, n]) * R[n][p] for n in range(2))
        for s in range(3):
            for p in range(2):
                assert abs(y[0, s, h, p] - (yy[s][p] + float(c["D"][h]) * float(f["x"][0, s, h, p]))) < 1e-12


def matrix_form(c):
    """The same linear recurrences solved in closed form: with cum_s = sum_{k<=s} dt_k,
    yf_s = exp(A cum_s) C_s^T h0 + sum_{j<=s} exp(A (cum_s - cum_j)) dt_j (C_s . B_j) x_j,
    yr_s = sum_{j>=s} exp(A_r sum_{k=s}^{j-1} dtr_k) dtr_j (Cr_s . Br_j) xr_j,
    h_out = exp(A cum_{S-1}) h0 + sum_j exp(A (cum_{S-1} - cum_j)) dt_j B_j x_j^T."""
    f, r = c["fwd"], c["rev"]
    B, S, H, P = f["x"].shape
    G = f["Bm"].shape[2]
    y = np.zeros((B, S, H, P))
    h_out = np.zeros_like(c["h0"])
    for b in range(B):
        for h in range(H):
            g = h * G // H
            cum = np.cumsum(f["dt"][b, :, h])
            Cg, Bg = f["Cm"][b, :, g], f["Bm"][b, :, g]                   # [S, N]
            Lf = np.tril(np.exp(c["A"][h] * (cum[:, None] - cum[None, :])))
            Mf = Lf * (Cg @ Bg.T) * f["dt"][b, :, h][None, :]
            yf = np.exp(c["A"][h] * cum)[:, None] * (Cg @ c["h0"][b, h]) + Mf @ f["x"][b, :, h]
            w = np.exp(c["A"][h] * (cum[-1] - cum)) * f["dt"][b, :, h]
            h_out[b, h] = np.exp(c["A"][h] * cum[-1]) * c["h0"][b, h] + (Bg * w[:, None]).T @ f["x"][b, :, h]
            cr = np.concatenate([[0.0], np.cumsum(r["dt"][b, :, h])])     # cr[s] = sum_{k<s} dtr_k
            Cr, Br = r["Cm"][b, :, g], r["Bm"][b, :, g]
            Lr = np.triu(np.exp(c["A_r"][h] * (cr[None, :-1] - cr[:-1, None])))   # [s, j]: sum_{k=s}^{j-1}
            Mr = Lr * (Cr @ Br.T) * r["dt"][b, :, h][None, :]
            y[b, :, h] = yf + Mr @ r["x"][b, :, h] + c["D"][h] * f["x"][b, :, h]
    return y, h_out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mamba_matches_the_matrix_form(seed):
    c = inputs(B=2, S=7, H=6, G=3, N=5, P=4, seed=10 + seed)
    y, h_out = run(c)
    ym, hm = matrix_form(c)
    np.testing.assert_allclose(y, ym, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(h_out, hm, rtol=1e-10, atol=1e-10)


def test_mamba_closed_forms():
    # no decay and unit steps: the forward state is h0 plus the running sum of B_j x_j^T
    c = inputs(B=1, S=5, H=2, G=1, N=3, P=2, seed=3)
    c["A"] = np.zeros(2)
    c["fwd"]["dt"] = np.ones((1, 5, 2))
    c["rev"]["x"] = np.zeros_like(c["rev"]["x"])
    c["D"] = np.zeros(2)
    y, h_out = run(c)
    f = c["fwd"]
    for h in range(2):
        Fs = c["h0"][0, h] + np.cumsum(f["Bm"][0, :, 0, :, None] * f["x"][0, :, h, None, :], axis=0)
        np.testing.assert_allclose(y[0, :, h], np.einsum("sn,snp->sp", f["Cm"][0, :, 0], Fs), rtol=1e-12)
        np.testing.assert_allclose(h_out[0, h], Fs[-1], rtol=1e-12)
    # no input at all: the cached state decays, the reverse scan contributes nothing
    c = inputs(B=1, S=4, H=2, G=2, N=3, P=2, seed=4)
    for side in ("fwd", "rev"):
        c[side]["x"] = np.zeros_like(c[side]["x"])
    y, h_out = run(c)
    for h in range(2):
        cum = np.cumsum(c["fwd"]["dt"][0, :, h])
        expect = np.exp(c["A"][h] * cum)[:, None] * (c["fwd"]["Cm"][0, :, h] @ c["h0"][0, h])
        np.testing.assert_allclose(y[0, :, h], expect, rtol=1e-12)
        np.testing.assert_allclose(h_out[0, h], np.exp(c["A"][h] * cum[-1]) * c["h0"][0, h], rtol=1e-12)
    # one position: y = C^T (a h0 + dt B x^T) + Cr^T (dtr Br xr^T) + D x
    c = inputs(B=1, S=1, H=1, G=1, N=4, P=3, seed=5)
    y, _ = run(c)
    f, r = c["fwd"], c["rev"]
    Fs = math.exp(f["dt"][0, 0, 0] * c["A"][0]) * c["h0"][0, 0] + f["dt"][0, 0, 0] * np.outer(f["Bm"][0, 0, 0], f["x"][0, 0, 0])
    Rs = r["dt"][0, 0, 0] * np.outer(r["Bm"][0, 0, 0], r["x"][0, 0, 0])
    np.testing.assert_allclose(y[0, 0, 0], f["Cm"][0, 0, 0] @ Fs + r["Cm"][0, 0, 0] @ Rs + c["D"][0] * f["x"][0, 0, 0],
                               rtol=1e-12)


def test_mamba_block_from_the_cached_boundary_state():
    """Scanning a sequence of three blocks and recomputing any block from the forward state the
    previous blocks left (the cache entry) gives the same outputs: the state at the block start is
    the cached boundary state."""
    S = 4
    c = inputs(B=2, H=4, G=2, N=5, P=3, seed=6, L=3 * S)
    y, bounds = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)
    for k in range(3):
        h0 = np.zeros_like(bounds[:, 0]) if k == 0 else bounds[:, k - 1]
        sl = slice(k * S, (k + 1) * S)
        yk, hk = O.mamba_block_scan(h0, {n: v[:, sl] for n, v in c["fwd"].items()},
                                    {n: v[:, sl] for n, v in c["rev"].items()}, c["A"], c["A_r"], c["D"])
        np.testing.assert_allclose(yk, y[:, sl], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hk, bounds[:, k], rtol=1e-12, atol=1e-12)
    # the boundary state equals one forward recurrence over the whole prefix (no reverse part)
    f = c["fwd"]
    Fz = np.zeros((2, 4, 5, 3))
    for s in range(2 * S):
        for h in range(4):
            g = h * 2 // 4
            Fz[:, h] = np.exp(f["dt"][:, s, h] * c["A"][h])[:, None, None] * Fz[:, h] + \
                f["dt"][:, s, h][:, None, None] * f["Bm"][:, s, g][:, :, None] * f["x"][:, s, h][:, None, :]
    np.testing.assert_allclose(bounds[:, 1], Fz, rtol=1e-12, atol=1e-12)


def test_mamba_prefix_does_not_depend_on_the_active_block():
    """Every input of the last (active) block redrawn: the outputs of the prefix blocks and the
    boundary states they leave are bit-identical, the active block's outputs change."""
    S = 4
    c = inputs(B=1, H=2, G=1, N=3, P=2, seed=7, L=3 * S)
    y, bounds = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)
    d = inputs(B=1, H=2, G=1, N=3, P=2, seed=8, L=3 * S)
    for side in ("fwd", "rev"):
        for n in c[side]:
            c[side][n][:, 2 * S:] = d[side][n][:, 2 * S:]
    y2, bounds2 = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)
    np.testing.assert_array_equal(y2[:, :2 * S], y[:, :2 * S])
    np.testing.assert_array_equal(bounds2[:, :2], bounds[:, :2])
    assert np.abs(y2[:, 2 * S:] - y[:, 2 * S:]).max() > 1e-3


def test_mamba_reverse_scan_stays_in_the_block():
    """Reverse inputs of the other blocks redrawn: a block's outputs are unchanged. A reverse scan
    over the whole window (the full-sequence bidirectional baseline) gives different outputs, so
    the confinement is what the pin checks."""
    S = 4
    c = inputs(B=1, H=2, G=2, N=3, P=2, seed=9, L=3 * S)
    y, _ = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)
    d = inputs(B=1, H=2, G=2, N=3, P=2, seed=10, L=3 * S)
    for n in c["rev"]:
        c["rev"][n][:, :S] = d["rev"][n][:, :S]
        c["rev"][n][:, 2 * S:] = d["rev"][n][:, 2 * S:]
    y2, _ = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)
    np.testing.assert_array_equal(y2[:, S:2 * S], y[:, S:2 * S])
    # the full-window reverse scan for comparison: block 1's outputs then see block 2's inputs
    r = c["rev"]
    R = np.zeros((1, 2, 3, 2))
    yr_full = np.zeros((1, 3 * S, 2, 2))
    for s in range(3 * S - 1, -1, -1):
        for h in range(2):
            R[:, h] = np.exp(r["dt"][:, s, h] * c["A_r"][h])[:, None, None] * R[:, h] + \
                r["dt"][:, s, h][:, None, None] * r["Bm"][:, s, h][:, :, None] * r["x"][:, s, h][:, None, :]
            yr_full[:, s, h] = np.einsum("bn,bnp->bp", r["Cm"][:, s, h], R[:, h])
    y_loc = O.mamba_sequence(c["fwd"], c["rev"], c["A"], c["A_r"], c["D"], S)[0]
    y_nr = O.mamba_sequence(c["fwd"], {n: (v * 0 if n == "x" else v) for n, v in r.items()}, c["A"], c["A_r"],
                            c["D"], S)[0]
    assert np.abs((y_nr + yr_full)[:, S:2 * S] - y_loc[:, S:2 * S]).max() > 1e-3


def slipped_scan(kind):
    """The forward/reverse recurrences with one plausible slip."""
    def scan(h0, fwd, rev, A, A_r, D_skip):
        B, S, H, P = fwd["x"].shape
        G = fwd["Bm"].shape[2]
        y = np.zeros((B, S, H, P))
        h_out = np.zeros(np.shape(h0))
        for b in range(B):
            for h in range(H):
                g = h % G if kind == "group" else h * G // H
                F = np.array(h0[b, h], dtype=np.float64)
                prev = F
                for s in range(S):
                    a = np.exp(fwd["dt"][b, s, h] * A[h])
                    u = (1.0 if kind == "no_dt" else fwd["dt"][b, s, h]) * np.outer(fwd["Bm"][b, s, g], fwd["x"][b, s, h])
                    prev = F
                    F = a * (F + u) if kind == "decay_after" else a * F + u
                    y[b, s, h] += fwd["Cm"][b, s, g] @ (prev if kind == "old_state" else F)
                h_out[b, h] = prev if kind == "h_out_early" else F
                R = np.zeros_like(F)
                order = range(S) if kind == "rev_order" else range(S - 1, -1, -1)
                for s in order:
                    R = np.exp(rev["dt"][b, s, h] * A_r[h]) * R + rev["dt"][b, s, h] * np.outer(rev["Bm"][b, s, g],
                                                                                                 rev["x"][b, s, h])
                    y[b, s, h] += rev["Cm"][b, s, g] @ R
                if kind != "no_skip":
                    y[b, :, h] += D_skip[h] * fwd["x"][b, :, h]
        return y, h_out
    return scan


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    orig = O.mamba_block_scan
    pins = [(test_mamba_scalar_brute_force,), (test_mamba_matches_the_matrix_form, 0), (test_mamba_closed_forms,)]
    for kind in ("group", "no_dt", "decay_after", "old_state", "h_out_early", "rev_order", "no_skip"):
        monkeypatch.setattr(O, "mamba_block_scan", slipped_scan(kind))
        with np.errstate(all="ignore"):
            assert any(_fails(*p) for p in pins), f"no pin caught the slip {kind}"
        monkeypatch.setattr(O, "mamba_block_scan", orig)
    # a sequence scan that carries the reverse state across blocks (the reverse scan not confined)
    orig_seq = O.mamba_sequence

    def unconfined(fwd, rev, A, A_r, D_skip, S, h_init=None):
        L = fwd["x"].shape[1]
        return orig_seq(fwd, rev, A, A_r, D_skip, L, h_init)[0], orig_seq(fwd, rev, A, A_r, D_skip, S, h_init)[1]
    monkeypatch.setattr(O, "mamba_sequence", unconfined)
    assert _fails(test_mamba_reverse_scan_stays_in_the_block) or _fails(test_mamba_block_from_the_cached_boundary_state)
    monkeypatch.setattr(O, "mamba_sequence", orig_seq)
