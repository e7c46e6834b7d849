"""Helpers shared by the GPU parity tests (device transfer, tolerances, guard canaries)."""
import numpy as np
import torch

ATOL = 2e-2      # attention: max-abs bound (bf16 in, fp32 accumulate)
RTOL_L2 = 1e-2   # attention: relative L2 bound
# LSE: the kernel sums the bf16-rounded probabilities it also feeds to the P V product, so the
# sum carries at most the bf16 unit roundoff 2^-9 relative -> |d LSE| <= ln(1 + 2^-9) ~ 1.95e-3,
# plus float32 accumulation.
LSE_ATOL = 2.5e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bf16 device tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Max-abs and relative-L2 bounds over the whole tensor, and the relative-L2 bound on every
    output row (the last axis) on its own: with long prefixes an output row is a tiny weighted
    mean of the values, so an error confined to a few rows would pass the whole-tensor bounds."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= ATOL, f"{what}: max-abs {err.max():.3e} > {ATOL}"
    assert rel <= RTOL_L2, f"{what}: rel-L2 {rel:.3e} > {RTOL_L2}"
    d = got.reshape(-1, got.shape[-1]) - ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    row_rel = np.linalg.norm(d, axis=1) / np.maximum(rn, 1e-30)
    worst = int(np.argmax(row_rel))
    assert row_rel[worst] <= RTOL_L2, f"{what}: row {worst} rel-L2 {row_rel[worst]:.3e} > {RTOL_L2}"
    return err.max(), rel


def oracle_attn_all(inp, causal=False, active=None):
    """The oracle's output and LSE for EVERY (b, s, h) of the inputs (bf16 bit arrays), computed by
    attn_rows one (sequence, KV head) slab at a time (memory bounded at full size). Rows of
    inactive sequences are NaN."""
    from oracle import bd_oracle as O
    q = inp["q"]
    B, S, Hq, D = q.shape
    rows = [(b, s, h) for b in range(B) if active is None or active[b] for s in range(S) for h in range(Hq)]
    res = O.attn_rows(q, inp["k_blk"], inp["v_blk"], inp["k_cache"], inp["v_cache"], inp["prefix_len"], rows,
                      causal=causal)
    out = np.full((B, S, Hq, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    for (b, s, h), (o, l) in res.items():
        out[b, s, h] = o
        lse[b, h, s] = l
    return out, lse


def guarded(shape, dtype, guard=64, fill=None):
    """A device tensor view with canary regions before and after it (all inside one allocation)."""
    n = int(np.prod(shape))
    big = torch.empty(n + 2 * guard, dtype=dtype, device="cuda")
    if dtype == torch.bfloat16:
        big.view(torch.int16).fill_(0x7F81)   # a NaN pattern
    elif dtype == torch.float32:
        big.fill_(float("nan"))
    else:
        big.fill_(-77 if dtype != torch.uint8 else 0xA5)
    view = big[guard:guard + n].view(shape)
    if fill is not None:
        view.copy_(fill)
    return big, view, guard


def guards_intact(big: torch.Tensor, guard: int, n: int, ref_big_before: torch.Tensor) -> bool:
    a = big.view(torch.uint8) if big.dtype != torch.uint8 else big
    b = ref_big_before.view(torch.uint8) if ref_big_before.dtype != torch.uint8 else ref_big_before
    esz = big.element_size()
    lo = slice(0, guard * esz)
    hi = slice((guard + n) * esz, None)
    return bool(torch.equal(a[lo], b[lo]) and torch.equal(a[hi], b[hi]))
