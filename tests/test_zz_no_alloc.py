"""GPU test of bd_confidence_unmask_noalloc -- the allocation-free variant of
bd_confidence_unmask whose slice partials live in the library's static per-device scratch --
called through the C ABI and compared with bd_confidence_unmask (caller workspace) on the same
inputs: two calls in a row, the second with a smaller problem (so the second call finds the first
call's partials in the shared scratch). Masks, tokens, argmax ids, confidences and commit counts
must be identical (the same kernels run on the same bytes), and both must match the float64
oracle's decisions."""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_lm_amd import _lib
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import dev, dev_bf16

pytestmark = pytest.mark.gpu


def _call(L, noalloc, w, logits_d, mask_h, tokens_h):
    is_bf16 = w.logits_dtype == "bf16"
    rows = w.B * w.S
    desc = _lib.UnmaskDesc(w.B, w.S, w.V, w.V, _lib.BD_BF16 if is_bf16 else _lib.BD_F32, w.gamma, 1, 0)
    mask = dev(mask_h.copy())
    tokens = dev(tokens_h.copy())
    conf = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda")
    argmax = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    nc = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = L.bd_confidence_unmask_noalloc(ctypes.byref(desc), logits_d.data_ptr(), mask.data_ptr(),
                                            tokens.data_ptr(), conf.data_ptr(), argmax.data_ptr(), nc.data_ptr(),
                                            stream)
    else:
        nbytes = L.bd_unmask_workspace_bytes(ctypes.byref(desc))
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        st = L.bd_confidence_unmask(ctypes.byref(desc), logits_d.data_ptr(), mask.data_ptr(), tokens.data_ptr(),
                                    conf.data_ptr(), argmax.data_ptr(), nc.data_ptr(), ws.data_ptr(), nbytes,
                                    stream)
    assert st == _lib.BD_OK, L.bd_last_error()
    torch.cuda.synchronize()
    return {"mask": mask.cpu().numpy(), "tokens": tokens.cpu().numpy(), "conf": conf.cpu().numpy(),
            "argmax": argmax.cpu().numpy(), "n_commit": nc.cpu().numpy()}


def test_noalloc_matches_workspace_entry_point_twice():
    L = _lib.load()
    # first the batched workload (512 rows of 131072 bf16 logits), then the tiny one (16 rows of
    # 4096 float32 logits): the second call is smaller and reuses the scratch the first one filled
    for name in ("batched16", "tiny"):
        w = I.WORKLOADS[name]
        print(f"[noalloc] {name}", flush=True)
        lg = I.logits(w)
        mask = I.initial_mask(w)
        tokens = np.full(w.B * w.S, -5, np.int32)
        is_bf16 = w.logits_dtype == "bf16"
        lg_d = dev_bf16(lg) if is_bf16 else dev(lg)
        got = _call(L, True, w, lg_d, mask, tokens)
        ref_ws = _call(L, False, w, lg_d, mask, tokens)
        for k in ("mask", "tokens", "argmax", "n_commit"):
            np.testing.assert_array_equal(got[k], ref_ws[k], err_msg=f"{name}: {k}")
        np.testing.assert_array_equal(got["conf"].view(np.uint32), ref_ws["conf"].view(np.uint32))
        ref = O.confidence_unmask(lg, mask, tokens, w.S, w.gamma, True, False,
                                  decode=O.bf16_to_f64 if is_bf16 else None)
        assert not O.near_ties(ref["conf"], mask, w.S, w.gamma, True, False)
        for k in ("mask", "tokens", "argmax", "n_commit"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{name}: {k} vs oracle")
        np.testing.assert_allclose(got["conf"], ref["conf"], rtol=2e-5, atol=1e-30)
        del lg_d
