"""Block-diffusion denoise step on MI355X (gfx950): a thin Python binding over libbd.so.

Every step of the path runs in the HIP kernels behind the C ABI (include/bd.h); this module only
marshals torch tensors (device memory) and the current torch stream into those calls. There is
no CPU or PyTorch fallback: a missing library raises.

    attn_step(q, k_blk, v_blk, k_cache, v_cache, prefix_len, ...)  -> (out, lse)
    confidence_unmask(logits, mask, tokens, block_len, gamma, ...)  -> dict
    confidence_unmask_noalloc(...)                  the same without a workspace (static scratch)
    denoise_block(get_qkv, get_logits, k_cache, v_cache, prefix_len, mask, tokens, T, ...) -> dict
    attn_step(..., causal=True)                     context-tower pass over a committed block
    kv_append(k_new, v_new, k_cache, v_cache, prefix_len, ...)  prefix-cache append
    spec_verify(logits, draft, first_choice, block_len, ...)     self-speculation acceptance
    loop_halt(h_prev, h_cur, iteration, eps, max_iter, ...)      adaptive loop halting
    mamba_block_scan(h0, fwd, rev, A, A_r, D, ...)               block-local bidirectional Mamba scan
"""
from __future__ import annotations

import ctypes
from typing import Callable, Optional

from . import _lib
from ._lib import AttnDesc, BdError, HaltDesc, StepHooks, UnmaskDesc  # noqa: F401

__all__ = ["attn_step", "attn_plan", "confidence_unmask", "confidence_unmask_noalloc", "denoise_block", "attn_desc", "unmask_desc", "Trace", "BdError",
           "attn_workspace_bytes", "unmask_workspace_bytes", "denoise_workspace_bytes", "version", "kv_append",
           "spec_verify", "loop_halt", "halt_desc", "loop_halt_workspace_bytes", "mamba_block_scan"]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev_tensor(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def version() -> str:
    return _lib.load().bd_version().decode()


def attn_desc(B, Hq, Hkv, D, S, prefix_capacity, max_prefix_len=None, softmax_scale=0.0, num_splits=0,
              causal=False) -> AttnDesc:
    return AttnDesc(B, Hq, Hkv, D, S, prefix_capacity,
                    prefix_capacity if max_prefix_len is None else max_prefix_len, softmax_scale, num_splits,
                    int(bool(causal)))


def unmask_desc(B, S, V, row_stride=None, bf16=True, gamma=0.9, min_commit=True, commit_all=False) -> UnmaskDesc:
    return UnmaskDesc(B, S, V, V if row_stride is None else row_stride, _lib.BD_BF16 if bf16 else _lib.BD_F32,
                      gamma, int(bool(min_commit)), int(bool(commit_all)))


def attn_plan(desc: AttnDesc) -> dict:
    """bd_attn_plan: how bd_attn_step runs this descriptor (work-group shape, row tiles, chunks)."""
    info = _lib.AttnPlanInfo()
    _lib.check(_lib.load().bd_attn_plan(ctypes.byref(desc), ctypes.byref(info)), "bd_attn_plan")
    return {f: int(getattr(info, f)) for f, _ in _lib.AttnPlanInfo._fields_}


def attn_workspace_bytes(desc: AttnDesc) -> int:
    return int(_lib.load().bd_attn_workspace_bytes(ctypes.byref(desc)))


def unmask_workspace_bytes(desc: UnmaskDesc) -> int:
    return int(_lib.load().bd_unmask_workspace_bytes(ctypes.byref(desc)))


def denoise_workspace_bytes(ad: AttnDesc, ud: UnmaskDesc) -> int:
    return int(_lib.load().bd_denoise_workspace_bytes(ctypes.byref(ad), ctypes.byref(ud)))


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def attn_step(q, k_blk, v_blk, k_cache, v_cache, prefix_len, active=None, out=None, lse=None, want_lse=True,
              max_prefix_len=None, softmax_scale=0.0, num_splits=0, workspace=None, stream=None, causal=False):
    """bd_attn_step on torch tensors. q [B,S,Hq,D], k_blk/v_blk [B,S,Hkv,D], k_cache/v_cache
    [B,Hkv,Lcap,D] (bf16), prefix_len [B] int32, active [B] uint8 or None. Returns (out, lse)."""
    torch = _torch()
    L = _lib.load()
    for t, n in ((q, "q"), (k_blk, "k_blk"), (v_blk, "v_blk"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_tensor(t, n, torch.bfloat16)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    if active is not None:
        _dev_tensor(active, "active", torch.uint8)
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    if k_blk.shape != (B, S, Hkv, D) or v_blk.shape != k_blk.shape:
        raise ValueError("k_blk / v_blk must be [B, S, Hkv, D]")
    if k_cache.shape[0] != B or k_cache.shape[1] != Hkv or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [B, Hkv, Lcap, D]")
    if prefix_len.shape != (B,):
        raise ValueError("prefix_len must be [B]")
    desc = attn_desc(B, Hq, Hkv, D, S, k_cache.shape[2], max_prefix_len, softmax_scale, num_splits, causal)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    nbytes = L.bd_attn_workspace_bytes(ctypes.byref(desc))
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check(L.bd_attn_step(ctypes.byref(desc), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache),
                              _ptr(prefix_len), _ptr(active), _ptr(out), _ptr(lse), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(stream)), "bd_attn_step")
    return out, lse


def kv_append(k_new, v_new, k_cache, v_cache, prefix_len, active=None, max_prefix_len=None, stream=None):
    """bd_kv_append on torch tensors: k_new/v_new [B,S,Hkv,D] bf16 go to cache rows
    prefix_len[b] .. +S-1 of k_cache/v_cache [B,Hkv,Lcap,D]; prefix_len [B] int32 advances by S
    (in place, for active sequences)."""
    torch = _torch()
    L = _lib.load()
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_tensor(t, n, torch.bfloat16)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    if active is not None:
        _dev_tensor(active, "active", torch.uint8)
    B, S, Hkv, D = k_new.shape
    if v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must have the same shape [B, S, Hkv, D]")
    if k_cache.shape[0] != B or k_cache.shape[1] != Hkv or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [B, Hkv, Lcap, D]")
    Lcap = k_cache.shape[2]
    mpl = Lcap - S if max_prefix_len is None else max_prefix_len
    desc = attn_desc(B, Hkv, Hkv, D, S, Lcap, mpl)
    _lib.check(L.bd_kv_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              _ptr(prefix_len), _ptr(active), _stream(stream)), "bd_kv_append")


def spec_verify(logits, draft, first_choice, block_len, vocab=None, tokens=None, n_commit=None, next_choice=None,
                workspace=None, stream=None):
    """bd_spec_verify on torch tensors: logits [B*S, row_stride] (bf16 or float32) of the causal pass
    over the drafted block, draft [B*S] int32, first_choice [B] int32. Returns dict(tokens,
    n_commit, next_choice)."""
    torch = _torch()
    L = _lib.load()
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be bfloat16 or float32")
    _dev_tensor(logits, "logits")
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(first_choice, "first_choice", torch.int32)
    rows, stride = logits.shape
    if rows % block_len != 0 or draft.numel() != rows:
        raise ValueError("logits rows and draft must be B * block_len")
    B = rows // block_len
    if first_choice.numel() != B:
        raise ValueError("first_choice must hold one entry per sequence")
    V = stride if vocab is None else vocab
    desc = unmask_desc(B, block_len, V, stride, bf16=logits.dtype == torch.bfloat16)
    dev = logits.device
    tokens = torch.empty(rows, dtype=torch.int32, device=dev) if tokens is None else tokens
    n_commit = torch.empty(B, dtype=torch.int32, device=dev) if n_commit is None else n_commit
    next_choice = torch.empty(B, dtype=torch.int32, device=dev) if next_choice is None else next_choice
    nbytes = L.bd_unmask_workspace_bytes(ctypes.byref(desc))
    ws = _workspace(nbytes, dev, workspace)
    _lib.check(L.bd_spec_verify(ctypes.byref(desc), _ptr(logits), _ptr(draft), _ptr(first_choice), _ptr(tokens),
                                _ptr(n_commit), _ptr(next_choice), _ptr(ws), ws.numel() if ws is not None else 0,
                                _stream(stream)), "bd_spec_verify")
    return {"tokens": tokens, "n_commit": n_commit, "next_choice": next_choice}


def halt_desc(B, n_per_seq, bf16=True, eps=1e-3, max_iter=8) -> HaltDesc:
    return HaltDesc(B, n_per_seq, _lib.BD_BF16 if bf16 else _lib.BD_F32, eps, max_iter)


def loop_halt_workspace_bytes(desc: HaltDesc) -> int:
    return _lib.load().bd_loop_halt_workspace_bytes(ctypes.byref(desc))


def loop_halt(h_prev, h_cur, iteration, eps, max_iter, rel=None, halt=None, want_rel=True, workspace=None,
              stream=None):
    """bd_loop_halt on torch tensors: h_prev / h_cur [B, ...] (bf16 or float32, same shape) are the
    hidden states after loop iterations iteration-1 and iteration. Returns dict(rel [B] float32 or
    None, halt [B] uint8)."""
    torch = _torch()
    L = _lib.load()
    if h_prev.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("hidden states must be bfloat16 or float32")
    _dev_tensor(h_prev, "h_prev")
    _dev_tensor(h_cur, "h_cur", h_prev.dtype)
    if h_cur.shape != h_prev.shape or h_prev.dim() < 1:
        raise ValueError("h_prev / h_cur must have the same shape [B, ...]")
    B = h_prev.shape[0]
    n = h_prev.numel() // B if B else 0
    desc = halt_desc(B, n, h_prev.dtype == torch.bfloat16, eps, max_iter)
    dev = h_prev.device
    if want_rel and rel is None:
        rel = torch.empty(B, dtype=torch.float32, device=dev)
    halt = torch.empty(B, dtype=torch.uint8, device=dev) if halt is None else halt
    nbytes = L.bd_loop_halt_workspace_bytes(ctypes.byref(desc))
    ws = _workspace(nbytes, dev, workspace)
    _lib.check(L.bd_loop_halt(ctypes.byref(desc), _ptr(h_prev), _ptr(h_cur), int(iteration), _ptr(rel), _ptr(halt),
                              _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)), "bd_loop_halt")
    return {"rel": rel, "halt": halt}


def confidence_unmask(logits, mask, tokens, block_len, gamma, vocab=None, min_commit=True, commit_all=False,
                      outputs=True, workspace=None, stream=None):
    """bd_confidence_unmask on torch tensors. logits [B*S, row_stride] bf16 or float32; mask [B*S]
    uint8 and tokens [B*S] int32 are updated in place. Returns dict(conf, argmax, n_commit)."""
    torch = _torch()
    L = _lib.load()
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be bfloat16 or float32")
    _dev_tensor(logits, "logits")
    _dev_tensor(mask, "mask", torch.uint8)
    _dev_tensor(tokens, "tokens", torch.int32)
    rows, stride = logits.shape
    S = int(block_len)
    if rows % S != 0 or mask.numel() != rows or tokens.numel() != rows:
        raise ValueError("logits rows, mask and tokens must all be B*S")
    B = rows // S
    V = stride if vocab is None else vocab
    desc = unmask_desc(B, S, V, stride, logits.dtype == torch.bfloat16, gamma, min_commit, commit_all)
    conf = argmax = n_commit = None
    if outputs:
        conf = torch.empty(rows, dtype=torch.float32, device=logits.device)
        argmax = torch.empty(rows, dtype=torch.int32, device=logits.device)
        n_commit = torch.empty(B, dtype=torch.int32, device=logits.device)
    nbytes = L.bd_unmask_workspace_bytes(ctypes.byref(desc))
    ws = _workspace(nbytes, logits.device, workspace)
    _lib.check(L.bd_confidence_unmask(ctypes.byref(desc), _ptr(logits), _ptr(mask), _ptr(tokens), _ptr(conf),
                                      _ptr(argmax), _ptr(n_commit), _ptr(ws), ws.numel(), _stream(stream)),
               "bd_confidence_unmask")
    return {"conf": conf, "argmax": argmax, "n_commit": n_commit}


def confidence_unmask_noalloc(logits, mask, tokens, block_len, gamma, vocab=None, min_commit=True,
                              commit_all=False, outputs=True, stream=None):
    """bd_confidence_unmask_noalloc on torch tensors: the same operation as confidence_unmask with
    the library's static per-device scratch instead of a workspace (nothing is allocated by the
    library; the optional outputs below are the caller's tensors). Returns dict(conf, argmax,
    n_commit)."""
    torch = _torch()
    L = _lib.load()
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be bfloat16 or float32")
    _dev_tensor(logits, "logits")
    _dev_tensor(mask, "mask", torch.uint8)
    _dev_tensor(tokens, "tokens", torch.int32)
    rows, stride = logits.shape
    S = int(block_len)
    if rows % S != 0 or mask.numel() != rows or tokens.numel() != rows:
        raise ValueError("logits rows, mask and tokens must all be B*S")
    B = rows // S
    V = stride if vocab is None else vocab
    desc = unmask_desc(B, S, V, stride, logits.dtype == torch.bfloat16, gamma, min_commit, commit_all)
    conf = argmax = n_commit = None
    if outputs:
        conf = torch.empty(rows, dtype=torch.float32, device=logits.device)
        argmax = torch.empty(rows, dtype=torch.int32, device=logits.device)
        n_commit = torch.empty(B, dtype=torch.int32, device=logits.device)
    _lib.check(L.bd_confidence_unmask_noalloc(ctypes.byref(desc), _ptr(logits), _ptr(mask), _ptr(tokens), _ptr(conf),
                                              _ptr(argmax), _ptr(n_commit), _stream(stream)),
               "bd_confidence_unmask_noalloc")
    return {"conf": conf, "argmax": argmax, "n_commit": n_commit}


def denoise_block(get_qkv: Optional[Callable], get_logits: Optional[Callable], k_cache, v_cache, prefix_len, mask,
                  tokens, T: int,
                  Hq: int, gamma: float, block_len: int, vocab: int, logits_bf16: bool = True, row_stride=None,
                  t0: int = 0, min_commit=True, max_prefix_len=None, softmax_scale=0.0, num_splits=0, out=None,
                  commits_per_step=True, workspace=None, stream=None, step_table=None, steps_used=None):
    """bd_denoise_block.

    Either Python hooks -- ``get_qkv(step, mask, tokens) -> (q, k_blk, v_blk)`` and
    ``get_logits(step, out) -> logits`` returning device tensors (kept alive until the next hook
    call) -- or ``step_table = (qs, k_blks, v_blks, logits)``: per-step tensor lists replayed by
    the library's native table hooks (no call back into Python). Returns
    dict(out, steps_used, commits_per_step)."""
    torch = _torch()
    L = _lib.load()
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_tensor(t, n, torch.bfloat16)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    _dev_tensor(mask, "mask", torch.uint8)
    _dev_tensor(tokens, "tokens", torch.int32)
    B, Hkv, lcap, D = k_cache.shape
    S = int(block_len)
    ad = attn_desc(B, Hq, Hkv, D, S, lcap, max_prefix_len, softmax_scale, num_splits)
    ud = unmask_desc(B, S, vocab, row_stride, logits_bf16, gamma, min_commit, False)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=k_cache.device)
    if steps_used is None:
        steps_used = torch.empty(B, dtype=torch.int32, device=k_cache.device)
    if commits_per_step is True:
        cps = torch.zeros((T, B), dtype=torch.int32, device=k_cache.device)
    elif commits_per_step is False or commits_per_step is None:
        cps = None
    else:
        cps = commits_per_step
    nbytes = L.bd_denoise_workspace_bytes(ctypes.byref(ad), ctypes.byref(ud))
    ws = _workspace(nbytes, k_cache.device, workspace)
    keep = {}
    errors = []

    def _qkv(user, step, mask_p, tokens_p, qp, kp, vp, stream_p):
        try:
            q, kb, vb = get_qkv(step, mask, tokens)
            keep["qkv"] = (q, kb, vb)
            qp[0], kp[0], vp[0] = q.data_ptr(), kb.data_ptr(), vb.data_ptr()
            return _lib.BD_OK
        except Exception as e:  # reported after the call returns
            errors.append(e)
            return _lib.BD_EINVAL

    def _logits(user, step, out_p, lp, stream_p):
        try:
            lg = get_logits(step, out)
            keep["logits"] = lg
            lp[0] = lg.data_ptr()
            return _lib.BD_OK
        except Exception as e:
            errors.append(e)
            return _lib.BD_EINVAL

    if step_table is not None:
        qs, ks, vs, ls = step_table
        if not (len(qs) == len(ks) == len(vs) == len(ls) >= T):
            raise ValueError("step_table needs T entries per list")
        arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
        keep["table"] = (arr(qs), arr(ks), arr(vs), arr(ls))
        table = _lib.StepTable(*[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in keep["table"]], len(qs))
        keep["tab"] = table
        hooks = StepHooks()
        _lib.check(L.bd_table_hooks(ctypes.byref(table), ctypes.byref(hooks)), "bd_table_hooks")
    else:
        hooks = StepHooks(_lib.GET_QKV(_qkv), _lib.GET_LOGITS(_logits), None)
    st = L.bd_denoise_block(ctypes.byref(ad), ctypes.byref(ud), T, t0, ctypes.byref(hooks), _ptr(k_cache),
                            _ptr(v_cache), _ptr(prefix_len), _ptr(out), _ptr(mask), _ptr(tokens), _ptr(steps_used),
                            _ptr(cps), _ptr(ws), ws.numel(), _stream(stream))
    if errors:
        raise errors[0]
    _lib.check(st, "bd_denoise_block")
    return {"out": out, "steps_used": steps_used, "commits_per_step": cps}


def mamba_block_scan(h0, fwd, rev, A, A_r, D, active=None, y=None, h_out=None, want_h_out=True, stream=None):
    """bd_mamba_block_scan on torch tensors. h0 [B,H,N,P] float32 (the cached forward boundary
    state); fwd / rev: (x [B,S,H,P] bf16, dt [B,S,H] float32, Bm [B,S,G,N] bf16, Cm [B,S,G,N] bf16)
    of the forward and the reverse direction; A, A_r, D [H] float32. Returns (y [B,S,H,P] bf16,
    h_out [B,H,N,P] float32 or None)."""
    torch = _torch()
    L = _lib.load()
    _dev_tensor(h0, "h0", torch.float32)
    B, H, N, P = h0.shape
    dirs = []
    for name, (x, dt, Bm, Cm), Ad in (("fwd", fwd, A), ("rev", rev, A_r)):
        _dev_tensor(x, f"{name} x", torch.bfloat16)
        _dev_tensor(dt, f"{name} dt", torch.float32)
        _dev_tensor(Bm, f"{name} Bm", torch.bfloat16)
        _dev_tensor(Cm, f"{name} Cm", torch.bfloat16)
        _dev_tensor(Ad, f"{name} A", torch.float32)
        S = x.shape[1]
        G = Bm.shape[2]
        if x.shape != (B, S, H, P) or dt.shape != (B, S, H) or Bm.shape != (B, S, G, N) or Cm.shape != Bm.shape \
                or Ad.shape != (H,):
            raise ValueError(f"{name} inputs must be x [B,S,H,P], dt [B,S,H], Bm/Cm [B,S,G,N], A [H]")
        dirs.append(_lib.MambaDir(_ptr(x), _ptr(dt), _ptr(Bm), _ptr(Cm), _ptr(Ad)))
    if fwd[0].shape != rev[0].shape or fwd[2].shape != rev[2].shape:
        raise ValueError("forward and reverse inputs must have the same shapes")
    _dev_tensor(D, "D", torch.float32)
    if active is not None:
        _dev_tensor(active, "active", torch.uint8)
    S, G = fwd[0].shape[1], fwd[2].shape[2]
    desc = _lib.MambaDesc(B, H, G, P, N, S)
    if y is None:
        y = torch.empty((B, S, H, P), dtype=torch.bfloat16, device=h0.device)
    if h_out is None and want_h_out:
        h_out = torch.empty_like(h0)
    _lib.check(L.bd_mamba_block_scan(ctypes.byref(desc), _ptr(h0), ctypes.byref(dirs[0]), ctypes.byref(dirs[1]),
                                     _ptr(D), _ptr(active), _ptr(y), _ptr(h_out), _stream(stream)),
               "bd_mamba_block_scan")
    return y, h_out


class Trace:
    """Kernel trace: while attached, every kernel libbd enqueues from this thread is bracketed by
    HIP events on its stream. ``records()`` waits for them and returns [(kernel, ms)]."""

    def __init__(self, capacity: int = 4096):
        self._L = _lib.load()
        h = ctypes.c_void_p()
        _lib.check(self._L.bd_trace_create(capacity, ctypes.byref(h)), "bd_trace_create")
        self.handle = h

    def __enter__(self):
        _lib.check(self._L.bd_trace_attach(self.handle), "bd_trace_attach")
        return self

    def __exit__(self, *exc):
        self._L.bd_trace_attach(None)
        return False

    def clear(self):
        _lib.check(self._L.bd_trace_clear(self.handle), "bd_trace_clear")

    def records(self):
        out = []
        for i in range(self._L.bd_trace_count(self.handle)):
            name = ctypes.c_char_p()
            ms = ctypes.c_float()
            _lib.check(self._L.bd_trace_get(self.handle, i, ctypes.byref(name), ctypes.byref(ms)), "bd_trace_get")
            out.append((name.value.decode(), ms.value))
        return out

    def close(self):
        if self.handle:
            self._L.bd_trace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
