"""ctypes declarations of the C ABI in include/bd.h (loading and prototypes only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbd.so")

BD_OK, BD_EINVAL, BD_EUNSUPPORTED, BD_EWORKSPACE, BD_EHIP = range(5)
BD_BF16, BD_F32 = 0, 1
STATUS_NAMES = {0: "BD_OK", 1: "BD_EINVAL", 2: "BD_EUNSUPPORTED", 3: "BD_EWORKSPACE", 4: "BD_EHIP"}


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("prefix_capacity", ctypes.c_int64),
        ("max_prefix_len", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("causal", ctypes.c_int32),
    ]


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("waves", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("chunk_keys", ctypes.c_int64),
        ("workgroups", ctypes.c_int64),
    ]


class UnmaskDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("row_stride", ctypes.c_int64),
        ("logits_dtype", ctypes.c_int32),
        ("gamma", ctypes.c_float),
        ("min_commit", ctypes.c_int32),
        ("commit_all", ctypes.c_int32),
    ]


class MambaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("state_dim", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
    ]


class MambaDir(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p),
                ("A", ctypes.c_void_p)]


class HaltDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_per_seq", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("max_iter", ctypes.c_int32),
    ]


GET_QKV = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p)
GET_LOGITS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                              ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p)


class StepHooks(ctypes.Structure):
    _fields_ = [("get_qkv", GET_QKV), ("get_logits", GET_LOGITS), ("user", ctypes.c_void_p)]


class StepTable(ctypes.Structure):
    _fields_ = [("q", ctypes.POINTER(ctypes.c_void_p)), ("k_blk", ctypes.POINTER(ctypes.c_void_p)),
                ("v_blk", ctypes.POINTER(ctypes.c_void_p)), ("logits", ctypes.POINTER(ctypes.c_void_p)),
                ("n_steps", ctypes.c_int32)]


EXPORTS = [
    "bd_attn_workspace_bytes", "bd_attn_step", "bd_unmask_workspace_bytes", "bd_confidence_unmask",
    "bd_denoise_workspace_bytes", "bd_denoise_block", "bd_last_error", "bd_trace_create", "bd_trace_destroy",
    "bd_trace_attach", "bd_trace_clear", "bd_trace_count", "bd_trace_get", "bd_version", "bd_table_hooks",
    "bd_kv_append", "bd_spec_verify", "bd_loop_halt_workspace_bytes", "bd_loop_halt",
    "bd_confidence_unmask_noalloc", "bd_attn_plan", "bd_mamba_block_scan",
]

_lib = None


def hip_runtimes() -> list:
    """Distinct HIP runtime libraries (libamdhip64) mapped into this process, by real path."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in os.path.basename(parts[5]):
                    found.add(os.path.realpath(parts[5]))
    except OSError:
        return []
    return sorted(found)


def load() -> ctypes.CDLL:
    """Load libbd.so (built in-tree). Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_diffusion_lm_amd.build`")
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one libbd binds to, so
    # streams and device pointers handed over from torch are valid inside the library.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    # two runtimes would give the library streams and pointers that are not its own
    rts = hip_runtimes()
    if len(rts) > 1:
        raise RuntimeError(f"more than one HIP runtime is mapped into this process: {rts}; libbd must share "
                           "torch's (import torch first, link libbd without a private runtime copy)")
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER
    L.bd_attn_workspace_bytes.argtypes = [P(AttnDesc)]
    L.bd_attn_workspace_bytes.restype = sz
    L.bd_attn_step.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bd_attn_step.restype = ctypes.c_int
    L.bd_unmask_workspace_bytes.argtypes = [P(UnmaskDesc)]
    L.bd_unmask_workspace_bytes.restype = sz
    L.bd_confidence_unmask.argtypes = [P(UnmaskDesc), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bd_confidence_unmask.restype = ctypes.c_int
    L.bd_mamba_block_scan.argtypes = [P(MambaDesc), vp, P(MambaDir), P(MambaDir), vp, vp, vp, vp, vp]
    L.bd_mamba_block_scan.restype = ctypes.c_int
    L.bd_attn_plan.argtypes = [P(AttnDesc), P(AttnPlanInfo)]
    L.bd_attn_plan.restype = ctypes.c_int
    L.bd_confidence_unmask_noalloc.argtypes = [P(UnmaskDesc), vp, vp, vp, vp, vp, vp, vp]
    L.bd_confidence_unmask_noalloc.restype = ctypes.c_int
    L.bd_denoise_workspace_bytes.argtypes = [P(AttnDesc), P(UnmaskDesc)]
    L.bd_denoise_workspace_bytes.restype = sz
    L.bd_denoise_block.argtypes = [P(AttnDesc), P(UnmaskDesc), i32, i32, P(StepHooks), vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp, sz, vp]
    L.bd_denoise_block.restype = ctypes.c_int
    L.bd_kv_append.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp, vp, vp]
    L.bd_kv_append.restype = ctypes.c_int
    L.bd_spec_verify.argtypes = [P(UnmaskDesc), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bd_spec_verify.restype = ctypes.c_int
    L.bd_loop_halt_workspace_bytes.argtypes = [P(HaltDesc)]
    L.bd_loop_halt_workspace_bytes.restype = sz
    L.bd_loop_halt.argtypes = [P(HaltDesc), vp, vp, i32, vp, vp, vp, sz, vp]
    L.bd_loop_halt.restype = ctypes.c_int
    L.bd_table_hooks.argtypes = [P(StepTable), P(StepHooks)]
    L.bd_table_hooks.restype = ctypes.c_int
    L.bd_last_error.argtypes = []
    L.bd_last_error.restype = ctypes.c_char_p
    L.bd_version.argtypes = []
    L.bd_version.restype = ctypes.c_char_p
    L.bd_trace_create.argtypes = [i32, P(vp)]
    L.bd_trace_create.restype = ctypes.c_int
    L.bd_trace_destroy.argtypes = [vp]
    L.bd_trace_destroy.restype = None
    L.bd_trace_attach.argtypes = [vp]
    L.bd_trace_attach.restype = ctypes.c_int
    L.bd_trace_clear.argtypes = [vp]
    L.bd_trace_clear.restype = ctypes.c_int
    L.bd_trace_count.argtypes = [vp]
    L.bd_trace_count.restype = i32
    L.bd_trace_get.argtypes = [vp, i32, P(ctypes.c_char_p), P(ctypes.c_float)]
    L.bd_trace_get.restype = ctypes.c_int
    _lib = L
    return L


class BdError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != BD_OK:
        raise BdError(status, where, load().bd_last_error().decode())
