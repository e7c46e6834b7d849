"""CPU tier of the C ABI: the library loads, exports every entry point include/bd.h declares, and
rejects invalid arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

from block_diffusion_lm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set()
    for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(bd_\w+)\s*\(", src, flags=re.M):
        if "(*" in m.group(0):
            continue
        names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from block_diffusion_lm_amd.build import build
        build()
    return _lib.load()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in bd.h but not exported"
    assert set(names) == set(_lib.EXPORTS)


def test_one_hip_runtime_is_mapped(L):
    # libbd binds to the runtime torch loaded (same soname), so exactly one libamdhip64 is mapped
    rts = _lib.hip_runtimes()
    assert len(rts) == 1, rts


def test_version(L):
    assert b"gfx950" in L.bd_version()


def good_attn():
    return _lib.AttnDesc(2, 32, 2, 128, 16, 4096, 4096, 0.0, 0)


def call_attn(L, d, ptr=16 * 1024, ws=None, nbytes=None):
    if nbytes is None:
        nbytes = L.bd_attn_workspace_bytes(ctypes.byref(d))
    p = ctypes.c_void_p(ptr)
    return L.bd_attn_step(ctypes.byref(d), p, p, p, p, p, p, None, p, None, ws if ws is not None else p, nbytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, _lib.BD_EINVAL),
    ("n_kv_heads", 3, _lib.BD_EINVAL),          # 32 % 3 != 0
    ("head_dim", 96, _lib.BD_EUNSUPPORTED),
    ("block_len", 0, _lib.BD_EINVAL),
    ("block_len", 65, _lib.BD_EINVAL),
    ("max_prefix_len", 5000, _lib.BD_EINVAL),   # > capacity
    ("prefix_capacity", 0, _lib.BD_EINVAL),
    ("num_splits", -1, _lib.BD_EINVAL),
    ("softmax_scale", math.nan, _lib.BD_EINVAL),
    ("causal", 2, _lib.BD_EINVAL),
    ("prefix_capacity", 1 << 23, _lib.BD_EUNSUPPORTED),   # 2 GiB slab at D = 128
])
def test_attn_descriptor_validation(L, field, value, status):
    d = good_attn()
    setattr(d, field, value)
    assert L.bd_attn_workspace_bytes(ctypes.byref(d)) == 0
    assert call_attn(L, d) == status
    assert L.bd_last_error()


def test_attn_pointer_validation(L):
    d = good_attn()
    nb = L.bd_attn_workspace_bytes(ctypes.byref(d))
    assert nb > 0     # this shape is split: partials need a workspace
    p = ctypes.c_void_p(4096)
    bad = ctypes.c_void_p(4096 + 2)
    args = [p] * 6
    for i in range(6):
        a = list(args)
        a[i] = None
        assert L.bd_attn_step(ctypes.byref(d), *a, None, p, None, p, nb, None) == _lib.BD_EINVAL
        a[i] = bad
        assert L.bd_attn_step(ctypes.byref(d), *a, None, p, None, p, nb, None) == _lib.BD_EINVAL
    # output NULL
    assert L.bd_attn_step(ctypes.byref(d), *args, None, None, None, p, nb, None) == _lib.BD_EINVAL
    # workspace too small / misaligned
    assert call_attn(L, d, nbytes=nb - 1) == _lib.BD_EWORKSPACE
    assert b"workspace too small" in L.bd_last_error()
    assert call_attn(L, d, ws=ctypes.c_void_p(4096 + 16), nbytes=nb) == _lib.BD_EINVAL


@pytest.mark.parametrize("desc", [
    (1 << 16, 1024, 64, 64, 64, 4096, 4096, 0.0, 0),      # 2^32 query rows for the merge
    (1024, 8, 8, 128, 16, 1 << 20, 1 << 20, 0.0, 1 << 14),  # 2^27 forced-split workgroups of 256 threads
])
def test_attn_plan_too_large_for_one_launch(L, desc):
    """Problems whose launches would not fit a grid (or the merge's 32-bit row indices) are refused
    before anything is planned into a workspace or enqueued."""
    d = _lib.AttnDesc(*desc)
    assert L.bd_attn_workspace_bytes(ctypes.byref(d)) == 0
    assert call_attn(L, d, nbytes=1 << 40) == _lib.BD_EUNSUPPORTED
    assert b"too large for one launch" in L.bd_last_error()
    info = _lib.AttnPlanInfo()
    assert L.bd_attn_plan(ctypes.byref(d), ctypes.byref(info)) == _lib.BD_EUNSUPPORTED


def test_small_problem_needs_no_workspace(L):
    d = _lib.AttnDesc(1, 8, 2, 64, 16, 256, 256, 0.0, 0)
    assert L.bd_attn_workspace_bytes(ctypes.byref(d)) == 0
    d.num_splits = 3
    assert L.bd_attn_workspace_bytes(ctypes.byref(d)) > 0


def good_unmask():
    return _lib.UnmaskDesc(2, 16, 131072, 131072, _lib.BD_BF16, 0.9, 1, 0)


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("block_len", 65), ("vocab", 0), ("row_stride", 100), ("logits_dtype", 7),
    ("gamma", math.nan), ("gamma", -0.1), ("gamma", 1.5), ("min_commit", 2), ("commit_all", -1),
])
def test_unmask_descriptor_validation(L, field, value):
    d = good_unmask()
    setattr(d, field, value)
    p = ctypes.c_void_p(4096)
    assert L.bd_unmask_workspace_bytes(ctypes.byref(d)) == 0
    assert L.bd_confidence_unmask(ctypes.byref(d), p, p, p, None, None, None, p, 1 << 20, None) == _lib.BD_EINVAL


def test_unmask_stride_alignment(L):
    d = _lib.UnmaskDesc(1, 16, 1001, 1001, _lib.BD_BF16, 0.9, 1, 0)   # 2002-byte rows
    p = ctypes.c_void_p(4096)
    assert L.bd_confidence_unmask(ctypes.byref(d), p, p, p, None, None, None, p, 1 << 20, None) == _lib.BD_EINVAL
    d.row_stride = 1008
    assert L.bd_unmask_workspace_bytes(ctypes.byref(d)) > 0


def test_unmask_pointer_validation(L):
    d = good_unmask()
    nb = L.bd_unmask_workspace_bytes(ctypes.byref(d))
    p = ctypes.c_void_p(4096)
    assert L.bd_confidence_unmask(ctypes.byref(d), None, p, p, None, None, None, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_confidence_unmask(ctypes.byref(d), ctypes.c_void_p(4100), p, p, None, None, None, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_confidence_unmask(ctypes.byref(d), p, None, p, None, None, None, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_confidence_unmask(ctypes.byref(d), p, p, None, None, None, None, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_confidence_unmask(ctypes.byref(d), p, p, p, None, None, None, p, nb - 1, None) == _lib.BD_EWORKSPACE


def test_unmask_noalloc_host_checks(L):
    """The allocation-free unmasking validates like bd_confidence_unmask and rejects, before any
    device call, problems whose slice partials exceed its 4 MiB static scratch (B*S > 349525)."""
    p = ctypes.c_void_p(4096)
    d = good_unmask()
    d.gamma = 2.0
    assert L.bd_confidence_unmask_noalloc(ctypes.byref(d), p, p, p, None, None, None, None) == _lib.BD_EINVAL
    d = good_unmask()
    assert L.bd_confidence_unmask_noalloc(ctypes.byref(d), None, p, p, None, None, None, None) == _lib.BD_EINVAL
    assert L.bd_confidence_unmask_noalloc(ctypes.byref(d), p, p, None, None, None, None, None) == _lib.BD_EINVAL
    big = _lib.UnmaskDesc(5462, 64, 4096, 4096, _lib.BD_F32, 0.9, 1, 0)     # 349568 rows
    assert L.bd_confidence_unmask_noalloc(ctypes.byref(big), p, p, p, None, None, None, None) == _lib.BD_EUNSUPPORTED
    assert b"static scratch" in L.bd_last_error()
    # the largest accepted problem fills the scratch exactly: its workspace query is 4 MiB
    edge = _lib.UnmaskDesc(349525, 1, 4096, 4096, _lib.BD_F32, 0.9, 1, 0)
    assert L.bd_unmask_workspace_bytes(ctypes.byref(edge)) == 4 << 20
    edge.batch += 1
    assert L.bd_unmask_workspace_bytes(ctypes.byref(edge)) > 4 << 20


def good_mamba():
    return _lib.MambaDesc(2, 8, 2, 64, 128, 16)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, _lib.BD_EINVAL), ("n_heads", 0, _lib.BD_EINVAL), ("n_groups", 0, _lib.BD_EINVAL),
    ("n_groups", 3, _lib.BD_EINVAL), ("head_dim", 128, _lib.BD_EUNSUPPORTED), ("state_dim", 96, _lib.BD_EUNSUPPORTED),
    ("state_dim", 256, _lib.BD_EUNSUPPORTED), ("block_len", 0, _lib.BD_EINVAL), ("block_len", 33, _lib.BD_EINVAL),
    ("batch", 1 << 28, _lib.BD_EUNSUPPORTED)])
def test_mamba_descriptor_validation(L, field, value, status):
    d = good_mamba()
    setattr(d, field, value)
    p = ctypes.c_void_p(4096)
    fw = _lib.MambaDir(p, p, p, p, p)
    assert L.bd_mamba_block_scan(ctypes.byref(d), p, ctypes.byref(fw), ctypes.byref(fw), p, None, p, p, None) == status
    assert L.bd_last_error()


def test_mamba_pointer_validation(L):
    d = good_mamba()
    p, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    fw = _lib.MambaDir(p, p, p, p, p)

    def run(h0=p, f=fw, r=fw, D=p, y=p, h_out=p):
        return L.bd_mamba_block_scan(ctypes.byref(d), h0, ctypes.byref(f) if f else None, ctypes.byref(r) if r else None,
                                     D, None, y, h_out, None)

    for kw in ({"h0": None}, {"D": None}, {"y": None}, {"f": None}, {"r": None}, {"h0": odd}, {"y": odd}, {"h_out": odd}):
        assert run(**kw) == _lib.BD_EINVAL, kw
    for i in range(5):
        for bad in (None, odd):
            vals = [p] * 5
            vals[i] = bad
            assert run(r=_lib.MambaDir(*vals)) == _lib.BD_EINVAL
            assert b"reverse" in L.bd_last_error()


def test_denoise_validation(L):
    ad = good_attn()
    ud = good_unmask()
    nb = L.bd_denoise_workspace_bytes(ctypes.byref(ad), ctypes.byref(ud))
    assert nb >= L.bd_attn_workspace_bytes(ctypes.byref(ad)) + L.bd_unmask_workspace_bytes(ctypes.byref(ud))
    p = ctypes.c_void_p(4096)
    hooks = _lib.StepHooks(_lib.GET_QKV(lambda *a: 0), _lib.GET_LOGITS(lambda *a: 0), None)

    def run(T=8, t0=0, h=hooks, ws_bytes=nb, ad_=ad, ud_=ud, steps=p):
        return L.bd_denoise_block(ctypes.byref(ad_), ctypes.byref(ud_), T, t0, ctypes.byref(h) if h else None, p, p, p,
                                  p, p, p, steps, None, p, ws_bytes, None)

    assert run(T=0) == _lib.BD_EINVAL
    assert run(t0=8) == _lib.BD_EINVAL
    assert run(t0=-1) == _lib.BD_EINVAL
    assert run(h=None) == _lib.BD_EINVAL
    assert run(steps=None) == _lib.BD_EINVAL
    assert run(ws_bytes=nb - 1) == _lib.BD_EWORKSPACE
    ud2 = good_unmask()
    ud2.block_len = 32
    assert run(ud_=ud2) == _lib.BD_EINVAL
    assert L.bd_denoise_workspace_bytes(ctypes.byref(ad), ctypes.byref(ud2)) == 0


def test_trace_lifecycle_without_gpu(L):
    h = ctypes.c_void_p()
    assert L.bd_trace_create(0, ctypes.byref(h)) == _lib.BD_EINVAL
    assert L.bd_trace_count(None) == 0
    assert L.bd_trace_get(None, 0, None, None) == _lib.BD_EINVAL


def test_kv_append_validation(L):
    d = good_attn()
    d.max_prefix_len = d.prefix_capacity - d.block_len + 1          # one row past the capacity
    p = ctypes.c_void_p(4096)
    assert L.bd_kv_append(ctypes.byref(d), p, p, p, p, p, None, None) == _lib.BD_EINVAL
    assert b"capacity" in L.bd_last_error()
    d.max_prefix_len = d.prefix_capacity - d.block_len
    for i in range(5):
        a = [p] * 5
        a[i] = None
        assert L.bd_kv_append(ctypes.byref(d), *a, None, None) == _lib.BD_EINVAL
    a = [p] * 5
    a[0] = ctypes.c_void_p(4096 + 8)
    assert L.bd_kv_append(ctypes.byref(d), *a, None, None) == _lib.BD_EINVAL
    d.head_dim = 96
    assert L.bd_kv_append(ctypes.byref(d), *([p] * 5), None, None) == _lib.BD_EUNSUPPORTED


def test_spec_verify_validation(L):
    d = good_unmask()
    nb = L.bd_unmask_workspace_bytes(ctypes.byref(d))
    p = ctypes.c_void_p(4096)
    for i in range(6):
        a = [p] * 6
        a[i] = None
        assert L.bd_spec_verify(ctypes.byref(d), *a, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_spec_verify(ctypes.byref(d), ctypes.c_void_p(4100), *([p] * 5), p, nb, None) == _lib.BD_EINVAL
    assert L.bd_spec_verify(ctypes.byref(d), *([p] * 6), p, nb - 1, None) == _lib.BD_EWORKSPACE
    d.vocab = 0
    assert L.bd_spec_verify(ctypes.byref(d), *([p] * 6), p, nb, None) == _lib.BD_EINVAL


def good_halt():
    return _lib.HaltDesc(4, 4096, _lib.BD_BF16, 1e-3, 8)


@pytest.mark.parametrize("field,value", [("batch", 0), ("n_per_seq", 0), ("n_per_seq", 4100), ("dtype", 7),
                                         ("eps", -1.0), ("eps", math.inf), ("eps", math.nan), ("max_iter", 0)])
def test_halt_descriptor_validation(L, field, value):
    d = good_halt()
    assert L.bd_loop_halt_workspace_bytes(ctypes.byref(d)) > 0
    setattr(d, field, value)
    assert L.bd_loop_halt_workspace_bytes(ctypes.byref(d)) == 0
    p = ctypes.c_void_p(4096)
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 1, p, p, p, 1 << 20, None) == _lib.BD_EINVAL


def test_halt_pointer_validation(L):
    d = good_halt()
    nb = L.bd_loop_halt_workspace_bytes(ctypes.byref(d))
    assert nb % 256 == 0
    p = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4104)
    assert L.bd_loop_halt(ctypes.byref(d), None, p, 1, p, p, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_loop_halt(ctypes.byref(d), p, odd, 1, p, p, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 1, p, None, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 1, ctypes.c_void_p(4098), p, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 0, p, p, p, nb, None) == _lib.BD_EINVAL
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 1, p, p, p, nb - 1, None) == _lib.BD_EWORKSPACE
    assert L.bd_loop_halt(ctypes.byref(d), p, p, 1, p, p, None, nb, None) == _lib.BD_EINVAL
    d.dtype = _lib.BD_F32
    d.n_per_seq = 4
    assert L.bd_loop_halt_workspace_bytes(ctypes.byref(d)) > 0


def test_header_is_c99_and_links_from_c(tmp_path):
    """include/bd.h compiles as strict C99 and a C program links against libbd.so and calls it
    (host-only entry points: version string and workspace planning)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include "bd.h"
#include <stdio.h>
int main(void) {
  bd_attn_desc d = {2, 32, 2, 128, 16, 4096, 4096, 0.0f, 0, 0};
  size_t ws = bd_attn_workspace_bytes(&d);
  d.head_dim = 96;
  size_t bad = bd_attn_workspace_bytes(&d);
  printf("%s %zu %zu\n", bd_version(), ws, bad);
  return (ws > 0 && bad == 0) ? 0 : 1;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lbd", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == "bd" and int(out[-2]) > 0 and int(out[-1]) == 0
