"""CPU tier: the library's host code built with AddressSanitizer and UndefinedBehaviorSanitizer
(hipcc -Xarch_host -fsanitize=..., device code untouched) and driven through the ABI's host
validation paths, the plan and workspace queries over the workloads' shapes and extreme values,
the table hooks and the trace objects (tests/sanitize/abi_paths.cpp). Any sanitizer report aborts
the driver, and the test fails on a non-zero exit or on report text in its output."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_lm_amd", "csrc")
SOURCES = ["bd_api.cpp", "bd_attn.hip", "bd_unmask.hip", "bd_cache.hip", "bd_halt.hip", "bd_mamba.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = tmp_path_factory.mktemp("sanitize")
    cc = hipcc()
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Wno-unused-function"] + SAN
    procs, objs = [], []
    for src in SOURCES + ["abi_paths.cpp"]:
        path = os.path.join(os.path.dirname(__file__), "sanitize", src) if src == "abi_paths.cpp" else os.path.join(CSRC, src)
        obj = str(out / (src + ".o"))
        objs.append(obj)
        cmd = [cc, *common]
        if src.endswith(".hip"):
            cmd += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip"]
        cmd += ["-c", path, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, pr in procs:
        text, _ = pr.communicate()
        assert pr.returncode == 0, f"compiling {src} failed:\n{text}"
    exe = str(out / "abi_paths")
    r = subprocess.run([cc, "--offload-arch=gfx950", *SAN, "-o", exe, *objs], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return exe


def test_host_paths_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([driver], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    out = r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out and "LeakSanitizer" not in out, out
    assert r.returncode == 0, out
    assert "ok: 0 failure(s)" in out, out
