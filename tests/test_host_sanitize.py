"""CPU: the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

The host-side sources (argument checks, workspace planning, the prefill
pipeline's bookkeeping, the allocation-free entry point, the host forward)
are rebuilt with both sanitizers on their host code only, linked with the
kernels' objects of the regular build and with `host_sanitize_driver.cpp`,
and run on this machine without a GPU: workspace planning over many shapes,
every refusal that returns before a launch, and the host forward of each
weight format.  A memory error or undefined behaviour aborts the run; a
failed expectation exits non-zero.  Skipped when the regular build's
objects are absent."""
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(REPO, "sparse_moe_expert_softmax_amd")
CSRC = os.path.join(PKG, "csrc")
BUILT = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# rebuilt with the sanitizers; the other objects come from the regular build
HOST_SOURCES = ["api.cpp", "pipeline.cpp", "hostfwd.cpp", "noalloc.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    kernels = [os.path.join(BUILT, os.path.splitext(s)[0] + ".o")
               for s in ("route.hip", "slot.hip", "permute.hip", "gemv.hip", "decode_mfma.hip", "mfma.hip",
                         "prefill_bf16.hip")]
    if not all(os.path.exists(k) for k in kernels):
        pytest.skip("the regular build's kernel objects are absent (run the package build first)")
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not found")
    objs = []
    for s in HOST_SOURCES:
        o = str(tmp_path / (os.path.splitext(s)[0] + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *SAN, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    drv = str(tmp_path / "driver.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-c", os.path.join(REPO, "tests", "host_sanitize_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "host_sanitize")
    _run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, *kernels, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-o", exe])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""   # no device work: every call here returns before a launch
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-6000:]}"
    assert "host checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
