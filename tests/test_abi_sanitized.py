"""The host side of the C ABI (argument checks, workspace sizing, dispatch and
error reporting in csrc/vq_api.hip) under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU: vq_api.hip is compiled with
host-only sanitizers (the device code is unchanged), linked with the library's
other objects, and tests/test_abi.py runs against that build in a child process
with the ASan runtime preloaded. Any sanitizer report fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_decoding_verify_vq_amd")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_under_sanitizers(tmp_path):
    from speculative_decoding_verify_vq_amd.build import ARCH, CSRC, HIPCC_FLAGS
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = _asan_runtime()
    others = [os.path.join(PKG, "_build", os.path.basename(s)[:-4] + ".o")
              for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if not s.endswith("vq_api.hip")]
    if not (os.path.exists(hipcc) and rt and all(os.path.exists(o) for o in others)):
        pytest.skip("needs hipcc, the ASan runtime and the objects of a build (python __graft_entry__.py build)")
    obj, lib = str(tmp_path / "vq_api_san.o"), str(tmp_path / "libvq_san.so")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([hipcc, *flags, *SAN, "-c", os.path.join(CSRC, "vq_api.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, obj, *others],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build carries no sanitizer hooks"
    env = dict(os.environ, VQ_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-p", "no:xdist"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
