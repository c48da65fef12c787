"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the host.

The argument validation, workspace sizing and dispatch code of ``rva_api.cpp`` is compiled
with ASan + UBSan on its host code (``-Xarch_host``: the kernels are the regular build's
objects), linked into a separate librva, and ``tests/test_abi_host.py`` runs against it in a
subprocess with the sanitizer runtime loaded first.  Any out-of-bounds access, use after
free or undefined behaviour on those paths aborts the subprocess.  CPU only: no kernel is
launched by these tests.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from ragged_verify_acceptance_amd import build as rvabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(rvabuild.BUILD_DIR, "hostcheck")
# host-only instrumentation (one "-Xarch_host -f..." pair per flag)
SAN = " ".join(f"-Xarch_host {f}" for f in ("-fsanitize=address", "-fsanitize=undefined",
                                             "-fno-sanitize-recover=undefined",
                                             "-fno-omit-frame-pointer")).split()


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_hostcheck() -> str:
    objs = [os.path.join(rvabuild.BUILD_DIR, f + ".o") for f in rvabuild.SOURCES if f != "rva_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        rvabuild.build()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "rva_api.o")
    cc = rvabuild.hipcc()
    cmd = [cc, *[f for f in rvabuild.CFLAGS if f != "-O3"], "-O1", "-g", *SAN, "-x", "hip", "-c",
           os.path.join(rvabuild.CSRC, "rva_api.cpp"), "-o", api]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lib = os.path.join(OUT, "librva_hostcheck.so")
    cmd = [cc, f"--offload-arch={rvabuild.ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN, api, *objs,
           "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return lib


def test_abi_host_under_asan_ubsan():
    rt = _runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this ROCm installation")
    lib = build_hostcheck()
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_" in undef and "__ubsan_handle_" in undef, "the API layer is not instrumented"
    env = dict(os.environ)
    env["RVA_LIBRARY"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # the instrumented library is the one loaded, and the sanitizer runtime is live
    probe = ("import ctypes; from ragged_verify_acceptance_amd import rva; L = rva.lib(); "
             f"assert L._name == {lib!r}, L._name; "
             "assert hasattr(ctypes.CDLL(None), '__asan_report_load8'); print('asan live')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "asan live" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_host.py"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
