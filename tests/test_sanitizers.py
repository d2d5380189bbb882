"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

Two programs under tests/sanitize/ drive (1) the CPU oracle (oracle/ssm_oracle.c, built
with gcc) and (2) the host side of the C ABI (every .hip source of the library compiled
with the sanitizers on the host pass only, linked into a driver that makes no GPU call).
Each must print OK and exit 0 with no sanitizer report.  Builds are cached under
_build/sanitize/, keyed on a hash of their sources and flags.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "speculative_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ssm_oracle.c")]
    exe = os.path.join(OUT, f"oracle_driver_{_digest(srcs, SAN)}")
    if not os.path.exists(exe):
        _run(["gcc", "-O1", "-std=c99", *SAN, "-o", exe, *srcs, "-lm", "-lpthread"])
    r = _run([exe], env=ENV)
    assert r.stdout.strip() == "OK", r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_abi_host_code_under_asan_ubsan():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    from speculative_decode_amd import build as hip_build
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in hip_build.SOURCES]
    headers = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]
    headers.append(os.path.join(ROOT, "include", "mil_ssm.h"))
    driver = os.path.join(HERE, "abi_driver.c")
    # the sanitizers go to the host pass only: each flag behind -Xarch_host
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    key = _digest(srcs + headers + [driver], hip_build.FLAGS + host_san)
    exe = os.path.join(OUT, f"abi_driver_{key}")
    if not os.path.exists(exe):
        objs = []

        def compile_one(src):
            obj = os.path.join(OUT, f"{os.path.basename(src)}.{key}.o")
            _run([hipcc, *hip_build.FLAGS, *host_san, "-c", src, "-o", obj])
            return obj

        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(compile_one, srcs))
        dobj = os.path.join(OUT, f"abi_driver.{key}.o")
        _run([clang, "-x", "c", "-std=c11", "-O1", *SAN, f"-I{os.path.join(ROOT, 'include')}", "-c", driver,
              "-o", dobj])
        _run([clang, *SAN, "-o", exe, dobj, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV)
    assert r.stdout.strip().endswith("OK"), r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
