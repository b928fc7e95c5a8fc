"""CPU sanitizer tier: the oracle and the host side of the C ABI built with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no GPU),
each driven over its entry points by a small C program under tests/sanitize/.
Any report fails the test: the builds stop at the first error."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "compressed_sparse_attention_06_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "oracle ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_capi_host_under_address_and_ub_sanitizers(tmp_path):
    """Every .hip file compiled with the host pass instrumented (the device
    code is built as usual and never runs), linked with a C driver that sizes
    workspaces over many shapes and drives every argument check."""
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")]
    objs = []
    procs = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            o = str(tmp_path / (f[:-4] + ".o"))
            objs.append(o)
            procs.append((f, subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, f), "-o", o],
                                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for f, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{f}: {err}"
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
          os.path.join(SAN, "capi_driver.c"), "-o", drv])
    exe = str(tmp_path / "capi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, drv, *objs, "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime's own allocations are not this library's: no leak check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "capi ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
