"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code (CPU
only; nothing here runs on a GPU):

* the C oracle, built with both sanitizers and driven through every function
  on small inputs with edge cases (tests/sanitize/oracle_driver.c);
* the library's host side -- argument validation, size queries and
  empty-batch no-ops of every C-ABI entry point, none of which launches a
  kernel -- with the sanitizers on the host compilation only
  (tests/sanitize/abi_driver.cpp).

Any sanitizer report fails the test (no recovery); leak detection is off for
the library run, whose HIP runtime keeps allocations for the process
lifetime."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _host_san_flags():
    out = []
    for f in SAN:
        out += ["-Xarch_host", f]
    return out


def _run(cmd, env=None, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_san")
        rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", *SAN,
                        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                        os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
        assert rc == 0, log
        rc, log = _run([exe])
        assert rc == 0 and log.strip().endswith("ok"), log


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_host_abi_under_asan_and_ubsan():
    csrc = os.path.join(ROOT, "moe_routing_fp8_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    with tempfile.TemporaryDirectory() as d:
        procs, objs = [], []
        for name in sorted(os.listdir(csrc)):
            if not name.endswith(".hip"):
                continue
            obj = os.path.join(d, name[:-4] + ".o")
            objs.append(obj)
            procs.append(subprocess.Popen(
                [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", *_host_san_flags(),
                 "-Xarch_device", "-O1", *inc, "-c", os.path.join(csrc, name), "-o", obj],
                stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        driver = os.path.join(d, "driver_main.o")
        procs.append(subprocess.Popen(
            [HIPCC, "-O1", "-g", "-std=c++17", *_host_san_flags(), *inc, "-c",
             os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", driver],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        for p in procs:
            out, _ = p.communicate(timeout=600)
            assert p.returncode == 0, out
        exe = os.path.join(d, "abi_san")
        rc, log = _run([CLANG, *SAN, driver, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
        assert rc == 0, log
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
        rc, log = _run([exe], env=env)
        assert rc == 0 and log.strip().endswith("ok"), log
