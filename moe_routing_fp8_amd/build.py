"""Build libmoe_fp8.so (gfx950) in the package directory with hipcc.

Flags:
  --offload-arch=gfx950       MI355X (CDNA4) only
  -ffp-contract=off           no silent FMA contraction: every fp32 multiply,
                              add and division rounds once, as written
  -target-feature -packed-fp32-ops
                              no packed fp32 VALU instructions
No fast-math: fp32 division stays correctly rounded and denormals are kept.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_fp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=None) -> str:
    cmd = [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-shared", *sources(), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU-only feature; that warning is noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(LIB + ".tmp", LIB)
    return LIB


DEMO_SRC = os.path.join(ROOT, "tests", "c_api", "pipeline_demo.cpp")
DEMO_BIN = os.path.join(ROOT, "tests", "c_api", "pipeline_demo")


def build_c_demo(verbose: bool = False) -> str:
    """The standalone C++ user of the C ABI (tests/c_api/pipeline_demo.cpp),
    linked against libmoe_fp8.so with a relative run path."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), DEMO_SRC,
           "-L", HERE, "-lmoe_fp8", "-Wl,-rpath,$ORIGIN/../../moe_routing_fp8_amd", "-o", DEMO_BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(DEMO_BIN + ".tmp", DEMO_BIN)
    return DEMO_BIN


if __name__ == "__main__":
    print(build(verbose=True))
