"""The C ABI used from a standalone C++ program (tests/c_api/pipeline_demo.cpp,
built by __graft_entry__.build()): HIP runtime and hipMalloc only, no Python
or torch in the process.  It runs top-k, token map, expand + cast and SwiGLU +
cast on one stream and checks what the definitions fix (see the program's
header), then checks moe_route's fused form and moe_dispatch in every mode
against those composed calls bit for bit; it prints "c-api pipeline ok" and
exits 0 when every check holds."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c_api", "pipeline_demo")


def test_c_api_pipeline_from_cpp():
    if not os.path.exists(DEMO):
        raise RuntimeError(f"{DEMO} is not built: run __graft_entry__.build() first")
    sys.__stderr__.write("[gpu-c-api] running tests/c_api/pipeline_demo\n")
    sys.__stderr__.flush()
    res = subprocess.run([DEMO], capture_output=True, text=True, timeout=90)
    assert res.returncode == 0 and "c-api pipeline ok" in res.stdout, res.stdout + res.stderr
