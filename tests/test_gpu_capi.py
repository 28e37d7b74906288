"""The library used from C++ through include/nvfp4moe.h alone (no Python
binding, no torch): tests/capi/closed_form.cpp builds the constant layer whose
output is known by hand (y = 5760 everywhere, as in test_oracle_closed_form)
with the library's weight quantizer and prepack, and runs nvfp4_moe_forward
and nvfp4_moe_forward_noalloc. nvfp4_block_scaled_quant_amd/build.py builds
the program next to its source; it runs here as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "capi", "closed_form")


def test_c_abi_closed_form_layer():
    assert os.path.exists(EXE), "build the library first (nvfp4_block_scaled_quant_amd/build.py)"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout} {r.stderr}"
    assert "nvfp4_moe_forward: 0 of 1024 elements differ" in r.stdout
    assert "nvfp4_moe_forward_noalloc: 0 of 1024 elements differ" in r.stdout
