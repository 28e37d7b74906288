"""Build libnvfp4moe.so in-tree with hipcc for gfx950.

    python nvfp4_block_scaled_quant_amd/build.py

Every HIP source is compiled with:
  -ffp-contract=off                          the quantizer's float32 steps must
                                             not be fused into FMAs
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division in the quantizer
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-FP32 instructions
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnvfp4moe.so")
SOURCES = ["api.hip", "quantize.hip", "route.hip", "gemm.hip", "skinny.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    build_capi_check(cc)
    return OUT


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "closed_form.cpp")
CAPI_BIN = os.path.join(ROOT, "tests", "capi", "closed_form")


def build_capi_check(cc):
    """The C-ABI check program of the GPU tests (host code only: it calls the
    library through include/nvfp4moe.h, linked against the in-tree .so)."""
    if not os.path.exists(CAPI_SRC):
        return
    cmd = [cc, "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", CAPI_SRC, "-o", CAPI_BIN + ".tmp",
           f"-L{PKG}", "-lnvfp4moe", "-Wl,-rpath,$ORIGIN/../../nvfp4_block_scaled_quant_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C-ABI check program failed to build:\n{r.stdout}\n{r.stderr}")
    os.replace(CAPI_BIN + ".tmp", CAPI_BIN)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
