"""Build libqk.so (the HIP kernels + C ABI) for gfx950, in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  --offload-arch=gfx950          the only target
  -O3 -std=c++17 -fPIC -shared
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 no packed FP32 instructions in device code
  (default FP modes: IEEE division, f32/f16 denormals kept, round to nearest even)
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqk.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["qk_capi.hip", "qk_quantize.hip", "qk_gemv.hip", "qk_gemm.hip", "qk_dequant.hip",
           "qk_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _compile(src, extra, obj_dir=OBJ_DIR):
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=(), verbose=False, lib=LIB, obj_dir=OBJ_DIR, link_extra=()):
    """Compile every source and link `lib` (the in-tree libqk.so by default; a
    host-sanitizer test build passes its own paths and flags)."""
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), obj_dir), SOURCES))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", lib + ".tmp", *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(lib + ".tmp", lib)
    if verbose:
        print(lib)
    return lib


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
