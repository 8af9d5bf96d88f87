"""Build tests/c/abi_check, a host program that drives libqk.so through its C ABI
(no Python runtime) and checks every result against the CPU oracle (test
infrastructure).  Needs libqk.so and oracle/liboracle.so built first; both are
found at run time through rpaths relative to the executable."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "abi_check")


def build():
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
    lib_dir = os.path.join(ROOT, "quantized_gemv_quantize_amd")
    orc_dir = os.path.join(ROOT, "oracle")
    cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", orc_dir,
           os.path.join(HERE, "abi_check.cpp"), "-o", EXE + ".tmp",
           "-L", lib_dir, "-lqk", "-L", orc_dir, "-loracle",
           "-Wl,-rpath,$ORIGIN/../../quantized_gemv_quantize_amd", "-Wl,-rpath,$ORIGIN/../../oracle"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(), file=sys.stderr)
