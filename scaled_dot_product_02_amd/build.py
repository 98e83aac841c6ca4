"""Build the C-ABI shared library (libsdpa02.so) for gfx950 with hipcc, in-tree.

Usage: python -m scaled_dot_product_02_amd.build [--resource-usage]
Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsdpa02.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
SOURCES = ["attn_kernels.hip", "attn_probe.hip", "attn_noalloc.hip", "attn_abi.cpp"]


def _compile(src, obj, extra):
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(resource_usage=False, verbose=True):
    """Compile every source and link libsdpa02.so next to this file. Returns its path."""
    with tempfile.TemporaryDirectory(prefix="sdpa02_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            logs = list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
        tmp_lib = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}")
    if resource_usage:
        for log in logs:
            for line in log.splitlines():
                if "remark" in line and ("Function Name" in line or "VGPRs:" in line or "AGPRs" in line
                                         or "ScratchSize" in line or "Occupancy" in line or "LDS Size" in line
                                         or "SGPRs:" in line):
                    print(line.split("remark:")[-1].strip())
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv)
