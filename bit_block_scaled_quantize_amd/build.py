"""Builds libnvfp4.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Usage: python -m bit_block_scaled_quantize_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4.so")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                      # bit-exact FP32 op order in the encoders
    "-fno-gpu-flush-denormals-to-zero",       # FP32 subnormals are part of the contract
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libnvfp4.so next to this file. Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


def resource_usage() -> dict[str, dict[str, int]]:
    """Per-kernel register and scratch use reported by the compiler for every source (device
    code only, nothing written): {mangled kernel name: {"vgpr", "agpr", "scratch"}}."""
    hipcc = _hipcc()
    out: dict[str, dict[str, int]] = {}

    def one(src):
        cmd = [hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-S", "-o", os.devnull, src,
               "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
        return res.stderr

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
        logs = list(ex.map(one, sources()))
    for log in logs:
        name = None
        for line in log.splitlines():
            if "Function Name:" in line:
                name = line.split("Function Name:")[1].strip()
                out[name] = {}
            elif name is not None:
                for key, tag in (("vgpr", "VGPRs:"), ("agpr", "AGPRs:"), ("scratch", "ScratchSize [bytes/lane]:")):
                    if tag in line:
                        out[name][key] = int(line.split(tag)[1].split()[0])
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
