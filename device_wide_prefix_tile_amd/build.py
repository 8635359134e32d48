"""Builds libdwpt_scan.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libdwpt_scan.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into one shared library; always recompiles."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC] + sources() + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\ncommand: %s" % (res.returncode, msg, " ".join(cmd)))
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_asan(driver: str, out: str, verbose: bool = False) -> str:
    """The library's sources and a test driver (C++ calling the C ABI) as one executable
    whose host code is built with AddressSanitizer (device code as in the library)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + flags + san + ["-I" + INCLUDE, "-I" + CSRC] + sources() + [driver, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\ncommand: %s" % (res.returncode, msg, " ".join(cmd)))
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
