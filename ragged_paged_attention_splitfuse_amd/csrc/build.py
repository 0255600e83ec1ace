"""Build libfg.so in-tree with hipcc for gfx950.

    python -m ragged_paged_attention_splitfuse_amd.csrc.build [--verbose]

Always recompiles (the check that the sources build is the point of calling
it).  Output: ragged_paged_attention_splitfuse_amd/libfg.so.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfg.so")
ARCH = os.environ.get("FG_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{HERE}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [("fg_device.hip", True), ("fg_probe.hip", True), ("plan.cpp", False)]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # hipcc's host pass does not know the device-only target feature; drop that note
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose=False):
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, is_hip in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + COMMON + (DEVICE if is_hip else []) + ["-c", os.path.join(HERE, src), "-o", obj]
        if not is_hip:
            cmd[1:1] = ["-x", "c++"]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
