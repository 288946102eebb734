"""Compile the gfx950 attention library (libfa.so) with hipcc.

Usage: ``python -m tiled_attention_11_amd._build`` or ``build()`` from Python.
The library is built in-tree, next to this file.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = [os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_kernel.hip"),
           os.path.join(CSRC, "fa_decode.hip"), os.path.join(CSRC, "fa_rope.hip"),
           os.path.join(CSRC, "fa_bwd.hip")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def command(out=LIB, extra=()):
    return ([HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-mcode-object-version=5", f"-I{INCLUDE}", f"-I{CSRC}"] + DEVICE_FLAGS + list(extra)
            + SOURCES + ["-o", out])


def build(out=LIB, extra=(), quiet=True):
    """Compile every source into ``out``; raise with the compiler output on failure."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("libfa build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if not quiet:
        noise = "is not a recognized feature for this target"
        lines = [l for l in res.stderr.splitlines() if noise not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
