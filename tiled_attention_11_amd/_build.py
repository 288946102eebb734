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
# The same sources built with FA_CONSERVATIVE_SYNC=1: every DMA and every LDS
# phase waited for, a barrier between the halves of every key step. It must
# give bit-identical results (a GPU test compares the two); not used otherwise.
LIB_SYNC = os.path.join(PKG, "libfa_sync.so")
SYNC_FLAGS = ("-DFA_CONSERVATIVE_SYNC=1",)
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


def _start(out, extra):
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    return cmd, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                      text=True)


def _finish(job, out, quiet):
    cmd, tmp, proc = job
    _, err = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"{os.path.basename(out)} build failed:\n" + " ".join(cmd) + "\n" + err)
    if not quiet:
        noise = "is not a recognized feature for this target"
        lines = [l for l in err.splitlines() if noise not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, out)
    return out


def build(out=LIB, extra=(), quiet=True, sync_variant=True):
    """Compile every source into ``out`` (and, by default, the conservative-sync
    variant into libfa_sync.so, in parallel); raise with the compiler output on
    failure."""
    jobs = [(_start(out, extra), out)]
    if sync_variant:
        jobs.append((_start(LIB_SYNC, tuple(extra) + SYNC_FLAGS), LIB_SYNC))
    for job, o in jobs:
        _finish(job, o, quiet)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
