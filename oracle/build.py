"""Build the fp64 CPU oracle (test infrastructure) with the host C compiler.

``build()`` compiles ``attn_oracle.c`` into ``liboracle.so`` next to this file.
``build(plant=N)`` builds a copy with deliberate mistake number N compiled in
(``ORACLE_PLANT``), used only by the test that shows the pins catch mistakes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")


def lib_path(plant=0):
    name = "liboracle.so" if not plant else f"liboracle_plant{plant}.so"
    return os.path.join(HERE, name)


def build(plant=0, out=None, quiet=True):
    """Compile the oracle; return the path of the shared library."""
    out = out or lib_path(plant)
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall",
           f"-DORACLE_PLANT={int(plant)}", SRC, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if res.stderr and not quiet:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
