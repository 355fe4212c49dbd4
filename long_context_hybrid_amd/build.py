"""Build step of the gfx950 library: compiles csrc/*.hip into liblightning.so in this directory
(linked against hipBLASLt, which runs the layer's two projection GEMMs).

Run ``python -m long_context_hybrid_amd.build`` (or call ``build()``).  The library is built for
gfx950 only.  Packed-fp32 VALU instructions are disabled for the device code.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblightning.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def command(out=LIB, extra=()):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), *extra, *sources(),
            "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib", "-o", out]


def build(out=LIB, extra=(), verbose=False):
    tmp = out + ".tmp"
    res = subprocess.run(command(tmp, extra), capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build liblightning.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
