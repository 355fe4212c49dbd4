"""Build step of the gfx950 library: compiles csrc/*.hip into liblightning.so in this directory.

Run ``python -m long_context_hybrid_amd.build`` (or call ``build()``).  Each source is compiled
to an object in its own hipcc process (in parallel), then the objects are linked.  The library is
built for gfx950 only.  Packed-fp32 VALU instructions are disabled for the device code.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblightning.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
LINK_FLAGS = ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def compile_command(src, obj, extra=()):
    return [HIPCC, *COMPILE_FLAGS, "-I", os.path.join(ROOT, "include"), *extra, "-c", src,
            "-o", obj]


def link_command(objs, out, extra=()):
    return [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, *LINK_FLAGS,
            "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(out=LIB, extra=(), link_extra=(), verbose=False, jobs=None):
    """Compile every source with `extra` flags and link them into `out` (replaced atomically)."""
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 16)))
    with tempfile.TemporaryDirectory(prefix="lt_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, (compile_command(s, o, extra)
                                           for s, o in zip(srcs, objs))))
        for src, (rc, log) in zip(srcs, results):
            if rc != 0:
                sys.stderr.write(log)
                raise RuntimeError(f"hipcc failed to compile {os.path.basename(src)}")
            if verbose:
                sys.stderr.write(log)
        tmp_out = out + ".tmp"
        rc, log = _run(link_command(objs, tmp_out, link_extra))
        if rc != 0:
            sys.stderr.write(log)
            raise RuntimeError("hipcc failed to link liblightning.so")
    os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
