"""Builds libfmdenoise.so (the gfx950 HIP kernels + the C ABI) in place.

hipcc compiles every source for gfx950 only.  Packed-fp32 VALU instructions
are disabled for all device code.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfmdenoise.so")
SOURCES = [os.path.join(CSRC, "fm_kernels.hip"), os.path.join(CSRC, "fm_engine.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Raises on a compiler error."""
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE, prefix=".libfmdenoise.")
    os.close(fd)
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
