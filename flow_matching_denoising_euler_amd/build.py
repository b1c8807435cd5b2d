"""Builds libfmdenoise.so (the gfx950 HIP kernels + the C ABI) in place.

hipcc compiles every source for gfx950 only.  Packed-fp32 VALU instructions
are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfmdenoise.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fm_gemm.hip", "fm_gemm_mx.hip", "fm_attn.hip", "fm_attn_wide.hip", "fm_attn_sf_a.hip", "fm_attn_sf_b.hip",
                                                  "fm_attn_sf_c.hip", "fm_attn_sf_d.hip", "fm_misc.hip", "fm_noalloc.hip", "fm_persist_bf16.hip",
                                                  "fm_persist_fp8.hip", "fm_engine.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), link the library in
    place; returns its path.  Raises on a compiler error."""
    tmpdir = tempfile.mkdtemp(prefix=".build.", dir=HERE)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE, prefix=".libfmdenoise.")
    os.close(fd)
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        procs = [(src, _run([HIPCC] + FLAGS + ["-c", src, "-o", o])) for src, o in zip(SOURCES, objs)]
        msgs = []
        for src, pr in procs:
            out, _ = pr.communicate()
            err = "\n".join(ln for ln in out.splitlines() if NOISE not in ln)
            if pr.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            msgs.append(err)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(link) + "\n" + r.stdout + r.stderr)
        if verbose and any(m.strip() for m in msgs):
            print("\n".join(msgs), file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
