"""Build libkvq.so in-tree for gfx950 with hipcc.

    python -m quantized_decode_attention_02_amd.build

Compiles every HIP source under csrc/ to an object (in parallel) and links
them into one shared library next to this file.  Flags: IEEE float32 division and square root and denormals are the
hipcc defaults and are left alone (the quantizers rely on correctly rounded
division); packed fp32 instructions are disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["api.cpp", "quant.hip", "decode_generic.hip", "decode_mfma.hip", "decode_rope.hip",
           "noalloc.hip", "ext.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Xclang",
            "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)


def build(verbose=False):
    """Compile every source to an object (in parallel), then link."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    cmds = [[hipcc()] + _flags() + ["-c", "-x", "hip", os.path.join(CSRC, s),
                                    "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    out_tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs +
         ["-o", out_tmp], verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
