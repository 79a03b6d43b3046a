"""Build the Compressor HIP library in-tree for gfx950.

Produces long_context_kv_wkv_amd/libcompressor.so from csrc/compressor.hip,
and libpeak.so from csrc/peak.hip (the measured MFMA and HBM ceilings the
benchmark reports beside its roofline; not part of the operator).
"""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "compressor.hip")
OUT = os.path.join(PKG, "libcompressor.so")
PEAK_SRC = os.path.join(PKG, "csrc", "peak.hip")
PEAK_OUT = os.path.join(PKG, "libpeak.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-shared", "-fPIC",
           "-I", os.path.join(ROOT, "include"),
           # no packed fp32 instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", tmp, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(PEAK_SRC, PEAK_OUT, verbose)
    _compile(SRC, OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
