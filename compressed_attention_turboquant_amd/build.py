"""Compile the HIP/C++ sources of the library into libtq.so (in-tree) for gfx950.

Run `python -m compressed_attention_turboquant_amd.build` (or call build()).
Every call recompiles; objects go to _build/ at the repository root.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
# The streaming-read probe bench.py measures the part's read rate with (not
# part of the TurboQuant library).
PROBE_SRC = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libtqprobe.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed-FP32 instructions are disabled for all device code (the compiler
# otherwise emits v_pk_*_f32 on its own from scalar float code).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include")]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include")]


# Sources compiled more than once, each time with its own defines: the decode
# split kernel's instantiations, one object per (head dimension, key kind).
MULTI = {
    "tq_decode_mfma_inst.hip": [(f"d{d}_k{k}", [f"-DTQ_INST_D={d}", f"-DTQ_INST_KIND={k}"])
                                for d in (128, 256) for k in (0, 1, 2)],
    "tq_decode_wide.hip": [(f"q{q}", [f"-DTQ_INST_QJL={q}"]) for q in (0, 1)],
}


def _sources():
    """(source, object name, extra flags) for every compilation."""
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            src = os.path.join(CSRC, name)
            for tag, defs in MULTI.get(name, [("", [])]):
                out.append((src, name + (f".{tag}" if tag else "") + ".o", defs))
    return out


def _compile(job):
    src, objname, defs = job
    obj = os.path.join(BUILD, objname)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", "-c", src, "-o", obj] + HIP_FLAGS + defs
    else:
        cmd = ["g++", "-c", src, "-o", obj] + CXX_FLAGS + defs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", "-shared", PROBE_SRC, "-o", tmp] + HIP_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
