"""Compile the HIP library libnectar.so for gfx950 (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnectar.so")
SOURCES = ["attn.hip", "attn_lds.hip", "merge.hip", "deep_mlp.hip", "metrics.hip", "train.hip", "mlp.hip", "mlp_prefill.hip", "mlp_lds.hip", "finish.hip", "step.hip", "nectar_abi.cpp"]
# Per-source code-generation options: the LDS-staged attention keeps its MFMA
# accumulators in ordinary VGPRs (with accumulation registers the compiler
# copies them back and forth around the softmax on every tile).
SOURCE_FLAGS = {"attn_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "mlp_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# Packed fp32 VALU ops are kept out of every HIP object.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str, extra_flags, verbose: bool, tag: str) -> str:
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    obj = os.path.join(CSRC, "%s.%s.o" % (src.rsplit(".", 1)[0], tag))
    cmd = ([hipcc()] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra_flags) + inc +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, log))
    if verbose:
        print(" ".join(cmd), flush=True)
        if log.strip():
            print(log)
    return obj


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    # the sources compile independently: one hipcc per source, in parallel
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    tag = "b%d" % os.getpid()
    objs = [os.path.join(CSRC, "%s.%s.o" % (src.rsplit(".", 1)[0], tag)) for src in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    try:
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda src: _compile(src, extra_flags, verbose, tag), SOURCES))
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp, out)
    finally:
        # objects of this build (also those of sources that compiled before a
        # failure) and a partial link never stay in the tree
        for o in objs + [tmp]:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
