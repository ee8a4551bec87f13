"""Build libmsa.so (the HIP kernels + C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "libmsa.so")
SOURCES = ["msa_abi.hip", "msa_index.hip", "msa_indexer.hip", "msa_forward.hip", "msa_backward.hip",
           "msa_backward_kv.hip", "msa_backward_kv2.hip", "msa_backward_dq.hip",
           "msa_backward_dqs.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-munsafe-fp-atomics",
         # no packed-fp32 VALU ops (v_pk_*_f32) in any generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-file code-generation options (none at present).
FILE_FLAGS = {}


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libmsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "%d" % os.getpid()
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".%s.o" % tag))
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + FILE_FLAGS.get(src, []) + \
            ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errors = []
    for src, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append("%s:\n%s%s" % (src, out, err))
    try:
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = LIB + ".tmp" + tag
        cmd = [HIPCC] + FLAGS + ["-o", tmp] + objs
        if verbose:
            print(" ".join(cmd))
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
