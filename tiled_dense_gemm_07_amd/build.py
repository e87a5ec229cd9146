"""Build libtilegemm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every HIP source is compiled with hipcc for gfx950 only; packed fp32 ALU ops are
disabled (-packed-fp32-ops) and the objects are linked into one shared library
next to this file.  Run ``python -m tiled_dense_gemm_07_amd.build``.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtilegemm.so")
SOURCES = ["tg_api.hip", "tg_gemm_f32.hip", "tg_gemm_f16.hip", "tg_gemm_bf16.hip",
           "tg_dequant_w4.hip", "tg_gemm_mx.hip", "tg_gemm_sp24.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    return _build_lib(SOURCES, LIB, verbose)


def _build_lib(sources, lib_path: str, verbose: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC] + FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-c",
                                 os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "not a recognized feature" not in l)
        if verbose and text.strip():
            print(text)
        if p.returncode != 0:
            failed.append((src, text))
    if failed:
        for src, text in failed:
            sys.stderr.write("---- %s ----\n%s\n" % (src, text))
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))
    tmp = lib_path + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                   check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
