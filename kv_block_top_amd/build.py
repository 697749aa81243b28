"""Build libkvbt.so in-tree with hipcc for gfx950.

    python -m kv_block_top_amd.build            # build (always recompiles)
    python -m kv_block_top_amd.build --isa DIR  # also write the gfx950 assembly to DIR

Every HIP source is compiled with packed-fp32 instructions disabled (the selector
does no floating-point math; this keeps the compiler from emitting them anywhere).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvbt.so")
SOURCES = ["kvbt_api.cpp", "kvbt_kernels.hip", "kvbt_bench.hip", "kvbt_attn.hip",
           "kvbt_index.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _flags():
    return ["--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


# per-source extra flags: the attention and index-score kernels keep their MFMA
# accumulators in ordinary VGPRs (vector instructions read and rescale them)
# kvbt_kernels.hip: the selector kernels' leading scalar arguments are preloaded into
# scalar registers at wave launch (kernels whose first argument is a struct preload none)
EXTRA_FLAGS = {"kvbt_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "kvbt_index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "kvbt_kernels.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=11"]}


def _compile(src: str, obj: str, isa_dir: str | None):
    cmd = [hipcc()] + _flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src),
                                                             "-o", obj]
    if isa_dir and src.endswith(".hip"):
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return r.stderr


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every source and link libkvbt.so next to this file. Returns its path."""
    tmp = tempfile.mkdtemp(prefix="kvbt_build_", dir=isa_dir or None)
    try:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            logs = list(ex.map(lambda so: _compile(so[0], so[1], isa_dir), zip(SOURCES, objs)))
        if verbose:
            for s, log in zip(SOURCES, logs):
                if log.strip():
                    print("[%s]\n%s" % (s, log))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
        os.replace(out_tmp, LIB)
        if isa_dir:
            for f in os.listdir(tmp):
                if f.endswith(".s") and ARCH in f:
                    shutil.copy(os.path.join(tmp, f), os.path.join(isa_dir, f))
    finally:
        if not isa_dir:
            shutil.rmtree(tmp, ignore_errors=True)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None, help="directory for the gfx950 assembly")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    if args.isa:
        os.makedirs(args.isa, exist_ok=True)
    print(build(args.isa, args.verbose))


if __name__ == "__main__":
    main()
