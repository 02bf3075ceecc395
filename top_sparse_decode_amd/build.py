"""Build libsparse_decode.so in-tree with hipcc for gfx950.

Run ``python -m top_sparse_decode_amd.build``.  The library is built from the
HIP sources in ``csrc/`` and the public header in ``include/``; it links
nothing but the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsparse_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("SD_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "score.hip", "topk.hip", "attn.hip", "tri.hip"]

# Per-source options.  The scorer keeps its matrix-core accumulators in
# ordinary VGPRs (its epilogue reads every one of them on the VALU; AGPR
# accumulators would cost a v_accvgpr_read per value).
EXTRA = {"score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # each written float operation rounds on its own unless a kernel asks for
    # a fused multiply-add explicitly (the exact scoring order depends on it)
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(CSRC, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False) -> str:
    # the sources compile independently: one hipcc per source, in parallel
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    # every kernel the library launches must be defined in it (a template
    # whose host side failed to instantiate leaves an undefined launch stub)
    undef = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    missing = [ln.split()[-1] for ln in undef.splitlines() if ln.split() and ln.split()[-1].startswith("_ZN2sd")]
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"libsparse_decode.so leaves library symbols undefined: {missing}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
