"""Builds libqwen3_prefill.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m transformer_lm_prefill_amd.build_lib   (or call build()).
Each .hip source is compiled to an object under _build/ in parallel, then linked into
transformer_lm_prefill_amd/libqwen3_prefill.so, which the Python binding loads.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqwen3_prefill.so")
# longest compiles first (the product kernels), so the parallel build ends sooner
SOURCES = ["gemm_part_f16.hip", "gemm_part_q4.hip", "gemm_part_f16_cvt.hip", "gemm_part_bf16.hip",
           "capi.hip", "norm_rope.hip", "gemm_mfma.hip", "attention_mfma.hip", "fp32_path.hip",
           "model_head.hip", "vision_rope.hip", "decode.hip",
           "quant.hip", "noalloc.hip", "measure.hip", "tiles.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose=False, jobs=None, defines=(), lib_path=LIB, build_dir=BUILD):
    """Compile every HIP source for gfx950 and link the shared library. Always rebuilds.

    defines: extra preprocessor definitions (e.g. ("Q3_GEMM_SCHED=0",)) for tuning builds,
    written with lib_path/build_dir elsewhere than the default library.
    """
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    dflags = [f"-D{d}" for d in defines]
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = lib_path + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub was not emitted fails here, not at load
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp])
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
