"""Build the gfx950 attention library in-tree with hipcc.

    python -m exact_io_aware_41_amd.build

produces exact_io_aware_41_amd/libfa_mi355x.so from csrc/ and include/.
Every HIP translation unit is compiled for gfx950 only, with packed fp32
VALU instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the same sources built with the race-check switches: LDS copy destinations
# poisoned with NaN before every copy, work-group ids visited in a scrambled
# order (tests compare it bit for bit with the default library)
DEBUG_LIB_NAME = "libfa_mi355x_debug.so"
DEBUG_LIB_PATH = os.path.join(PKG, DEBUG_LIB_NAME)
DEBUG_FLAGS = ["-DFA_LDS_POISON=1", "-DFA_WG_PERMUTE=1"]

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_f32.hip", "fa_decode.hip",
           "fa_fwd_fp8.hip", "fa_noalloc.hip"]
# per-source code-generation options (none at present)
EXTRA_FLAGS: dict[str, list[str]] = {}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators and operands in VGPRs: kernels with more than 256
        # live registers (one wave per SIMD: d = 192 and 256, the fp32 paths)
        # otherwise had the compiler park values in AGPRs and copy them back
        # and forth, several hundred v_accvgpr moves per loop iteration
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the library, and the same
    sources with the race-check switches into the debug library.

    Always recompiles.  Each library is written to a temporary name and moved
    into place, so a concurrent reader never sees a partial file.
    """
    cc = hipcc()
    variants = [(LIB_NAME, LIB_PATH, []), (DEBUG_LIB_NAME, DEBUG_LIB_PATH, DEBUG_FLAGS)]
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        cmds = []
        objs = {name: [] for name, _, _ in variants}
        for name, _, flags in variants:
            for src in SOURCES:
                obj = os.path.join(tmp, f"{name}.{src}.o")
                lang = ["-x", "hip"] if src.endswith(".hip") else []
                cmds.append([cc, *common_flags(), *flags, *EXTRA_FLAGS.get(src, []), *lang, "-c",
                             os.path.join(CSRC, src), "-o", obj])
                objs[name].append(obj)
        with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 4)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        for name, path, _ in variants:
            tmp_lib = os.path.join(tmp, name)
            _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs[name], "-o", tmp_lib],
                 verbose)
            staged = path + ".tmp"
            shutil.copyfile(tmp_lib, staged)
            os.replace(staged, path)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
