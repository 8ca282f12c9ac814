"""Build libisa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m sparse_attention_context_block_amd.build
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libisa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled for every kernel.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
# Per-source additions.  The backward kernels run one wave per SIMD, where the
# compiler would otherwise place every MFMA accumulator in AGPRs and copy S, dP
# and the staging registers between AGPRs and VGPRs on every key tile; the VGPR
# form keeps the loops free of those copies.
EXTRA = {"isa_attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # its direct-to-LDS loads set m0 in inline asm and list it as clobbered,
         # which the compiler notes (m0 is reserved) on every expansion
         "isa_attn_w64.hip": ["-Wno-inline-asm"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False, jobs=8):
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose and err:
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
