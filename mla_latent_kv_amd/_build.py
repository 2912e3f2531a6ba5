"""Builds the shared libraries in-tree with hipcc for gfx950:

* libmla_latent.so  -- the absorbed decode path (HIP kernels + C ABI of include/mla_latent.h);
  depends on the HIP runtime only;
* libmla_normal.so  -- the Normal-path comparison (include/mla_normal.h), whose
  up-projection GEMMs are rocBLAS calls;
* libmla_probe.so   -- the benchmark's practical-roof probe (csrc/roof_probe.hip),
  not part of the decode path.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_latent.so")
NORMAL_LIB = os.path.join(HERE, "libmla_normal.so")
PROBE_LIB = os.path.join(HERE, "libmla_probe.so")
# library -> (sources, extra link flags)
LIBRARIES = {
    LIB: (["api.cpp", "decode_latent.hip", "merge_splits.hip", "merge_unabsorb.hip", "bmm.hip", "append.hip",
           "noalloc.hip"], []),
    NORMAL_LIB: (["normal_api.cpp", "normal.hip"],
                 ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocblas"]),
    PROBE_LIB: (["roof_probe.hip"], []),
}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic is left to nobody: the kernels are compiled without it
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm", "-Wno-unused-command-line-argument",
    # intrinsic MFMAs keep their accumulators in VGPRs; the decode kernel's
    # 256-register value accumulator is pinned to AGPRs by its inline assembly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel) and link the shared libraries."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    sources = sorted({src for srcs, _ in LIBRARIES.values() for src in srcs})
    for src in sources:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            errors.append(f"{src}:\n{out.decode(errors='replace')}")
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    for lib, (srcs, flags) in LIBRARIES.items():
        tmp = lib + ".tmp"
        objs = [os.path.join(BUILD, src + ".o") for src in srcs]
        subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *flags])
        os.replace(tmp, lib)
    return LIB



# sources the decode kernel is built from (a stored counter record of the
# decode kernel stays valid while these are unchanged)
DECODE_SOURCES = ("decode_latent.hip", "common.hpp", "launch.hpp")


def kernel_source_hash(names=DECODE_SOURCES) -> str:
    """sha256 over the named kernel sources with comments and whitespace
    removed (identifies which code a stored counter measurement belongs to;
    editing a comment does not change it)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode())
        h.update(text.encode())
    return h.hexdigest()


if __name__ == "__main__":
    print(build(verbose=True))
