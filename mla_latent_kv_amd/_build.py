"""Builds the shared libraries in-tree with hipcc for gfx950:

* libmla_latent.so  -- the absorbed decode path (HIP kernels + C ABI of include/mla_latent.h);
  depends on the HIP runtime only;
* libmla_normal.so  -- the Normal-path comparison (include/mla_normal.h), whose
  up-projection GEMMs are rocBLAS calls;
* libmla_probe.so   -- the benchmark's practical-roof probe (csrc/roof_probe.hip),
  not part of the decode path;
* libmla_timeline.so -- libmla_latent.so with the decode kernel built with
  MLA_DECODE_TIMELINE: each wave stamps the real-time counter at eight points
  of its work unit (bench.py --timeline reads them); not for production use.
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
TIMELINE_LIB = os.path.join(HERE, "libmla_timeline.so")
TIMELINE = ("decode_latent.hip", "MLA_DECODE_TIMELINE")   # (source, macro) of the timeline build
_PATH_SOURCES = ["api.cpp", "decode_latent.hip", "merge_splits.hip", "merge_unabsorb.hip", "bmm.hip",
                 "append.hip", "noalloc.hip"]
# library -> (sources, extra link flags); a source given as (file, macro) is
# compiled with that macro defined, into an object of its own
LIBRARIES = {
    LIB: (_PATH_SOURCES, []),
    NORMAL_LIB: (["normal_api.cpp", "normal.hip"],
                 ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocblas"]),
    PROBE_LIB: (["roof_probe.hip"], []),
    TIMELINE_LIB: ([TIMELINE if s == TIMELINE[0] else s for s in _PATH_SOURCES], []),
}


def _object(src) -> str:
    if isinstance(src, tuple):
        return os.path.join(BUILD, f"{src[0]}.{src[1]}.o")
    return os.path.join(BUILD, src + ".o")
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
    sources = sorted({src for srcs, _ in LIBRARIES.values() for src in srcs}, key=str)
    for src in sources:
        name, defs = (src[0], [f"-D{src[1]}"]) if isinstance(src, tuple) else (src, [])
        cmd = [cc, *HIPCC_FLAGS, *defs, "-c", os.path.join(CSRC, name), "-o", _object(src)]
        if name.endswith(".hip"):
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
        objs = [_object(src) for src in srcs]
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
