"""Build libswa.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m sliding_window_attention_sink_amd.build

compiles every source under csrc/ for gfx950 and links
sliding_window_attention_sink_amd/libswa.so.  Object files go to _build/.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libswa.so")

SOURCES = ["swa_api.cpp", "prefill.hip", "prefill_bf16.hip", "decode.hip", "append.hip", "rope.hip",
           "backward.hip", "global.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
            # packed fp32 VALU ops stay off: ordinary float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the kernels never produce NaN (masked scores are -inf), so max
            # needs no NaN canonicalisation; infinities keep IEEE semantics
            "-fno-honor-nans",
            "-Wno-unused-command-line-argument"]


# Per-source flags.  backward.hip: the MFMA accumulators of the dK/dV and dQ
# loops are carried across iterations; in the AGPR form of the MFMA the
# compiler copies every accumulator block in and out of AGPRs around each
# product (160+ extra moves per iteration), so the VGPR form is forced.
SOURCE_FLAGS = {
    "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}

# Kernels allowed to spill, with the reason.
SPILL_OK = {
    # fp32 inputs at d = 128: the register prefetch of a 64-key fp32 tile
    # (64 VGPRs) spills a few values; fp32 is the precision path, bf16 the
    # performance path
    "_ZN3swa12_GLOBAL__N_114prefill_kernelIfLi128EEEvNS_11PrefillArgsE",
    # the bf16 prefill with the global-key tile at d = 128 (task-bound
    # global tokens only): the tile after the band keeps the running max
    # alive through the band's last products, and two values held across the
    # band go to scratch (one reloaded in the masked-tile path); the plain
    # kernel, which every other call runs, has no spill
    "_ZN3swa12_GLOBAL__N_117prefill_pp_kernelILi128ELb1ELb0EEEvNS_11PrefillArgsE",
    # the bf16 prefill with the fused cache append at d = 128: with the band
    # walked rotated (one more scalar across the band) the query row's
    # address and two scalars of the query-reload path go to scratch and VGPR
    # lanes; that path runs at most once per work item (the switch from the
    # sink tile to the band without the sink turn), and the launches
    # measured no slower than without the rotation
    "_ZN3swa12_GLOBAL__N_117prefill_pp_kernelILi128ELb0ELb1EEEvNS_11PrefillArgsE",
}


def _check_resources(src: str, remarks: str) -> None:
    """Every kernel must run from registers: no scratch, no spills (a lambda
    the inliner leaves out of line, or an array indexed at run time, puts
    accumulators in scratch memory and costs far more than it looks)."""
    kernel = None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) != 0 and kernel not in SPILL_OK:
            raise RuntimeError("%s: kernel %s has %s = %s" % (src, kernel, m.group(1), m.group(2)))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + SOURCE_FLAGS.get(src, []) + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip",
                                                              "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    _check_resources(src, r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libswa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
