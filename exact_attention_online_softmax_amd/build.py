"""Build libosm.so (the gfx950 kernels and the C ABI) in-tree with hipcc, and
libosm_probe.so (the benchmark's reference copy and matrix-core kernels).

Usage: python -m exact_attention_online_softmax_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIBRARY = os.path.join(HERE, "libosm.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["abi.cpp", "layout.cpp", "softmax_rows.hip", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "decode.hip", "merge_lse.hip"]
ARCH = "gfx950"
PROBE_SOURCE = "probe.hip"
PROBE_LIBRARY = os.path.join(HERE, "libosm_probe.so")

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# per-file extra flags.  The attention kernel never lets a NaN reach its
# arithmetic (padding rows are never loaded, masked scores are -inf), so it
# runs with the IEEE mode bit off: max/min then need no NaN-quieting of their
# inputs.  Its score MFMAs must write VGPRs (the softmax reads them), so the
# compiler is told to select the VGPR form of the MFMA builtins; the output
# accumulators stay in AGPRs through inline assembly.  The FP8 forward is
# built the same way, for the same reasons, and so is the backward (its
# gradient accumulators are the AGPR-resident ones).
EXTRA = {"attn_fwd.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=true"],
         "attn_fwd_fp8.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=true"],
         "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", "-x", "hip", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        # warnings other than the host pass not knowing the gfx-only feature
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    # the benchmark's reference kernels (copy, matrix-core loop): their own library
    obj = _compile(PROBE_SOURCE)
    tmp = PROBE_LIBRARY + ".tmp"
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIBRARY)
    if verbose:
        print(f"built {LIBRARY} and {PROBE_LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build()
