"""Build libflashattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m online_softmax_flash_amd.build`` (or ``build()`` from Python).
Every source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into ``online_softmax_flash_amd/libflashattn.so``.
``probe/mfma_peak.hip`` becomes ``libfaprobe.so``, the benchmark's
matrix-core throughput probe.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflashattn.so")
# Matrix-core throughput probe for the benchmark's roofline (not the library).
PROBE_SRC = os.path.join(PKG, "probe", "mfma_peak.hip")
PROBE_LIB = os.path.join(PKG, "libfaprobe.so")
ARCH = "gfx950"

# No packed fp32 arithmetic (v_pk_*_f32) in device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source additions: MFMA accumulators in VGPRs for the bf16 forward and
# the bf16 dQ kernel (fewer copies between the AGPR and VGPR files).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"fa_bwd_dq_bf16.hip": _VGPR_FORM, "fa_bwd_fused_bf16.hip": _VGPR_FORM, "fa_fwd_bf16.hip": _VGPR_FORM,
               "fa_fwd_kv_bf16.hip": _VGPR_FORM, "fa_naive_bf16.hip": _VGPR_FORM}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libflashattn.so)")
    return p


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libflashattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
