"""Build libmq.so (and the benchmark's calibration probes, libmq_probe.so)
in-tree with hipcc for gfx950.

    python -m quantized_moe_grouped_amd.build        (or __graft_entry__.build())

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass prints a
harmless "not a recognized feature" warning for it.  The quantiser and the
router are built with ``-ffp-contract=off`` so that no fused multiply-add can
change a rounding the oracle performs in two steps.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmq.so")
PROBE_LIB = os.path.join(HERE, "libmq_probe.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = os.environ.get("MQ_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", CSRC, "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-fast-math", "-Wall", "-Wno-unused-function"]
SOURCES = {
    "quantize.hip": ["-ffp-contract=off"],
    "route.hip": ["-ffp-contract=off"],
    # keep MFMA results in VGPRs: the per-group epilogue reads every one of
    # them, and an AGPR would cost an extra v_accvgpr_read per value
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "small_m.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gather_mm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gather_mx.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gather_nn.hip": [],
    "noalloc.hip": [],
    "api.cpp": [],
}
# the calibration probes: a library of their own (the benchmark loads it)
PROBE_SOURCES = {"probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmq.so)")


def _compile(hipcc: str, src: str, extra: list[str]) -> tuple[str, str]:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def _link(hipcc: str, objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source, link libmq.so and libmq_probe.so; returns
    the path of libmq.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    every = {**SOURCES, **PROBE_SOURCES}
    with cf.ThreadPoolExecutor(max_workers=min(6, len(every))) as ex:
        futs = {s: ex.submit(_compile, hipcc, s, e) for s, e in every.items()}
        objs = {}
        for s, f in futs.items():
            obj, err = f.result()
            objs[s] = obj
            if verbose and err.strip():
                print(err, file=sys.stderr)
    _link(hipcc, [objs[s] for s in SOURCES], LIB)
    _link(hipcc, [objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
