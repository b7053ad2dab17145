"""Build libqsa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m top_sparse_attention_pooled_amd.build [--stamps]

--stamps builds libqsa_stamps.so instead: the same library compiled with
QSA_STAMPS, whose kernels record per-workgroup phase timestamps (a
measurement build, read by ``profiling.py stamps``; never loaded otherwise).

Every translation unit is compiled with -ffp-contract=off (the fixed-order
fp32 arithmetic must not be fused) and with packed fp32 instructions disabled.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqsa.so")
# per-kernel VGPRs / scratch / occupancy reported by the compiler
RESOURCES = os.path.join(BUILD, "resources.json")
SOURCES = ["api.hip", "pooled.hip", "score.hip", "select.hip", "attn.hip", "attn_prefill.hip",
           "prefill.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # code object v5: loadable by the ROCm 7.0 runtime that torch bundles
    "-mcode-object-version=5",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")


def _resources(stderr: str) -> dict:
    """Kernel -> {VGPRs, AGPRs, scratch, occupancy, lds} from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for m in _REMARK.finditer(stderr):
        k, v = m.group(1), m.group(2)
        if k == "Function Name":
            cur = out.setdefault(v, {})
        elif cur is not None:
            cur[keys[k]] = int(v)
    return out


STAMPS_LIB = os.path.join(HERE, "libqsa_stamps.so")
STAMPS_BUILD = os.path.join(HERE, "_build_stamps")


def _compile(src: str, stamps: bool = False):
    obj = os.path.join(STAMPS_BUILD if stamps else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DQSA_STAMPS"] if stamps else []),
           "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(jobs: int = 8, stamps: bool = False) -> str:
    """Compile every source and link libqsa.so, or libqsa_stamps.so with
    stamps=True (always rebuilds)."""
    os.makedirs(STAMPS_BUILD if stamps else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        results = list(ex.map(lambda src: _compile(src, stamps), SOURCES))
    objs = [o for o, _ in results]
    lib = STAMPS_LIB if stamps else LIB
    if not stamps:
        res = {k: v for _, r in results for k, v in r.items()}
        with open(RESOURCES, "w") as f:
            json.dump(res, f, indent=1, sort_keys=True)
        spills = sorted(k for k, v in res.items() if v.get("scratch", 0) > 0)
        if spills:  # a spilled register array turns a register-resident loop into memory traffic
            print(f"warning: kernels using scratch memory: {spills}", file=sys.stderr)
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared",
                        "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--stamps"]
    print(build(int(args[0]) if args else 8, stamps="--stamps" in sys.argv[1:]))
