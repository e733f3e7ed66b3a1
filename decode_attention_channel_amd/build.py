"""Build libkivi.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["kivi_api.hip", "quantize.hip", "decode_attn.hip"]
LIB = os.path.join(PKG, "libkivi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 ops anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # MFMA accumulators in VGPRs: the kernels stay well inside 256 registers,
    # and AGPR<->VGPR copies around the softmax rescale disappear
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # atomics stay as written: the LDS group counter is bumped by one lane,
    # and its result is consumed a step later, not right after the atomic
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    # per-kernel register / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]


def kernel_resources(remarks: str) -> dict:
    """{kernel: {"VGPRs": n, "ScratchSize": bytes per lane, ...}} from the
    compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkivi.so")
    # a kernel that lands in scratch memory (spills, or an argument copy with
    # an indexed member) runs several times slower: refuse to ship it.  (VGPR
    # spills into the AGPR half of the register file, which the largest head
    # blocks have, cost a register move each and use no memory.)
    res = kernel_resources(r.stderr)
    if not res:
        raise RuntimeError("no kernel resource report from hipcc")
    bad = {k: v for k, v in res.items() if v.get("ScratchSize", 0)}
    if bad:
        os.remove(tmp)
        raise RuntimeError(f"kernels using scratch memory: {bad}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
