"""Builds the HIP library libgpt2mi.so (gfx950) in-tree with hipcc.

Each source is compiled separately (in parallel) into _build/, then linked
into decoder_only_transformer_02_amd/libgpt2mi.so.  Packed-fp32 VALU
instructions are disabled for all device code.  The compiler's per-kernel
resource report (registers, scratch, LDS, occupancy) is kept in
_build/kernel_resources.json, which a CPU test checks.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libgpt2mi.so")
SOURCES = ["elementwise.hip", "gemm.hip", "attention.hip", "decode.hip", "engine.hip"]
ARCH = "gfx950"
# Per-source code generation options.  The attention kernels keep their
# MFMA accumulators and results in ordinary VGPRs: by default the compiler
# put them in AGPRs and copied them to VGPRs and back every key tile for
# the softmax (272 accumulator moves in the forward's loop, 192 in dQ's),
# and dQ fits three waves per SIMD instead of two this way.  The GEMM tiles
# need the AGPRs for capacity and keep the default.
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
           "LDS Size [bytes/block]": "lds", "Occupancy [waves/SIMD]": "occupancy"}


def parse_resources(stderr: str) -> dict:
    """Kernel (mangled name) -> {vgpr, agpr, scratch, lds, occupancy} from
    the -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\d+)", line)
        if m and cur is not None and m.group(1).strip() in _FIELDS:
            cur[_FIELDS[m.group(1).strip()]] = int(m.group(2))
    return {k: v for k, v in out.items() if v}


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *flags(), *EXTRA.get(src, []), "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose:
            rest = [ln for ln in r.stderr.splitlines() if "remark" not in ln]
            if any(ln.strip() for ln in rest):
                print("\n".join(rest))
        return obj, parse_resources(r.stderr)

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        done = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in done]
    res = {}
    for _, d in done:
        res.update(d)
    with open(os.path.join(bdir, "kernel_resources.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
