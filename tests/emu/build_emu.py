"""Builds the CPU emulation of the HIP library: _build/emu/libgpt2mi_emu.so.

TEST INFRASTRUCTURE ONLY.  The kernel and engine sources under
decoder_only_transformer_02_amd/csrc are copied with three mechanical
rewrites and compiled for the host against tests/emu/include/hip/hip_runtime.h:
  * `kernel<<<grid, block, shmem, stream>>>(args)` becomes
    `::emu::launch(kernel, grid, block, shmem, stream)(args)`;
  * `extern __shared__ T name[];` becomes a pointer to the block's dynamic LDS;
  * address-space and waves-per-EU attributes are dropped.
Nothing else in the sources changes.  The product library is never built or
loaded from here, and the product binding never loads this one.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "decoder_only_transformer_02_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "emu")
LIB = os.path.join(OUT_DIR, "libgpt2mi_emu.so")
CLANG = "/opt/rocm/llvm/bin/clang++"
EMU_SOURCES = ["emu_rt.cpp", "kernel_entry.cpp"]


def _match_back(text: str, end: int) -> int:
    """Start of the kernel expression whose last character is text[end - 1]."""
    i = end
    while i > 0 and text[i - 1].isspace():
        i -= 1
    if text[i - 1] == ">":  # template argument list
        depth = 0
        j = i - 1
        while j >= 0:
            if text[j] == ">":
                depth += 1
            elif text[j] == "<":
                depth -= 1
                if depth == 0:
                    break
            j -= 1
        i = j
    while i > 0 and (text[i - 1].isalnum() or text[i - 1] in "_:"):
        i -= 1
    return i


def rewrite(text: str) -> str:
    text = re.sub(r"__attribute__\(\(address_space\(3\)\)\)", "", text)
    text = re.sub(r"__attribute__\(\(amdgpu_waves_per_eu\([^)]*\)\)\)", "", text)
    text = re.sub(r"extern\s+__shared__\s+([\w:]+)\s+(\w+)\s*\[\s*\]\s*;",
                  r"\1* \2 = (\1*)::emu::dyn_shared();", text)
    out = []
    pos = 0
    while True:
        k = text.find("<<<", pos)
        if k < 0:
            out.append(text[pos:])
            break
        e = text.find(">>>", k)
        if e < 0:
            raise ValueError("unterminated launch configuration")
        s = _match_back(text, k)
        kernel = text[s:k].strip()
        cfg = text[k + 3:e]
        out.append(text[pos:s])
        out.append(f"::emu::launch({kernel}, {cfg})")
        pos = e + 3
    return "".join(out)


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))


def _digest() -> str:
    h = hashlib.sha256()
    for d, names in ((CSRC, _sources()), (HERE, EMU_SOURCES + ["emu_switch.S", "build_emu.py"]),
                     (os.path.join(HERE, "include", "hip"), ["hip_runtime.h"]),
                     (os.path.join(ROOT, "include"), sorted(os.listdir(os.path.join(ROOT, "include"))))):
        for n in names:
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def flags():
    return ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I", os.path.join(HERE, "include"),
            "-I", os.path.join(OUT_DIR, "src"), "-I", os.path.join(ROOT, "include"),
            "-I", CSRC,
            "-Wno-unknown-attributes", "-Wno-ignored-attributes", "-Wno-unused-command-line-argument",
            "-Wno-return-type-c-linkage", "-Wno-psabi", "-pthread"]


def build(force: bool = False, verbose: bool = False) -> str:
    os.makedirs(os.path.join(OUT_DIR, "src"), exist_ok=True)
    stamp = os.path.join(OUT_DIR, "stamp")
    dg = _digest()
    if not force and os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == dg:
        return LIB
    src_dir = os.path.join(OUT_DIR, "src")
    units = []
    for n in _sources():
        with open(os.path.join(CSRC, n)) as f:
            t = rewrite(f.read())
        dst = os.path.join(src_dir, n if n.endswith(".h") else n.replace(".hip", ".cpp"))
        with open(dst, "w") as f:
            f.write(t)
        if n.endswith(".hip"):
            units.append(dst)
    units += [os.path.join(HERE, s) for s in EMU_SOURCES]

    def cc(src):
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([CLANG, *flags(), "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"emulator build failed for {src}:\n{r.stderr[-6000:]}")
        if verbose and r.stderr.strip():
            print(r.stderr[-3000:])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(cc, units))
    asm = os.path.join(OUT_DIR, "emu_switch.o")
    r = subprocess.run([CLANG, "-c", os.path.join(HERE, "emu_switch.S"), "-o", asm],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    tmp = LIB + ".tmp"
    r = subprocess.run([CLANG, "-shared", "-fPIC", "-pthread", "-Wl,--no-undefined", "-o", tmp, *objs, asm],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"emulator link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    with open(stamp, "w") as f:
        f.write(dg)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose=True))
