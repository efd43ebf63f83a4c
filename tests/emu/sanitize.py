"""Builds the emulated library and tests/emu/san_driver.cpp into one host
executable instrumented with AddressSanitizer and UndefinedBehaviorSanitizer:
_build/emu_san/san_driver.  TEST INFRASTRUCTURE ONLY: the GPU library is never
built here.  The sources are rewritten exactly as for the emulator
(build_emu.rewrite); the sanitizers instrument the engine's host code and
the kernels' emulated code, with the heap standing in for device memory."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

from tests.emu import build_emu

OUT_DIR = os.path.join(build_emu.ROOT, "_build", "emu_san")
EXE = os.path.join(OUT_DIR, "san_driver")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build() -> str:
    os.makedirs(os.path.join(OUT_DIR, "src"), exist_ok=True)
    stamp = os.path.join(OUT_DIR, "stamp")
    dg = build_emu._digest() + str(os.path.getmtime(os.path.join(build_emu.HERE, "san_driver.cpp")))
    if os.path.exists(EXE) and os.path.exists(stamp) and open(stamp).read() == dg:
        return EXE
    src_dir = os.path.join(OUT_DIR, "src")
    units = []
    for n in build_emu._sources():
        with open(os.path.join(build_emu.CSRC, n)) as f:
            t = build_emu.rewrite(f.read())
        dst = os.path.join(src_dir, n if n.endswith(".h") else n.replace(".hip", ".cpp"))
        with open(dst, "w") as f:
            f.write(t)
        if n.endswith(".hip"):
            units.append(dst)
    units += [os.path.join(build_emu.HERE, s) for s in ("emu_rt.cpp", "san_driver.cpp")]
    fl = [f for f in build_emu.flags() if f not in ("-O2", "-fPIC", "-fvisibility=hidden")]
    fl = ["-O1", "-g", *SAN, *[("-I" if f == "-I" else f) for f in fl]]
    fl = [os.path.join(OUT_DIR, "src") if f == os.path.join(build_emu.OUT_DIR, "src") else f for f in fl]

    def cc(src):
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([build_emu.CLANG, *fl, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed for {src}:\n{r.stderr[-6000:]}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(cc, units))
    asm = os.path.join(OUT_DIR, "emu_switch.o")
    r = subprocess.run([build_emu.CLANG, "-c", os.path.join(build_emu.HERE, "emu_switch.S"), "-o", asm],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    r = subprocess.run([build_emu.CLANG, *SAN, "-pthread", "-o", EXE, *objs, asm], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr[-4000:]}")
    with open(stamp, "w") as f:
        f.write(dg)
    return EXE


if __name__ == "__main__":
    print(build())
