"""Build libsas.so (gfx950) in-tree with hipcc.

Every ``*.hip`` file under ``csrc/`` is compiled for ``--offload-arch=gfx950``
and linked into one shared library next to this file.  Packed-fp32 ops are
disabled for device code (``-packed-fp32-ops`` off).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsas.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(HERE, "..", "include"), "-I" + CSRC]


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, build_dir: str = BUILD,
          extra_flags: tuple = (), link_flags: tuple = ()) -> str:
    """Compile every csrc/*.hip and link ``out``.  ``extra_flags`` /
    ``link_flags`` are appended to the compile / link lines (the host-side
    sanitizer build passes its options here and its own output path)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [cc, *flags(), *extra_flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *link_flags, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # A kernel whose host-side launch stub the compiler dropped leaves an
    # undefined __device_stub__ symbol that only fails when the library
    # registers its kernels on a GPU: refuse such a build here.
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-u", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the build: %s" % ", ".join(missing))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
