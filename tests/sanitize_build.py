"""Builds of the host code with AddressSanitizer and UndefinedBehaviorSanitizer.

* the oracle: sas_oracle.c with clang, -fsanitize=address,undefined, serial
  (its OpenMP pragmas are ignored: the same arithmetic on one thread);
* libsas.so: every csrc/*.hip with the sanitizers on the host side only (each
  -fsanitize= option behind -Xarch_host, so the gfx950 device code is built
  exactly as in the product library), linked against the shared sanitizer
  runtime.
Outputs go to gated_block_sparse_sas_amd/_build/sanitize/.  The runtime
(clang's libclang_rt.asan) must be preloaded into the process that loads
them; ``runtime()`` returns its path.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "gated_block_sparse_sas_amd", "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found")
    return hits[-1]


def build_oracle() -> str:
    os.makedirs(OUT, exist_ok=True)
    out = os.path.join(OUT, "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "sas_oracle.c")
    subprocess.check_call([CLANG, "-O1", "-std=c99", *SAN, "-shared-libsan", "-fPIC", "-shared",
                           src, "-o", out, "-lm"])
    return out


def build_library() -> str:
    from gated_block_sparse_sas_amd import build as b
    host = []
    for f in SAN:
        host += ["-Xarch_host", f]
    return b.build(out=os.path.join(OUT, "libsas_san.so"), build_dir=os.path.join(OUT, "obj"),
                   extra_flags=tuple(host), link_flags=("-shared-libsan", *SAN))


if __name__ == "__main__":
    print(build_oracle())
    print(build_library())
