"""Build libpaged_attn.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpaged_attn.so")
# sha256 of the sources and flags the library was built from, written beside it
STAMP = LIB + ".srchash"
SOURCES = [os.path.join(CSRC, "paged_attn.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-fp32 VALU forms stay off in all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def source_hash(extra=()) -> str:
    """sha256 over every source, header and compile flag the library is built
    from (file contents, not modification times, so a copied tree keeps it)."""
    h = hashlib.sha256()
    deps = sorted(set(SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC)] +
                      [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]))
    for d in deps:
        if os.path.isfile(d):
            h.update(os.path.relpath(d, ROOT).encode())
            with open(d, "rb") as fh:
                h.update(fh.read())
    h.update(" ".join(compile_flags() + list(extra)).encode())
    return h.hexdigest()


def build(out: str = LIB, extra=()) -> str:
    """Compile every HIP source of the library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + list(extra) + SOURCES + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    if out == LIB and not extra:
        with open(STAMP + ".tmp%d" % os.getpid(), "w") as fh:
            fh.write(source_hash() + "\n")
        os.replace(STAMP + ".tmp%d" % os.getpid(), STAMP)
    return out


def lib_is_current() -> bool:
    """True when the built library exists and was built from the current sources."""
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return False
    with open(STAMP) as fh:
        return fh.read().strip() == source_hash()


if __name__ == "__main__":
    print(build())
