"""Build the HIP library in-tree: mla_decode_concat_amd/libmla_dq.so (gfx950).

The library carries a digest of the sources it was built from
(mla_dq_source_digest()), so that a library left over from other sources is
refused when it is loaded instead of being tested or timed.
"""
from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_dq.so")
SOURCES = [os.path.join(CSRC, "mla_dq_api.hip"), os.path.join(CSRC, "mla_dq_kernel.hip"),
           os.path.join(CSRC, "mla_dq_uk.hip"), os.path.join(CSRC, "mla_attn.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # each fp32 product and sum of the rotation rounds on its own
    "-ffp-contract=off",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def source_files(pkg: str = PKG, root: str = ROOT) -> list[str]:
    """Every file the library is compiled from: csrc/ and include/ headers."""
    files = glob.glob(os.path.join(pkg, "csrc", "*.hip")) + glob.glob(os.path.join(pkg, "csrc", "*.h"))
    files += glob.glob(os.path.join(root, "include", "*.h"))
    return sorted(files, key=lambda f: os.path.relpath(f, root))


def source_digest(pkg: str = PKG, root: str = ROOT) -> str:
    """SHA-256 (hex, first 32 digits) over the names and bytes of the sources."""
    h = hashlib.sha256()
    for f in source_files(pkg, root):
        h.update(os.path.relpath(f, root).replace(os.sep, "/").encode() + b"\0")
        with open(f, "rb") as fh:
            data = fh.read()
        h.update(len(data).to_bytes(8, "little") + data)
    return h.hexdigest()[:32]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the gfx950 library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libmla_dq.so (always recompiles)."""
    tmp = LIB + ".tmp"
    digest = f'-DMLA_DQ_SOURCE_DIGEST="{source_digest()}"'
    cmd = [hipcc(), *HIPCC_FLAGS, digest, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
