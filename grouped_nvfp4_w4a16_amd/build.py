"""Build libmoe_w4a16.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: python -m grouped_nvfp4_w4a16_amd.build [--verbose]
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libmoe_w4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = os.environ.get("MOE_W4A16_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> list[str]:
    csrc = os.path.join(PKG_DIR, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))


def hashed_files() -> list[str]:
    """Every file the library is compiled from: the sources, their headers and the C ABI."""
    csrc = os.path.join(PKG_DIR, "csrc")
    return sorted(sources() + glob.glob(os.path.join(csrc, "*.h")) +
                  glob.glob(os.path.join(ROOT, "include", "*.h")))


def source_sha256() -> str:
    """SHA-256 over the names and contents of hashed_files(). The build compiles it into
    the library (moe_w4a16_source_sha256), so a loaded library can be matched to the
    sources on disk."""
    import hashlib

    h = hashlib.sha256()
    for path in hashed_files():
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def built_source_sha256(path: str = LIB_PATH) -> str | None:
    """The source hash a built library carries, read from the file's bytes (the library is
    not loaded: a process must load its HIP runtime through torch first). None if absent."""
    import re

    try:
        data = open(path, "rb").read()
    except OSError:
        return None
    m = re.search(rb"moe_w4a16_source_sha256=([0-9a-f]{64})", data)
    return m.group(1).decode() if m else None


def command(out_path: str) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # Packed FP32 VALU forms stay off: only scalar FP32 instructions are emitted.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
        f"-I{os.path.join(ROOT, 'include')}",
        f"-I{os.path.join(PKG_DIR, 'csrc')}",
        f'-DMOE_W4A16_SOURCE_SHA256="{source_sha256()}"',
        *sources(),
        "-o", out_path,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles). Returns the path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
