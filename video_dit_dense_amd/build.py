"""Build step: compiles the HIP sources under csrc/ into libh3attn.so (gfx950
only) next to this file. Run `python -m video_dit_dense_amd.build`."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libh3attn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # Scores and activations are finite or -inf: no NaN canonicalisation in max.
    "-fno-honor-nans",
    # No packed fp32 VALU ops anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results in architectural vector registers, where the softmax
    # reads its scores without copies and the QK^T accumulator starts from
    # the row offset in place.
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))


def build(verbose: bool = False) -> str:
    """Compile every source into one shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    # The library must resolve every symbol: a kernel whose host-side launch
    # stub the compiler dropped (device-only builtins in its body) links but
    # fails to load.
    chk = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load:\n{chk.stderr.strip()[-2000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
