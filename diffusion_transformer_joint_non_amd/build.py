"""Build libjpa.so in-tree for gfx950 with hipcc.

    python -m diffusion_transformer_joint_non_amd.build

The library lands in ``diffusion_transformer_joint_non_amd/_lib/libjpa.so``;
the Python binding loads it from there and nowhere else.  A check build of the
same sources, ``libjpa_strict_waits.so`` (JPA_STRICT_WAITS: the attention
kernel waits for every tile copy at each barrier), is built beside it for the
GPU test that compares the two bit for bit.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libjpa.so")
STRICT_LIB = os.path.join(LIB_DIR, "libjpa_strict_waits.so")
ARCH = "gfx950"

SOURCES = ["jpa_kernel.hip", "jpa_scratch.hip", "jpa_host.cpp", "jpa_norm_rope.hip", "jpa_norm_rope_host.cpp",
           "jpa_shard_host.cpp", "jpa_cat_pad.hip", "jpa_cat_pad_host.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # MFMA results in VGPRs: the softmax reads the scores with no AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libjpa")
    return path


def build(verbose: bool = True, extra_flags=None, lib: str = LIB) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = True) -> list:
    """The library and its strict-waits check build, compiled side by side."""
    with ThreadPoolExecutor(2) as ex:
        jobs = [ex.submit(build, verbose),
                ex.submit(build, verbose, ["-DJPA_STRICT_WAITS"], STRICT_LIB)]
        return [j.result() for j in jobs]


if __name__ == "__main__":
    print("\n".join(build_all()))
