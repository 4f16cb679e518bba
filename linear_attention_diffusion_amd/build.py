"""Compile the HIP library libsana_linattn.so for gfx950, in-tree.

hipcc cross-compiles without a GPU.  The library lands in
linear_attention_diffusion_amd/_lib/ next to this file.
"""

import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_NAME = "libsana_linattn.so"
LIB_PATH = os.path.join(LIB_DIR, LIB_NAME)
SOURCES = ["sana_linattn.hip"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU ops; the
# host pass warns that it does not know the feature, which is harmless.
# -amdgpu-mfma-vgpr-form has MFMA write its results to ordinary VGPRs: the
# kernels convert most MFMA results with VALU right away, and results left in
# AGPRs would each cost a v_accvgpr_read first.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-command-line-argument",
]


def source_hash(csrc=CSRC):
    """sha256[:16] over the kernel sources in `csrc` (every *.h and *.hip, by
    name then content, in name order); compiled into the library, whose
    sana_linattn_source_hash() returns it."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build the HIP library")
    return exe


def build(verbose=False):
    """Compile every HIP source into LIB_PATH (always recompiles)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *FLAGS, f'-DSANA_SOURCE_HASH="{source_hash()}"', "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
