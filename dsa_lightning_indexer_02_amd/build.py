"""Compile the HIP kernels and the C ABI into dsa_lightning_indexer_02_amd/libdsa.so (gfx950)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of every kernel (compiler-generated ones included).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall",
         "-Wno-unused-command-line-argument", "-munsafe-fp-atomics"] + DEVICE_FLAGS


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Per-source flags.  The sparse-MLA kernel issues its gather DMA as inline assembly, and keeps
# its MFMA accumulators in the architectural VGPRs (the score tiles are read by VALU code right
# after each product, which the accumulation-register form would turn into copies).
PER_SOURCE = {"sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Wno-inline-asm"]}


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *PER_SOURCE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for %s" % src)
    return obj


def build(out: str = LIB, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), sources()))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
