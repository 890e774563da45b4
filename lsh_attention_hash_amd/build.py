"""Build the HIP library liblsh_attn.so for gfx950 (in-tree).

    python -m lsh_attention_hash_amd.build

Each .hip source under csrc/ is compiled to an object in parallel, then linked
into lsh_attention_hash_amd/_lib/liblsh_attn.so. hipcc cross-compiles, so this
runs without a GPU.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "liblsh_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Device pass only: no packed-fp32 instructions in device code. Each source is
# compiled in two passes (device code object, then the host object that
# embeds it) so this target feature never reaches the x86 host compiler; both
# passes get the same compilation-unit id, so the host registers exactly the
# device symbols (kernels, static device arrays) of its own device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source extra flags. The hash kernel folds every MFMA result with vector
# instructions; with the accumulators in ordinary VGPRs it reads them in
# place instead of copying each one out of the accumulation registers.
EXTRA_FLAGS = {
    "hash_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "backward_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attend_variants.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, src):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return r.stderr


def _compile(src: str, csrc: str = CSRC, obj_dir: str = OBJ_DIR) -> str:
    base = os.path.basename(src)[:-4]
    obj = os.path.join(obj_dir, base + ".o")
    fatbin = os.path.join(obj_dir, base + ".hipfb")
    cuid = "cuid=" + hashlib.sha1(os.path.relpath(src, ROOT).encode()).hexdigest()[:16]
    flags = [f if f != CSRC else csrc for f in CFLAGS]
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    warnings = _run([HIPCC, "-x", "hip", *flags, f"-{cuid}", "--cuda-device-only", *DEVICE_FLAGS,
                     *extra, "-c", src, "-o", fatbin], src)
    warnings += _run([HIPCC, "-x", "hip", *flags, f"-{cuid}", "--cuda-host-only", "-Xclang",
                      "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", src, "-o", obj], src)
    if warnings.strip():
        print(f"{os.path.basename(src)}:\n{warnings}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
