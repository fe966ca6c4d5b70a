"""Build the gfx950 HIP library librouter_gemm_amd.so in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librouter_gemm_amd.so")
# Host code built with AddressSanitizer + UBSan (device code unchanged), for the
# CPU tests of the C ABI's validation (tests/run_sanitized.py); never the product.
LIB_SAN = os.path.join(PKG, "librouter_gemm_amd_san.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are disabled for device code (-packed-fp32-ops); the
# host pass warns that it does not know the feature, which is harmless.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


# Per-file flags.  The grouped GEMMs fold each fp8 block product into fp32
# accumulators with VALU FMAs; selecting the VGPR form of MFMA keeps those
# products out of AGPRs (no AGPR read-back per product).
EXTRA = {
    "expert_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "expert_gemm_tiled.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "expert_gemm_tiled_mx.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".san.o" if sanitize else ".o"))
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    san = SAN_HOST if sanitize else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), *san, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
