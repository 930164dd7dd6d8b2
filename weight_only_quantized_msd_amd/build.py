"""Build step for the HIP library ``libwqbmm.so`` (gfx950 only).

Every source is compiled with hipcc for --offload-arch=gfx950 with
-ffp-contract=off (the MSD expansion must be rounded exactly as written; the
kernels spell out the fused multiply-adds they want) and with the packed-fp32
target feature disabled.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(_HERE, "libwqbmm.so")
SOURCES = ["msd_api.cpp", "msd_prepack.hip", "msd_prepass.hip", "msd_prefill.hip", "msd_prefill64.hip",
           "msd_decode.hip", "msd_decode_gemv.hip", "msd_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the fused epilogues read every accumulator, and
    # the AGPR form costs one v_accvgpr_read per value
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_host_sanitized(verbose: bool = False) -> str:
    """libwqbmm_san.so: the library with its host code (msd_api.cpp: argument
    validation, dispatch, workspace bookkeeping) built with AddressSanitizer
    and UndefinedBehaviorSanitizer; device code and the kernel objects are the
    normal ones (build() must have run).  The process that loads it must
    preload clang's ASan runtime.  The sanitizers apply to host code only."""
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "msd_api.cpp"]
    for o in objs:
        if not os.path.exists(o):
            raise RuntimeError(f"{o} missing: run build() first")
    api_obj = os.path.join(BUILD_DIR, "msd_api_san.o")
    cmd = [HIPCC, "-x", "hip"] + CFLAGS + ["-g", "-Xarch_host", "-fsanitize=address",
                                             "-Xarch_host", "-fsanitize=undefined",
                                             "-Xarch_host", "-fno-sanitize-recover=all",
                                             "-c", os.path.join(CSRC, "msd_api.cpp"), "-o", api_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on msd_api.cpp (sanitized):\n{r.stdout}\n{r.stderr}")
    out = os.path.join(_HERE, "libwqbmm_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", out + ".tmp", api_obj] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
