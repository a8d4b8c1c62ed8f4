"""Compile the HIP library (gfx950) into bit_quantized_mamba_amd/libdfssm.so,
the stand-alone exchange-latency probe into bit_quantized_mamba_amd/hop_probe,
and the host CPU backend (g++, OpenMP) into bit_quantized_mamba_amd/libdfssm_host.so."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdfssm.so")
PROBE = os.path.join(HERE, "hop_probe")
HOST_SRC = os.path.join(HERE, "host", "dfssm_host.cpp")
HOST_OUT = os.path.join(HERE, "libdfssm_host.so")
CXX = os.environ.get("CXX_HOST", "g++")
# x86-64-v3 baseline (AVX2) for the shared code; the AVX-512 VNNI products are
# compiled per function and chosen at run time.  No floating-point
# contraction: the results do not depend on which path or CPU runs them.
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-march=x86-64-v3", "-ffp-contract=off"]
BUILD = os.path.join(HERE, "_build")
SOURCES = ["gen.hip", "kernels.hip", "persistent.hip", "gemm.hip", "scan.hip", "codec.hip", "runtime.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         # packed fp32 instructions stay off in every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", OUT + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    probe = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], os.path.join(CSRC, "hop_probe.hip"), "-o", PROBE + ".tmp"]
    r = subprocess.run(probe, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for hop_probe.hip:\n{r.stdout}{r.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    build_host()
    return OUT


def build_host() -> str:
    cmd = [CXX, *HOST_FLAGS, HOST_SRC, "-o", HOST_OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{CXX} failed for dfssm_host.cpp:\n{r.stdout}{r.stderr}")
    os.replace(HOST_OUT + ".tmp", HOST_OUT)
    return HOST_OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
