"""Build the HIP library (libgpt2mi.so) in-tree for gfx950 with hipcc.

Every source is compiled on each call (objects in parallel), then linked into
decoder_only_transformer_04_amd/libgpt2mi.so.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgpt2mi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["layout.cpp", "gemm.hip", "elementwise.hip", "attention_simple.hip", "attention_mfma.hip", "generate.hip", "dropout.hip",
           "data.hip", "gpt2.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         # packed fp32 ALU ops stay off (hipcc's host pass warns that it does not know the feature)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results in ordinary VGPRs: the attention kernels read every score
         # accumulator with VALU code, and AGPR results cost one v_accvgpr move
         # per element and iteration (and, in the dK/dV kernel, a second wave per SIMD)
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip" if src.endswith(".hip") else "c++", "-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
