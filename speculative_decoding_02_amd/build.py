"""Builds libspec.so (HIP, gfx950) in-tree with hipcc."""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "libspec")
LIB = os.path.join(HERE, "libspec.so")
RUNNER = os.path.join(HERE, "spec_run")   # native driver of the C ABI (no Python in the process)
SOURCES = ["k_gemm.hip", "k_attn.hip", "k_misc.hip", "k_accept.hip", "k_ngram.hip", "k_gemm_rows.hip",
           "k_gemm_wide.hip", "k_heads.hip", "k_batch.hip", "spec_api.cpp", "spec_batch.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("SPEC_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs (gfx950)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-file additions: the wide rows GEMM keeps its MFMA accumulators in VGPRs
# (with them in AGPRs the compiler copies every accumulator at each k-block).
FILE_FLAGS = {"k_gemm_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        # host pass warns about the packed-fp32 target feature; show other warnings
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines), file=sys.stderr)
    return obj


# Host code built with AddressSanitizer + UndefinedBehaviorSanitizer (device
# code unchanged), loaded instead of LIB when SPEC_LIBSPEC points at it
# (tests/run_sanitizers.sh).
SAN_OBJ = os.path.join(ROOT, "_build", "sanitize", "libspec")
SAN_LIB = os.path.join(ROOT, "_build", "sanitize", "libspec.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_OBJ, exist_ok=True)
    host = [s for s in SOURCES if s.endswith(".cpp")]

    def comp(src):
        obj = os.path.join(SAN_OBJ, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *SAN_FLAGS, "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(comp, host))
    kern = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, *objs, *kern,
           "-o", SAN_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    # the native driver links the library by its in-tree path
    cmd = [HIPCC, *FLAGS, "-x", "hip", os.path.join(CSRC, "spec_run.cpp"), "-x", "none",
           "-L", HERE, "-lspec", "-Wl,-rpath,$ORIGIN", "-o", RUNNER + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for spec_run.cpp:\n{r.stdout}\n{r.stderr}")
    os.replace(RUNNER + ".tmp", RUNNER)
    return LIB


if __name__ == "__main__":
    print(build_sanitized(verbose=True) if "--sanitize" in sys.argv else build(verbose=True))
