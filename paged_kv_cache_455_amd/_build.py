"""Build the HIP library ``libpa.so`` in-tree for gfx950 with hipcc.

Every translation unit under ``csrc/`` (``.hip`` kernels, ``.cpp`` host code) is
compiled to an object (in parallel)
and linked into ``paged_kv_cache_455_amd/libpa.so``.  Run as
``python -m paged_kv_cache_455_amd._build``.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the attention kernels rescale and read
    # them with VALU ops every key step, which AGPR accumulators would turn into
    # copies back and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host modules that need no HIP runtime: they also build with g++ on their own.
HOST_ONLY = ("status.cpp", "block_manager.cpp")


def build_host_sanitized(out_path: str) -> str:
    """The host-only modules (the block manager and status reporting) as a shared
    library built by g++ with AddressSanitizer and UndefinedBehaviorSanitizer, for
    CPU test runs of the block manager (load it with the sanitizer runtimes
    preloaded; it exports only the pa_bm_* and status calls)."""
    srcs = [os.path.join(CSRC, f) for f in HOST_ONLY]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           *srcs, "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed:\n{r.stdout}\n{r.stderr}")
    return out_path


if __name__ == "__main__":
    build()
