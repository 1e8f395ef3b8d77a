"""Build librmm.so (the HIP kernels and the C ABI of include/rmm.h) for gfx950.

    python -m input_adaptive_reduced_02_amd.build

Each csrc/*.hip is compiled on its own (in parallel) to _build/*.o with hipcc,
then linked into input_adaptive_reduced_02_amd/librmm.so.  Cross-compiles on a
machine without a GPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["rmm_api.hip", "rmm_score.hip", "rmm_select.hip", "rmm_gather.hip", "rmm_gemm.hip",
           "rmm_pv.hip", "rmm_q8.hip", "rmm_attn.hip"]


def _compile(src, objdir=OBJ, extra=(), csrc=CSRC):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, out=LIB, extra=(), objdir=OBJ, csrc=CSRC):
    """Compile every HIP source and link librmm.so (or `out`, with `extra`
    compiler flags, sources from `csrc` and objects in `objdir`); returns the
    library path."""
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda src: _compile(src, objdir, extra, csrc), SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
