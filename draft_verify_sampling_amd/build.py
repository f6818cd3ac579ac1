"""Build libspecverify.so (gfx950) in-tree with hipcc.

    python -m draft_verify_sampling_amd.build

Every HIP translation unit is compiled with packed fp32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["api.cpp", "k_stats.hip", "k_draw.hip", "k_walk.hip", "k_greedy.hip", "k_ngram.hip", "k_tree_build.hip", "k_shard.hip", "noalloc.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str = LIB) -> str:
    """Compile every source to an object under _build/ and link the shared
    library; returns its path.  Always recompiles."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stdout.strip() or r.stderr.strip()):
            print(r.stdout, r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
