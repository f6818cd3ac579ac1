"""Build libspecverify.so (gfx950) in-tree with hipcc.

    python -m draft_verify_sampling_amd.build [--sanitize | --timeline]

Every HIP translation unit is compiled with packed fp32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.

--sanitize builds a copy whose host code (the C ABI's argument checks, the
workspace carve-up, the launch set-up) carries AddressSanitizer and
UndefinedBehaviorSanitizer checks, into _build/san/libspecverify.so; the
device code is built as usual.  A process loads it with the sanitizer
runtime preloaded (see sanitizer_env).

--timeline builds a copy whose walk, statistics and draw kernels record
in-kernel timestamps (csrc/timeline.hpp), into
draft_verify_sampling_amd/libspecverify_timeline.so; `bench.py --timeline`
loads it.  The normal library's kernels are the same code without them.
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
SAN_LIB = os.path.join(ROOT, "_build", "san", "libspecverify.so")
TIMELINE_LIB = os.path.join(HERE, "libspecverify_timeline.so")
# host-side sanitizers only: each flag applies to the host compilation pass
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
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


def build(verbose: bool = False, out: str = None, sanitize: bool = False, timeline: bool = False) -> str:
    """Compile every source to an object under _build/ (_build/san/ for the
    sanitized copy, _build/timeline/ for the timestamped one) and link the
    shared library; returns its path.  Always recompiles."""
    out = out or (SAN_LIB if sanitize else TIMELINE_LIB if timeline else LIB)
    sub = "san" if sanitize else "timeline" if timeline else ""
    bdir = os.path.join(ROOT, "_build", sub) if sub else os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cc = hipcc()
    extra = SAN_FLAGS if sanitize else ["-DSV_TIMELINE"] if timeline else []

    def one(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stdout.strip() or r.stderr.strip()):
            print(r.stdout, r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp"
    link_extra = ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] \
        if sanitize else []
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


def sanitizer_env(env: dict) -> dict:
    """Environment for a process that loads the sanitized library: its path
    in SPECVERIFY_LIB and the AddressSanitizer runtime (which carries the
    UndefinedBehaviorSanitizer handlers too) preloaded ahead of whatever was
    preloaded already."""
    cc = hipcc()
    rt = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not rt or not os.path.exists(rt):
        raise RuntimeError("AddressSanitizer runtime not found")
    env = dict(env)
    env["SPECVERIFY_LIB"] = SAN_LIB
    env["LD_PRELOAD"] = " ".join(x for x in (rt, env.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:protect_shadow_gap=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:], timeline="--timeline" in sys.argv[1:])
