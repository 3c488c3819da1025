"""Build libtreeverify.so (gfx950) in-tree with hipcc.

    python -m tree_verification_best_amd.build        # or build() from Python

Kernel files that take integer decisions from floating point (the tree
builder and the acceptance walk) are compiled with -ffp-contract=off so that
every float operation is the single IEEE operation written in the source.
All HIP code is compiled without packed-fp32 instructions.  The attention
file assumes no NaN inputs (-fno-honor-nans), so float max needs no operand
canonicalisation.
"""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtreeverify.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]
SOURCES = {
    "tv_build.hip": ["-ffp-contract=off"],
    "tv_accept.hip": ["-ffp-contract=off"],
    "tv_attention.hip": ["-fno-honor-nans"],
    "tv_commit.hip": [],
    "tv_api.cpp": ["-ffp-contract=off", "-x", "hip"],
}


def _compile(src, extra, verbose, objdir=BUILD, host_flags=()):
    obj = os.path.join(objdir, src + ".o")
    host = [f for flag in host_flags for f in ("-Xarch_host", flag)]
    cmd = ["hipcc"] + COMMON + extra + host + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose: bool = False, lib: str = LIB, objdir: str = BUILD, host_flags=()) -> str:
    """Compile every source and link `lib`.  `host_flags` go to the host
    compilation and the link only (e.g. a sanitizer build of the host code
    into another directory); the device code is the same."""
    os.makedirs(objdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose, objdir, host_flags),
                           SOURCES.items()))
    tmp = lib + ".tmp"
    cmd = (["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC"] + list(host_flags) +
           ["-o", tmp] + objs)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
