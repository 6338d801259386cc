"""Build librea.so in-tree with hipcc for gfx950.

    python -m top_kv_cache_amd._build
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librea.so")

SOURCES = ["rea_api.cpp", "score.hip", "score_mfma.hip", "topk.hip", "window.hip", "attend.hip", "attend_mfma.hip",
           "decode_attend.hip", "noalloc.hip", "probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel, then link the library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="rea_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *compile_flags, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(compile_one, SOURCES))
        for _, r in results:
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc failed building librea.so")
        cmd = [hipcc, *FLAGS, *extra, "-o", LIB + ".tmp", *[o for o, _ in results]]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking librea.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
