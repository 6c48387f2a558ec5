"""Build libmk.so (the megakernel library and the one-kernel-per-op baseline) for gfx950 in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["graph.cpp", "prefill_graph.cpp", "runtime.cpp", "megakernel.hip", "baseline.hip", "micro.hip"]

# Packed-FP32 instructions are kept out of every kernel of this library.  Functions start on
# 256-byte boundaries: the decode step is sensitive to where its operations' code lands (measured
# on the 1B shape: 779.9 -> 778.0 us per step at batch 1, 1514.2 -> 1511.5 at batch 16).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-falign-functions=256", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False, out=None, extra_flags=()):
    """Compile every source and link libmk.so (always rebuilds).  out / extra_flags: another library
    path and extra compiler flags (e.g. -D overrides of tuning constants) for variant builds."""
    objs = []
    lib = out or LIB
    bdir = os.path.join(HERE, "_build") if out is None else os.path.splitext(out)[0] + "_build"
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + HIP_FLAGS + list(extra_flags) + lang + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "unused-command-line" not in l
                        and l.strip() != "1 warning generated.")
        if r.returncode != 0:
            sys.stderr.write(out + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if out.strip() and verbose:
            print(out)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp"] + objs
    subprocess.check_call(cmd)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
