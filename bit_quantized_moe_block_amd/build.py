"""Build the gfx950 shared library libmoedecode.so in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoedecode.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("moe_decode.hip", "kernels.hip")]
# measurement probes (plain streaming read, empty kernels), a library of their own
PROBE_LIB = os.path.join(HERE, "libmoeprobe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "probes.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-I", os.path.join(ROOT, "include"),
    # Packed-fp32 VALU forms stay off (only scalar / MFMA fp32 arithmetic).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    # leading scalar kernel arguments arrive in scalar registers at launch
    # (the route and combine kernels put theirs first)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def build(verbose=False):
    _build_one(LIB, SOURCES, verbose)
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


def _build_one(lib, sources, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)


if __name__ == "__main__":
    build(verbose=True)
