"""Build librowstats.so (HIP, gfx950) in-tree with hipcc."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librowstats.so")
# the streaming-ceiling kernels timed by bench.py --ceiling (measurement only)
CEILING_SRC = os.path.join(CSRC, "ceiling", "stream_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libstreamceiling.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics stay single instructions: the atomic optimizer would turn a
    # one-lane counter claim into a wave reduction that waits for its result
    # (and so for every memory operation in flight) right where it is issued
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-pragmas",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(out: str, srcs, verbose: bool):
    cmd = [HIPCC, *FLAGS, "-o", out + ".tmp", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-6000:]}")
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    _hipcc(CEILING_LIB, [CEILING_SRC], verbose)
    return _hipcc(LIB, sources(), verbose)


if __name__ == "__main__":
    print(build(verbose=True))
