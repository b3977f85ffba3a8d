"""Build libmoe_mi355x.so in-tree: hipcc compiles every csrc/*.hip for gfx950,
g++ links the objects against the HIP runtime that torch loads (so one HIP
runtime serves torch's allocations, streams and these kernels)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    # packed fp32 arithmetic stays off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is required to locate the HIP runtime it loads")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    if verbose and r.stderr.strip():
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, defines=(), build_dir: str = BUILD,
          csrc: str = CSRC) -> str:
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *HIP_FLAGS, *["-D" + d for d in defines], "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tl = _torch_lib_dir()
    tmp = out + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, "-L" + tl, "-l:libamdhip64.so",
          "-Wl,-rpath," + tl, "-Wl,--no-undefined"], verbose)
    os.replace(tmp, out)
    return out


def _wait(item, verbose):
    cmd, p = item
    out, err = p.communicate()
    if p.returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError("compile failed: " + " ".join(cmd))
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in err.splitlines() if noise not in l)
    if verbose and msg.strip():
        sys.stderr.write(msg + "\n")


if __name__ == "__main__":
    print(build(verbose=True))
