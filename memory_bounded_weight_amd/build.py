"""Build the HIP C-ABI library ``libpsi.so`` for gfx950, in-tree.

``python -m memory_bounded_weight_amd.build`` compiles every source under
``csrc/`` with hipcc (cross-compiling on a machine without a GPU works).
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpsi.so")
ARCH = os.environ.get("PSI_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instruction selection; epilogue arithmetic stays plain
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


def hip_runtime_dir():
    """Directory of the HIP runtime the library must share with its caller.

    PyTorch-ROCm ships its own libamdhip64.so; a process must not hold two
    HIP runtimes (their streams would not be ordered with each other), so the
    library links against torch's copy when torch is installed, else the
    system ROCm one.  PSI_HIP_RUNTIME_DIR overrides."""
    d = os.environ.get("PSI_HIP_RUNTIME_DIR")
    if d:
        return d
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            lib = os.path.join(os.path.dirname(spec.origin), "lib")
            if os.path.exists(os.path.join(lib, "libamdhip64.so")):
                return lib
    except Exception:
        pass
    return "/opt/rocm/lib"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build", "psi")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc, "-x", "hip", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    rt = hip_runtime_dir()
    clangxx = os.environ.get("PSI_CLANGXX", "/opt/rocm/llvm/bin/clang++")
    # plain host link (no implicit --hip-link, which would add the system
    # runtime): the device code is already embedded in the objects
    link = [clangxx, "-shared", "-fPIC", "-o", LIB + ".tmp", *objs,
            "-L" + rt, "-l:libamdhip64.so", "-Wl,-rpath," + rt, "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if verbose and lines:
        print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
