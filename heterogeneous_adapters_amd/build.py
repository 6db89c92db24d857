"""Build liblora.so for gfx950 with hipcc (in-tree, next to this file).

The library links the HIP runtime that ships with the installed torch
package, so a process that imports torch and loads liblora maps exactly one
libamdhip64 and torch's hipStream_t handles are valid inside the library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "liblora.so")
SOURCES = [os.path.join(CSRC, "lora_kernels.hip"), os.path.join(CSRC, "lora_abi.cpp"),
           os.path.join(CSRC, "lora_pool.cpp"), os.path.join(CSRC, "lora_noalloc.hip")]
ARCH = "gfx950"


def torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is required to link the HIP runtime it ships")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra=(), out: str = None) -> str:
    tl = torch_lib_dir()
    out = out or os.path.join(HERE, "liblora.so")
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 VALU instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
           f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp,
           f"-L{tl}", f"-Wl,-rpath,{tl}", "-lamdhip64", *extra]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
