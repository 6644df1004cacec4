"""Build libdg.so (the C-ABI library with the gfx950 kernels) in-tree.

Each csrc/*.hip is compiled by hipcc for gfx950 and the objects are linked into
uniform_state_discrete_amd/libdg.so against the HIP runtime that torch loads
(torch ships its own libamdhip64.so), so a process that uses torch for device
memory and streams has a single HIP runtime and torch's stream handles are
valid arguments.

    python -m uniform_state_discrete_amd.build [--verbose]
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-source flags.  The 16-row d = 4096 vocabulary kernel uses the
# scheduler's ILP strategy: about 4% faster there, while the CU-pair kernel
# (in k_vocab.hip, default strategy) measured no gain and more waiting with it.
SOURCE_FLAGS = {
    "k_vocab16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdg)")


def torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is required (its HIP runtime is the one libdg links against)")
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {d}: torch must be a ROCm build")
    return d


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj])

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return r.stderr

    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        for err in ex.map(run, cmds):
            if verbose and err.strip():
                print(err)
    tl = torch_lib_dir()
    tmp = LIB + ".tmp"
    link = ["g++", "-shared", "-o", tmp, *objs, f"-L{tl}", "-l:libamdhip64.so",
            f"-Wl,-rpath,{tl}", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
