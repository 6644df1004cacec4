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


# Host-side AddressSanitizer (the device code is compiled as usual): every
# sanitizer flag applies to the host pass only.
HOST_ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-g"]


def build(verbose=False, host_asan=None):
    """Compile every source for gfx950 and link libdg.so in the package.
    host_asan: a path; then the host code is built with AddressSanitizer
    into that library instead (load it through DG_LIB, with the clang
    AddressSanitizer runtime preloaded, to run the CPU tests under it)."""
    bdir = BUILD if host_asan is None else BUILD + "_host_asan"
    os.makedirs(bdir, exist_ok=True)
    hipcc = _hipcc()
    extra = [] if host_asan is None else HOST_ASAN_FLAGS
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
                     "-o", obj])

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
    out = LIB if host_asan is None else os.path.abspath(host_asan)
    tmp = out + ".tmp"
    if host_asan is None:
        link = ["g++", "-shared", "-o", tmp, *objs, f"-L{tl}", "-l:libamdhip64.so",
                f"-Wl,-rpath,{tl}", "-Wl,--no-undefined"]
    else:  # the sanitizer runtime is clang's, shared, preloaded by the caller
        link = [hipcc, "-shared", "-Xarch_host", "-fsanitize=address", "-shared-libsan", "-o", tmp, *objs,
                f"-L{tl}", "-l:libamdhip64.so", f"-Wl,-rpath,{tl}"]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    asan = sys.argv[sys.argv.index("--host-asan") + 1] if "--host-asan" in sys.argv else None
    print(build(verbose="--verbose" in sys.argv, host_asan=asan))
