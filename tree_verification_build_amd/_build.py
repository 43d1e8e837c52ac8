"""Compile libddtree.so (HIP kernels + C-ABI) for gfx950 with hipcc.

Every call recompiles: each csrc/*.hip becomes an object file under _build/
(in parallel), then they are linked into tree_verification_build_amd/libddtree.so.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libddtree.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps hipcc from emitting packed fp32 arithmetic.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-source extras.  attention.hip: keep MFMA accumulators in ordinary VGPRs;
# with the AGPR forms the compiler copies the attention accumulators between the
# two register files on every key tile.
FILE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libddtree needs the ROCm toolchain")


# Host-only sanitizer build (argument checks, split planning, workspace sizing):
# AddressSanitizer and UndefinedBehaviorSanitizer on the host pass of every
# source, each flag behind -Xarch_host so that the device code is built as
# usual.  The library goes to _build/sanitize/ and is loaded in place of the
# product one through DDTREE_LIBRARY, with the sanitizer runtime preloaded into
# the Python process.
SANITIZE_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                  "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_OUT = os.path.join(ROOT, "_build", "sanitize", "libddtree.so")


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of the HIP toolchain's clang."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang AddressSanitizer runtime was not found")
    return path


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build", "sanitize") if sanitize else os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = SANITIZE_FLAGS if sanitize else []
    out = SANITIZE_OUT if sanitize else OUT

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIP_FLAGS, *extra, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src,
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
