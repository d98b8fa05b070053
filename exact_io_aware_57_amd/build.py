"""Build the HIP library libfa_mi355x.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_57_amd.build [-v]
    python -m exact_io_aware_57_amd.build --candidate ID   (a kernel-candidate copy, see build_candidate)

Every source in csrc/ is compiled to an object under _build/ (in parallel), then
the objects are linked into exact_io_aware_57_amd/libfa_mi355x.so.  Packed fp32
VALU instructions are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Keep MFMA results in ordinary VGPRs: the softmax reads every score, and
# AGPR-resident accumulators would cost a v_accvgpr move per element.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# Sources whose kernels run one wave per SIMD and need the accumulation
# registers as well (head size 256: 64 registers of Q and 128 of O^T per lane).
AGPR_FORM_SOURCES = {"fa_fwd_bf16_d256.hip"}


def device_flags(src):
    """hipcc flags for one source file."""
    return DEVICE_FLAGS + ([] if os.path.basename(src) in AGPR_FORM_SOURCES else VGPR_FORM)


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build the HIP library")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


CANDIDATE_DIR = os.path.join(BUILD_DIR, "candidates")


def candidate_path(cid):
    return os.path.join(CANDIDATE_DIR, f"libfa_candidate{int(cid)}.so")


def build_candidate(cid, verbose=False):
    """A copy of the library whose bf16 forward pass always runs kernel form
    ``cid`` (fa_fwd_bf16.hip built with -DFA_FORCE_FWD=cid; the other objects are
    the library's own), for measuring each kernel candidate on one workload.
    Requires build_library() first; returns the path."""
    os.makedirs(CANDIDATE_DIR, exist_ok=True)
    cc = hipcc()
    src = os.path.join(CSRC, "fa_fwd_bf16.hip")
    obj = os.path.join(CANDIDATE_DIR, f"fa_fwd_bf16_c{int(cid)}.o")
    _run([cc, *device_flags(src), f"-DFA_FORCE_FWD={int(cid)}", "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj], verbose)
    others = [os.path.join(BUILD_DIR, os.path.basename(x)[:-4] + ".o") for x in sources()
              if os.path.basename(x) != "fa_fwd_bf16.hip"]
    out = candidate_path(cid)
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *others, "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    os.remove(obj)
    return out


def build_library(verbose=False, jobs=None):
    """Compile every csrc/*.hip and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[cc, *device_flags(s), "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--candidate" in args:
        print(build_candidate(int(args[args.index("--candidate") + 1]), verbose="-v" in args))
    else:
        print(build_library(verbose="-v" in args))
