"""Build libsgemm_f32.so (the HIP library behind include/sgemm_f32.h) for gfx950.

Each source under csrc/ is compiled with hipcc into an object under _build/
(in parallel), then linked into fp32_sgemm_f32_amd/libsgemm_f32.so.  Packed
FP32 instructions are disabled in code generation (-packed-fp32-ops): the
kernels use scalar v_fma_f32 and the FP32 matrix cores only.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsgemm_f32.so")

SOURCES = ["sgemm_f32.hip", "plan.cpp", "gemm_mfma.hip", "gemm_mfma_dl.hip", "gemm_generic.hip", "gemm_valu.hip", "pack.hip", "sk_fixup.hip", "skinny.hip", "rowdot.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, extra, verbose: bool, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the gfx target feature; that warning is noise.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if lines and (verbose or r.returncode):
        print("\n".join(lines), file=sys.stderr, flush=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, extra=None, out: str = LIB) -> str:
    """Compile every source and link the library (extra: more hipcc flags,
    out: library path); returns its path."""
    extra = list(extra or [])
    tag = "" if out == LIB else "_" + os.path.splitext(os.path.basename(out))[0]
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose, tag), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
