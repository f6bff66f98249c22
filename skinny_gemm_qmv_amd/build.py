"""Build libqmv.so (the HIP library) in-tree for gfx950.

    python skinny_gemm_qmv_amd/build.py          # or __graft_entry__.build()

(Run it as a script: importing the package first would need the library.)

Flags:
  --offload-arch=gfx950        MI355X only
  -ffp-contract=off            HIP's default contracts a*b+c; the fixed order
                               writes every fused multiply-add explicitly
  -target-feature -packed-fp32-ops
                               no v_pk_{add,mul,fma}_f32 in generated code
  (no -ffast-math, no denormal flushing: the gfx950 default float mode keeps
   fp32 and fp16 denormals)
Set QMV_SAVE_TEMPS=1 to keep the generated gfx950 assembly under _build/.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmv.so")
MEASURE_LIB = os.path.join(PKG, "libqmv_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qmv_api.hip", "qmv_fo.hip", "qmv_mfma.hip"]
# the benchmark's reference kernels (streaming read, empty kernel): a library
# of their own, so that the product library holds only the method
MEASURE_SOURCES = ["qmv_measure.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
]


def _compile(src, build_dir=BUILD, defines=()):
    os.makedirs(build_dir, exist_ok=True)
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *["-D" + d for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if os.environ.get("QMV_SAVE_TEMPS"):
        cmd += ["-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=build_dir)
    # the host pass does not know the gfx950 feature flag: drop that one warning
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=False, out=LIB, defines=(), build_dir=BUILD, sources=SOURCES):
    """Compile every HIP source for gfx950 and link libqmv.so; returns its path.
    `defines` (NAME=VALUE strings) and `out` build a variant elsewhere, e.g. to
    compare launch shapes (QMV_BLOCK, QMV_MAX_GRID, QMV_RING, QMV_XREG_BUDGET)."""
    with cf.ThreadPoolExecutor(max_workers=len(sources)) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir, defines), sources))
    for _, err in results:
        if err.strip() and verbose:
            sys.stderr.write(err + "\n")
    objs = [o for o, _ in results]
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(tmp, out)
    return out


def build_measure(verbose=False):
    """Compile the benchmark's reference kernels into libqmv_measure.so."""
    return build(verbose=verbose, out=MEASURE_LIB, sources=MEASURE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_measure(verbose=True))
