"""Build the gfx950 BoB library (libflashbob.so) in-tree with hipcc.

Usage: python -m exact_second_order_amd.build   (or call build()).
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflashbob.so")
# a plain C program that drives the C ABI without torch (run by the tests)
C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi_check.c")
C_CHECK = os.path.join(PKG, "_build", "c_abi_check")
# a standalone program measuring the sustained MFMA rate under the power limit
# (run by bench.py after its timed region)
CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")
CEILING = os.path.join(PKG, "_build", "mfma_ceiling")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# (source, extra flags): bob_query.hip is built twice. The pass-1 object keeps
# MFMA results in VGPRs (its register budget allows it, and its elementwise
# work then reads them without AGPR copies); the pass-2 object lets the
# compiler place accumulators in AGPRs.
OBJECTS = [
    ("flashbob_api.hip", []),
    ("bob_query.hip", ["-DFLASHBOB_QUERY_PASS1", "-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("bob_query.hip", ["-DFLASHBOB_QUERY_PASS2"]),
    ("bob_key.hip", []),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    # no packed fp32 VALU ops (v_pk_*_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # only the C ABI (marked FLASHBOB_API in include/flashbob.h) is exported
    "-fvisibility=hidden",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        ln for ln in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in ln  # the host pass does not know the device feature
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False):
    """Compile every object and link libflashbob.so (always rebuilds)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, f"{i}_{os.path.splitext(src)[0]}.o") for i, (src, _) in enumerate(OBJECTS)]
    cmds = [[hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            for (src, extra), obj in zip(OBJECTS, objs)]
    # the objects compile independently: one hipcc per object, a few at a time
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 4))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
          "-Wl,--version-script=" + os.path.join(CSRC, "exports.map"), "-o", tmp], verbose)
    os.replace(tmp, LIB)
    _run([hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")], CEILING_SRC,
          "-o", CEILING], verbose)
    if os.path.exists(C_CHECK_SRC):
        _run(["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
              "-I", INCLUDE, C_CHECK_SRC, "-L", PKG, "-lflashbob", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
              "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", C_CHECK], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
