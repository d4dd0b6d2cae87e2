"""Ahead-of-time build of the HIP library (hipcc, gfx950), in-tree."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdsa_indexer_bwd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# A second build whose kernels keep deeper buffer rings (IBWD_DEEP_BUFFERS) with
# the same copy schedule: a verification aid, its results must equal the
# library's bit for bit (no buffer of the library may be reused too early).
DEEPBUF_LIB_PATH = os.path.join(PKG, "libdsa_indexer_bwd_deepbuf.so")
DEEPBUF_SOURCES = ("indexer_bwd_rows_export.hip", "indexer_bwd_dk.hip")

HIP_SOURCES = ["indexer_bwd_kernels.hip", "indexer_bwd_rows.hip", "indexer_bwd_rows_export.hip",
               "indexer_bwd_dk.hip", "indexer_fwd.hip"]
HOST_SOURCES = ["indexer_bwd_api.cpp"]

# Device code: gfx950 only; packed-fp32 VALU forms disabled (they are formed
# by the compiler from ordinary float code otherwise).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The range kernel's MFMA accumulators are consumed by VALU right away: keep
# them in VGPRs (the default AGPR form costs a copy per accumulator register).
PER_FILE_FLAGS = {"indexer_bwd_dk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                  "indexer_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = ([hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS
               + PER_FILE_FLAGS.get(src, []))
        _run(cmd, verbose)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
        _run(cmd, verbose)
        objs.append(obj)
    _link(objs, LIB_PATH, verbose)
    deep = []
    for obj in objs:
        src = os.path.basename(obj)[:-2]
        if src in DEEPBUF_SOURCES:
            obj = os.path.join(objdir, src + ".deepbuf.o")
            _run([hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj, "-DIBWD_DEEP_BUFFERS"]
                 + COMMON + DEVICE_FLAGS + PER_FILE_FLAGS.get(src, []), verbose)
        deep.append(obj)
    _link(deep, DEEPBUF_LIB_PATH, verbose)
    return LIB_PATH


def _link(objs, path, verbose):
    tmp = path + ".tmp%d" % os.getpid()
    _run([hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs, verbose)
    os.replace(tmp, path)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose=True))
