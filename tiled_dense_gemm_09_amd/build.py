"""Build the HIP library libtg.so in-tree for gfx950 (hipcc cross-compiles; no GPU needed).

    python -m tiled_dense_gemm_09_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtg.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gemm_tiled.hip", "gemm_async.hip", "gemm_mx.hip", "attention.hip", "gemm_skinny.hip",
           "gemm_generic.hip", "gemm_kpad.hip", "tg_api.cpp"]
ARCH = os.environ.get("TG_ARCH", "gfx950")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from emitting packed FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc():
    h = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return h if os.path.exists(h) else "hipcc"


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + (["-x", "hip"] if src.endswith(".cpp") else []) + [
        "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return obj, err


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [
        o for o, _ in results]
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
