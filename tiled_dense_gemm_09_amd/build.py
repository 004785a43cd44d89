"""Build the HIP library libtg.so in-tree for gfx950 (hipcc cross-compiles; no GPU needed).

    python -m tiled_dense_gemm_09_amd.build

Also builds libtg_debugsync.so, the same sources compiled with
-DTG_DEBUG_SYNC: every partial wait of a copy pipeline waits for all
outstanding memory operations and every pipeline barrier waits first, so its
outputs must equal libtg.so's bit for bit (a GPU test compares the two).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtg.so")
DEBUG_SYNC_OUT = os.path.join(HERE, "libtg_debugsync.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# (output library, object directory, extra compile flags)
VARIANTS = [(OUT, BUILD_DIR, []),
            (DEBUG_SYNC_OUT, os.path.join(BUILD_DIR, "debugsync"), ["-DTG_DEBUG_SYNC"])]
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


def _compile(job):
    src, obj_dir, extra = job
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + extra + (["-x", "hip"] if src.endswith(".cpp") else []) + [
        "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s%s:\n%s" % (src, " ".join([""] + extra), err))
    return obj, err


def build(verbose=True):
    jobs = []
    for _, obj_dir, extra in VARIANTS:
        os.makedirs(obj_dir, exist_ok=True)
        jobs += [(src, obj_dir, extra) for src in SOURCES]
    workers = min(len(jobs), max(1, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_compile, jobs))
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    for i, (out, _, _) in enumerate(VARIANTS):
        objs = [o for o, _ in results[i * len(SOURCES):(i + 1) * len(SOURCES)]]
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] +
                              objs)
        os.replace(tmp, out)
        if verbose:
            print("built", out)
    return OUT


if __name__ == "__main__":
    build()
