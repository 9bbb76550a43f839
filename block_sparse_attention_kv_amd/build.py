"""Build libmsa.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m block_sparse_attention_kv_amd.build

Each csrc/*.hip file is compiled to an object in parallel, then linked into
block_sparse_attention_kv_amd/libmsa.so. Packed fp32 instructions are
disabled for the device code (-packed-fp32-ops).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-file flags. The indexer keeps matrix-core results in VGPRs (its
# accumulators are consumed at once by vector code; the AGPR round trip costs
# one extra instruction per element); so does the single-launch layer, which
# holds the indexer's code.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "layer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    warnings = "\n".join(l for l in r.stderr.splitlines()
                         if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    return obj, warnings


def build(extra=(), verbose=False):
    """Compile every csrc/*.hip and link libmsa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    for _, w in results:
        if verbose and w.strip():
            print(w, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
