"""ctypes loader for the seeded input generator (workloads/csrc/msagen.c).

The generator is plain C with OpenMP; it is compiled with gcc into
``workloads/libmsagen.so`` by :func:`build` (also called lazily on first use
when the library is missing). Floating-point contraction is disabled so the
draws do not depend on the host CPU's instruction set.
"""
import ctypes
import os
import subprocess
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "csrc", "msagen.c")
LIB = os.path.join(_HERE, "libmsagen.so")
_lock = threading.Lock()
_lib = None


def build(force=True):
    """Compile libmsagen.so in-tree with gcc."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build(force=True)
            L = ctypes.CDLL(LIB)
            u64, i64, i32, dbl, p = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_double, ctypes.c_void_p)
            L.msagen_stream_key.restype = u64
            L.msagen_stream_key.argtypes = [u64, u64]
            L.msagen_bf16_rne.restype = ctypes.c_uint16
            L.msagen_bf16_rne.argtypes = [ctypes.c_float]
            L.msagen_e4m3_rne.restype = ctypes.c_uint8
            L.msagen_e4m3_rne.argtypes = [dbl]
            L.msagen_e2m1_rne.restype = ctypes.c_uint8
            L.msagen_e2m1_rne.argtypes = [dbl]
            L.msagen_normal_bf16.restype = None
            L.msagen_normal_bf16.argtypes = [u64, i64, i64, dbl, p]
            L.msagen_uniform_f32.restype = None
            L.msagen_uniform_f32.argtypes = [u64, i64, i64, p]
            L.msagen_normal_f32.restype = None
            L.msagen_normal_f32.argtypes = [u64, i64, i64, dbl, p]
            L.msagen_kv_cache.restype = None
            L.msagen_kv_cache.argtypes = [u64, u64, i32, p, p, i32, i32, p, p, i32, p, p, p, p]
            L.msagen_idx_cache.restype = None
            L.msagen_idx_cache.argtypes = [u64, i32, p, p, i32, dbl, p, p, i32, p, p]
            _lib = L
    return _lib
