"""ctypes binding of libmsa (include/msa.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libmsa.so. Device buffers are torch tensors on the current HIP
device; the stream defaults to torch's current stream. If the library has
not been built, loading fails with an error -- there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)
KV_BF16, KV_NVFP4 = 0, 1
IDX_BF16, IDX_FP8, IDX_NVFP4 = 0, 1, 2
NUM_STAGES = 2
STAGE_NAMES = ("indexer_pool", "select_sparse_attn")


class MSAError(RuntimeError):
    def __init__(self, status, where, detail):
        super().__init__("%s: status %d (%s): %s" % (where, status, _STATUS.get(status, "?"), detail))
        self.status = status


_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED", 3: "MSA_ERR_WORKSPACE",
           4: "MSA_ERR_HIP"}


class Params(ctypes.Structure):
    """msa_params_t."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "q_len", "num_q_heads", "num_kv_heads", "head_dim", "idx_heads", "idx_dim",
        "block_size", "top_k", "keep_last", "max_blocks_per_seq", "num_pages")] + [
        ("softmax_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32), ("idx_dtype", ctypes.c_int32)]

    @classmethod
    def from_dict(cls, d):
        p = cls()
        for name, ctype in cls._fields_:
            setattr(p, name, float(d[name]) if ctype is ctypes.c_float else int(d[name]))
        return p


class Cache(ctypes.Structure):
    """msa_cache_t."""
    _fields_ = [("k_data", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_data", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("k_tensor_scale", ctypes.c_float),
                ("v_tensor_scale", ctypes.c_float), ("idx_k", ctypes.c_void_p),
                ("idx_k_scale", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("ctx_lens", ctypes.c_void_p), ("idx_k_tensor_scale", ctypes.c_float)]


_lib = None


def load():
    """Load libmsa.so (built by block_sparse_attention_kv_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmsa.so is not built (%s); run `python -m block_sparse_attention_kv_amd.build`"
                           % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, C, vp, i64, st = (ctypes.POINTER(Params), ctypes.POINTER(Cache), ctypes.c_void_p, ctypes.c_int64,
                         ctypes.c_int)
    sz = ctypes.c_size_t
    sig = {
        "msa_workspace_size": (sz, [P]),
        "msa_indexer_scores": (st, [P, C, vp, vp, vp, vp]),
        "msa_pool_select_blocks": (st, [P, vp, vp, vp, vp, vp, vp]),
        "msa_sparse_attn_decode": (st, [P, C, vp, vp, vp, vp, vp, sz, vp]),
        "msa_decode_layer": (st, [P, C, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "msa_decode_layer_traced": (st, [P, C, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]),
        "msa_decode_layer_single": (st, [P, C, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "msa_decode_layer_single_traced": (st, [P, C, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]),
        "msa_decode_layer_single_static": (st, [P, C, vp, vp, vp, vp, vp, vp, vp]),
        "msa_kv_insert": (st, [P, C, vp, vp, vp, vp]),
        "msa_debug_dequant_nvfp4": (st, [vp, vp, i64, vp, vp]),
        "msa_debug_dequant_fp8": (st, [vp, i64, vp, vp]),
        "msa_debug_read_bandwidth": (st, [vp, i64, vp, vp]),
        "msa_debug_layer_spin_limit": (st, [ctypes.c_int32]),
        "msa_debug_layer_splits": (st, [ctypes.c_int32]),
        "msa_decode_layer_gave_up": (st, [P, vp, sz, vp, ctypes.POINTER(ctypes.c_int64)]),
        "msa_status_string": (ctypes.c_char_p, [st]),
        "msa_last_error": (ctypes.c_char_p, []),
        "msa_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTED = ("msa_workspace_size", "msa_indexer_scores", "msa_pool_select_blocks", "msa_sparse_attn_decode",
            "msa_decode_layer", "msa_decode_layer_traced", "msa_decode_layer_single",
            "msa_decode_layer_single_traced", "msa_decode_layer_single_static", "msa_kv_insert", "msa_debug_dequant_nvfp4",
            "msa_debug_dequant_fp8", "msa_debug_read_bandwidth", "msa_debug_layer_spin_limit",
            "msa_debug_layer_splits", "msa_decode_layer_gave_up",
            "msa_status_string", "msa_last_error", "msa_version")


def _check(status, where):
    if status != MSA_OK:
        raise MSAError(status, where, load().msa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class DeviceCache:
    """Device-resident paged cache (layouts of include/msa.h)."""
    k_data: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_data: torch.Tensor
    v_scale: Optional[torch.Tensor]
    idx_k: torch.Tensor
    idx_k_scale: Optional[torch.Tensor]
    block_table: torch.Tensor
    ctx_lens: torch.Tensor
    k_tensor_scale: float = 1.0
    v_tensor_scale: float = 1.0
    idx_k_tensor_scale: float = 1.0

    def c(self):
        return Cache(_v(self.k_data), _v(self.k_scale), _v(self.v_data), _v(self.v_scale),
                     float(self.k_tensor_scale), float(self.v_tensor_scale), _v(self.idx_k),
                     _v(self.idx_k_scale), _v(self.block_table), _v(self.ctx_lens),
                     float(self.idx_k_tensor_scale))


def _v(t):
    return None if t is None else _ptr(t).value


def _dev(a, device):
    if a is None:
        return None
    import numpy as np
    arr = np.ascontiguousarray(a)
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(arr).to(device)


def to_device(host, device="cuda"):
    """Copy a host-side workload (any object with the buffers of msa.h as
    numpy arrays: q, idx_q, idx_w, k_data, ..., block_table, ctx_lens, params)
    to the device. Returns (params, DeviceCache, dict of the query tensors)."""
    cache = DeviceCache(_dev(host.k_data, device), _dev(host.k_scale, device), _dev(host.v_data, device),
                        _dev(host.v_scale, device), _dev(host.idx_k, device), _dev(host.idx_k_scale, device),
                        _dev(host.block_table, device), _dev(host.ctx_lens, device),
                        float(host.k_tensor_scale), float(host.v_tensor_scale),
                        float(getattr(host, "idx_k_tensor_scale", 1.0)))
    qs = dict(q=_dev(host.q, device), idx_q=_dev(host.idx_q, device), idx_w=_dev(host.idx_w, device))
    return Params.from_dict(host.params), cache, qs


# ------------------------------------------------------------------ calls

def msa_workspace_size(params):
    return int(load().msa_workspace_size(ctypes.byref(params)))


def msa_indexer_scores(params, cache, idx_q, idx_w, scores, stream=None):
    c = cache.c()
    _check(load().msa_indexer_scores(ctypes.byref(params), ctypes.byref(c), _ptr(idx_q), _ptr(idx_w),
                                     _ptr(scores), _stream(stream)), "msa_indexer_scores")


def msa_pool_select_blocks(params, ctx_lens, scores, sel, pooled=None, nsel=None, stream=None):
    _check(load().msa_pool_select_blocks(ctypes.byref(params), _ptr(ctx_lens), _ptr(scores), _ptr(pooled),
                                         _ptr(sel), _ptr(nsel), _stream(stream)), "msa_pool_select_blocks")


def msa_sparse_attn_decode(params, cache, q, sel, out, lse=None, workspace=None, stream=None):
    c = cache.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().msa_sparse_attn_decode(ctypes.byref(params), ctypes.byref(c), _ptr(q), _ptr(sel), _ptr(out),
                                         _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)),
           "msa_sparse_attn_decode")


def msa_decode_layer(params, cache, q, idx_q, idx_w, out, workspace, lse=None, sel_out=None, stream=None,
                     stage_events=None):
    """Whole decode step. stage_events: optional list of 2 * NUM_STAGES
    torch.cuda.Event(enable_timing=True): the start and end of kernel i are
    recorded into events 2i and 2i+1 by the kernel's dispatch."""
    c = cache.c()
    ws_bytes = workspace.numel() * workspace.element_size()
    L = load()
    if stage_events is None:
        st = L.msa_decode_layer(ctypes.byref(params), ctypes.byref(c), _ptr(q), _ptr(idx_q), _ptr(idx_w),
                                _ptr(out), _ptr(lse), _ptr(sel_out), _ptr(workspace), ws_bytes, _stream(stream))
    else:
        if len(stage_events) != 2 * NUM_STAGES:
            raise ValueError("need %d events" % (2 * NUM_STAGES))
        s = torch.cuda.current_stream() if stream is None else stream
        for e in stage_events:
            if e.cuda_event == 0:   # torch creates the HIP event lazily on first record
                e.record(s)
        arr = (ctypes.c_void_p * len(stage_events))(*[e.cuda_event for e in stage_events])
        st = L.msa_decode_layer_traced(ctypes.byref(params), ctypes.byref(c), _ptr(q), _ptr(idx_q), _ptr(idx_w),
                                       _ptr(out), _ptr(lse), _ptr(sel_out), _ptr(workspace), ws_bytes,
                                       _stream(stream), arr)
    _check(st, "msa_decode_layer")


def msa_decode_layer_single(params, cache, q, idx_q, idx_w, out, workspace, lse=None, sel_out=None, stream=None):
    """msa_decode_layer in one kernel launch (NVFP4 K/V, FP8 or NVFP4
    indexer keys, q_len <= 4)."""
    c = cache.c()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().msa_decode_layer_single(ctypes.byref(params), ctypes.byref(c), _ptr(q), _ptr(idx_q), _ptr(idx_w),
                                          _ptr(out), _ptr(lse), _ptr(sel_out), _ptr(workspace), ws_bytes,
                                          _stream(stream)), "msa_decode_layer_single")


def msa_decode_layer_single_static(params, cache, q, idx_q, idx_w, out, lse=None, sel_out=None, stream=None):
    """msa_decode_layer_single on the library's static per-GPU scratch: no
    workspace, no allocation (calls that may overlap on one GPU race)."""
    c = cache.c()
    _check(load().msa_decode_layer_single_static(ctypes.byref(params), ctypes.byref(c), _ptr(q), _ptr(idx_q),
                                                 _ptr(idx_w), _ptr(out), _ptr(lse), _ptr(sel_out), _stream(stream)),
           "msa_decode_layer_single_static")


def msa_kv_insert(params, cache, new_k, new_v, new_idx_k, stream=None):
    """Quantise the q_len new tokens (bf16 [B][q_len][num_kv_heads][128] K and
    V, bf16 [B][q_len][64] indexer keys) into the paged cache in place."""
    L = load()
    c = cache.c()
    _check(L.msa_kv_insert(ctypes.byref(params), ctypes.byref(c), _ptr(new_k), _ptr(new_v), _ptr(new_idx_k),
                           _stream(stream)), "msa_kv_insert")


def msa_debug_dequant_nvfp4(codes, scales, out, stream=None):
    n_groups = scales.numel()
    _check(load().msa_debug_dequant_nvfp4(_ptr(codes), _ptr(scales), n_groups, _ptr(out), _stream(stream)),
           "msa_debug_dequant_nvfp4")


def msa_debug_layer_spin_limit(polls):
    """Poll limit of msa_decode_layer_single's waits for later calls (0 =
    default)."""
    _check(load().msa_debug_layer_spin_limit(int(polls)), "msa_debug_layer_spin_limit")


def msa_debug_layer_splits(splits):
    """Workgroups per attention item of later msa_decode_layer_single calls
    (1, 2 or 4; 0 = automatic)."""
    _check(load().msa_debug_layer_splits(int(splits)), "msa_debug_layer_splits")


def msa_decode_layer_gave_up(params, workspace, stream=None):
    """Workgroups of the latest msa_decode_layer_single call on `workspace`
    that gave up a bounded wait (synchronises the stream)."""
    n = ctypes.c_int64(-1)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().msa_decode_layer_gave_up(ctypes.byref(params), _ptr(workspace), ws_bytes, _stream(stream),
                                           ctypes.byref(n)), "msa_decode_layer_gave_up")
    return int(n.value)


def msa_debug_dequant_fp8(codes, out, stream=None):
    _check(load().msa_debug_dequant_fp8(_ptr(codes), codes.numel(), _ptr(out), _stream(stream)),
           "msa_debug_dequant_fp8")


def msa_debug_read_bandwidth(buf, out, stream=None):
    """Stream the device tensor `buf` (a multiple of 16 bytes) through the
    library's read kernel; out: a device tensor of at least 4 bytes."""
    nbytes = buf.numel() * buf.element_size()
    _check(load().msa_debug_read_bandwidth(_ptr(buf), nbytes, _ptr(out), _stream(stream)),
           "msa_debug_read_bandwidth")


def alloc_workspace(params, device="cuda"):
    """Workspace for the decode calls, zero-filled once (the single-launch
    layer's tagged scores then cannot match a call's tag by accident)."""
    n = msa_workspace_size(params)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
