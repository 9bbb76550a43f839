"""CPU tests of the C-ABI boundary: libmsa.so loads, exports every entry point
include/msa.h declares, and rejects bad arguments with the documented status
before anything is launched (no GPU is touched: every call below fails host
validation)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_kv_amd as msa
from block_sparse_attention_kv_amd import _lib
from workloads import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    L = msa.load()
    names = _header_functions()
    assert "msa_decode_layer" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def _params(**over):
    d = dict(make_config(1).params)
    d.update(over)
    return msa.Params.from_dict(d)


def _status(fn, *args):
    st = fn(*args)
    return st, msa.load().msa_last_error().decode()


def _null_cache():
    return msa.Cache()


def test_workspace_size():
    p = _params()
    n = msa.msa_workspace_size(p)
    assert n >= 4 * 1 * 1 * 32 and n % 256 == 0
    assert msa.msa_workspace_size(_params(head_dim=64)) == 0
    # fp32 pooled scores of the two-kernel layer plus the single launch's
    # tagged 64-bit words, each in a 256-byte aligned region of its own
    for B, Tq, maxb in ((32, 4, 1024), (3, 2, 17), (1, 1, 1)):
        q = _params(num_seqs=B, q_len=Tq, max_blocks_per_seq=maxb, num_pages=B * maxb)
        entries = B * Tq * maxb
        align = lambda x: (x + 255) // 256 * 256
        assert msa.msa_workspace_size(q) >= align(4 * entries) + align(8 * entries)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(idx_dim=128), _lib.MSA_ERR_UNSUPPORTED),
    (dict(block_size=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(top_k=17), _lib.MSA_ERR_UNSUPPORTED),
    (dict(top_k=0), _lib.MSA_ERR_INVALID_ARG),
    (dict(num_q_heads=9), _lib.MSA_ERR_INVALID_ARG),
    (dict(num_q_heads=32, num_kv_heads=1), _lib.MSA_ERR_UNSUPPORTED),
    (dict(q_len=5, idx_heads=8), _lib.MSA_ERR_UNSUPPORTED),
    (dict(q_len=9, idx_heads=2), _lib.MSA_ERR_UNSUPPORTED),
    (dict(q_len=0), _lib.MSA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=8193), _lib.MSA_ERR_UNSUPPORTED),
    (dict(keep_last=2), _lib.MSA_ERR_INVALID_ARG),
    (dict(kv_dtype=7), _lib.MSA_ERR_UNSUPPORTED),
    (dict(num_pages=0), _lib.MSA_ERR_INVALID_ARG),
])
def test_bad_params_rejected(over, status):
    L = msa.load()
    p = _params(**over)
    c = _null_cache()
    st, msg = _status(L.msa_decode_layer, ctypes.byref(p), ctypes.byref(c), None, None, None, None, None,
                      None, None, 0, None)
    assert st == status, msg
    assert msg
    st, msg = _status(L.msa_sparse_attn_decode, ctypes.byref(p), ctypes.byref(c), None, None, None, None,
                      None, 0, None)
    assert st == status, msg


def test_null_pointers_rejected():
    L = msa.load()
    p = _params()
    c = _null_cache()
    assert L.msa_decode_layer(None, ctypes.byref(c), None, None, None, None, None, None, None, 0,
                              None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_decode_layer(ctypes.byref(p), None, None, None, None, None, None, None, None, 0,
                              None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_decode_layer(ctypes.byref(p), ctypes.byref(c), None, None, None, None, None, None, None, 0,
                              None) == _lib.MSA_ERR_INVALID_ARG
    assert "NULL" in L.msa_last_error().decode()
    assert L.msa_indexer_scores(ctypes.byref(p), ctypes.byref(c), None, None, None, None) == \
        _lib.MSA_ERR_INVALID_ARG
    assert L.msa_pool_select_blocks(ctypes.byref(p), None, None, None, None, None, None) == \
        _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_dequant_nvfp4(None, None, 4, None, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_dequant_fp8(None, -1, None, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_read_bandwidth(None, 64, None, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_read_bandwidth(None, 17, None, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_read_bandwidth(None, -16, None, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_read_bandwidth(ctypes.c_void_p(8), 64, ctypes.c_void_p(16), None) == _lib.MSA_ERR_INVALID_ARG
    assert "aligned" in L.msa_last_error().decode()
    assert L.msa_debug_read_bandwidth(None, 0, None, None) == _lib.MSA_OK  # nothing to read, no launch


def test_dtype_scale_consistency_rejected():
    L = msa.load()
    fake = ctypes.c_void_p(0x1000)
    # bf16 KV must not carry scales; NVFP4 must
    p = _params(kv_dtype=0, idx_dtype=0)
    c = msa.Cache(fake, fake, fake, None, 1.0, 1.0, fake, None, fake, fake)
    assert L.msa_sparse_attn_decode(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None, None, 0,
                                    None) == _lib.MSA_ERR_INVALID_ARG
    p = _params(kv_dtype=1, idx_dtype=1)
    c = msa.Cache(fake, None, fake, fake, 1.0, 1.0, fake, None, fake, fake)
    assert L.msa_sparse_attn_decode(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None, None, 0,
                                    None) == _lib.MSA_ERR_INVALID_ARG
    c = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, None, fake, fake)
    assert L.msa_indexer_scores(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None) == \
        _lib.MSA_ERR_INVALID_ARG       # FP8 keys without idx_k_scale


def test_nvfp4_index_keys_and_insert_args_rejected():
    L = msa.load()
    fake = ctypes.c_void_p(0x1000)
    p = _params(kv_dtype=1, idx_dtype=2)
    c = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, None, fake, fake, 1.0)
    assert L.msa_indexer_scores(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None) == \
        _lib.MSA_ERR_INVALID_ARG       # NVFP4 keys without their scales
    c = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, fake, fake, fake, float("nan"))
    assert L.msa_indexer_scores(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None) == \
        _lib.MSA_ERR_INVALID_ARG       # non-finite tensor scale
    p = _params(kv_dtype=1, idx_dtype=3)
    assert L.msa_indexer_scores(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None) == \
        _lib.MSA_ERR_UNSUPPORTED
    p = _params(kv_dtype=1, idx_dtype=2)
    c = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, fake, fake, fake, 0.0)
    assert L.msa_kv_insert(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, None) == \
        _lib.MSA_ERR_INVALID_ARG       # a zero tensor scale cannot be divided by
    c = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, fake, fake, fake, 1.0)
    assert L.msa_kv_insert(ctypes.byref(p), ctypes.byref(c), None, fake, fake, None) == \
        _lib.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert(None, ctypes.byref(c), fake, fake, fake, None) == _lib.MSA_ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    L = msa.load()
    fake = ctypes.c_void_p(0x1000)
    p = _params()
    c = msa.Cache(fake, None, fake, None, 1.0, 1.0, fake, None, fake, fake)
    need = msa.msa_workspace_size(p)
    assert L.msa_decode_layer(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, fake, None, None, None, 0,
                              None) == _lib.MSA_ERR_WORKSPACE
    assert L.msa_decode_layer(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, fake, None, None, fake,
                              need - 1, None) == _lib.MSA_ERR_WORKSPACE
    assert L.msa_decode_layer(ctypes.byref(p), ctypes.byref(c), fake, fake, fake, fake, None, None,
                              ctypes.c_void_p(0x1010), need, None) == _lib.MSA_ERR_WORKSPACE  # misaligned


def test_status_strings():
    L = msa.load()
    assert L.msa_status_string(0) == b"MSA_OK"
    assert L.msa_status_string(3) == b"MSA_ERR_WORKSPACE"
    assert L.msa_version().startswith(b"libmsa")


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_single_launch_layer_args_rejected():
    # msa_decode_layer_single: unsupported problems, null pointers and a short
    # workspace are reported before anything is launched
    L = msa.load()
    fake = ctypes.c_void_p(0x1000)
    nv = msa.Cache(fake, fake, fake, fake, 1.0, 1.0, fake, fake, fake, fake, 1.0)
    bf = msa.Cache(fake, None, fake, None, 1.0, 1.0, fake, None, fake, fake)
    for over, cache in ((dict(kv_dtype=0, idx_dtype=0), bf),        # bf16 K/V
                        (dict(kv_dtype=1, idx_dtype=0), nv),        # bf16 indexer keys
                        (dict(kv_dtype=1, idx_dtype=1, q_len=5, idx_heads=4), nv)):  # q_len > 4
        p = _params(**over)
        st, msg = _status(L.msa_decode_layer_single, ctypes.byref(p), ctypes.byref(cache), fake, fake, fake, fake,
                          None, None, fake, 1 << 30, None)
        assert st == _lib.MSA_ERR_UNSUPPORTED, (over, st, msg)
    p = _params(kv_dtype=1, idx_dtype=1)
    need = msa.msa_workspace_size(p)
    assert L.msa_decode_layer_single(ctypes.byref(p), ctypes.byref(nv), None, fake, fake, fake, None, None, fake,
                                     need, None) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_decode_layer_single(ctypes.byref(p), ctypes.byref(nv), fake, fake, fake, fake, None, None, fake,
                                     need - 1, None) == _lib.MSA_ERR_WORKSPACE
    assert L.msa_decode_layer_single(ctypes.byref(p), ctypes.byref(nv), fake, fake, fake, fake, None, None,
                                     ctypes.c_void_p(0x1010), need, None) == _lib.MSA_ERR_WORKSPACE
    assert L.msa_decode_layer_single(None, ctypes.byref(nv), fake, fake, fake, fake, None, None, fake, need,
                                     None) == _lib.MSA_ERR_INVALID_ARG


def test_debug_spin_limit_argument():
    L = msa.load()
    assert L.msa_debug_layer_spin_limit(-5) == _lib.MSA_ERR_INVALID_ARG
    assert L.msa_debug_layer_spin_limit(0) == _lib.MSA_OK


def test_static_layer_rejects_oversized_scratch():
    # the allocation-free entry refuses, before anything is enqueued, a
    # problem whose tagged scores alone exceed its static scratch
    fake = ctypes.c_void_p(256)
    c = msa.Cache(k_data=fake, k_scale=fake, v_data=fake, v_scale=fake, k_tensor_scale=1.0, v_tensor_scale=1.0,
                  idx_k=fake, idx_k_scale=fake, block_table=fake, ctx_lens=fake, idx_k_tensor_scale=1.0)
    limit = _lib.load().msa_decode_layer_single_static
    p = _params(num_seqs=1024, q_len=4, num_q_heads=64, num_kv_heads=4, idx_heads=8, max_blocks_per_seq=1024,
                num_pages=4096, kv_dtype=1, idx_dtype=1)
    st, err = _status(limit, ctypes.byref(p), ctypes.byref(c), fake, fake, fake, fake, None, None, None)
    assert st == msa.MSA_ERR_UNSUPPORTED and "static scratch" in err, err
    p = _params(kv_dtype=0)                     # bf16 K/V: not a single-launch problem
    st, err = _status(limit, ctypes.byref(p), ctypes.byref(c), fake, fake, fake, fake, None, None, None)
    assert st == msa.MSA_ERR_UNSUPPORTED
    st, err = _status(limit, ctypes.byref(_params(kv_dtype=1, idx_dtype=1)), ctypes.byref(c), None, fake, fake, fake,
                      None, None, None)
    assert st == msa.MSA_ERR_INVALID_ARG
