"""GPU parity of msa_kv_insert (through the C ABI) against oracle.kv_insert:
every byte of every cache buffer is compared, written slots and untouched
ones alike (bit-exact: the codes and scales are integer results of exact
rounding decisions), then the decode of the inserted cache is checked
against the oracle with the tolerances of tests/gpu_util.py."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_attention_kv_amd as msa
from oracle import msa_oracle as O
from tests import gpu_util as G
from workloads import make_workload, make_config, make_new_tokens, KV_BF16, KV_NVFP4, IDX_BF16, IDX_FP8

pytestmark = pytest.mark.gpu

FIELDS = ("k_data", "k_scale", "v_data", "v_scale", "idx_k", "idx_k_scale")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _gpu_insert(w, nk, nv, ni):
    params, cache, qs = msa.to_device(w)
    msa.msa_kv_insert(params, cache, _dev(nk), _dev(nv), _dev(ni))
    torch.cuda.synchronize()
    return params, cache, qs


def _assert_same_cache(cache, ref, label):
    for f in FIELDS:
        want = ref[f]
        got = getattr(cache, f)
        if want is None:
            assert got is None, (label, f)
            continue
        g = got.cpu().numpy().view(np.uint8).reshape(-1)
        wb = np.ascontiguousarray(want).view(np.uint8).reshape(-1)
        bad = np.flatnonzero(g != wb)
        assert bad.size == 0, (label, f, "bytes differ", bad.size, bad[:8])


CASES = {
    # odd first slot (ctx 5), a block boundary inside the new tokens (ctx
    # 129), new tokens before position 0 (ctx 2), extreme groups
    "nvfp4_fp8": dict(ctx=[300, 129, 1000, 5, 2], q_len=4, kv=KV_NVFP4, idx=IDX_FP8),
    # non-unit tensor scales (the quotient by 0.75 is inexact)
    "nvfp4_tensor_scales": dict(ctx=[2049, 640], q_len=3, kv=KV_NVFP4, idx=IDX_FP8, k_ts=0.75, v_ts=1.5),
    # more new tokens than one workgroup's chunk of 64, odd start (77 - 70)
    "nvfp4_70_tokens": dict(ctx=[200, 77], q_len=70, kv=KV_NVFP4, idx=IDX_FP8),
    "bf16": dict(ctx=[300, 129, 3], q_len=4, kv=KV_BF16, idx=IDX_BF16),
    "nvfp4_bf16_idx": dict(ctx=[300, 131], q_len=4, kv=KV_NVFP4, idx=IDX_BF16),
    "bf16_fp8_idx": dict(ctx=[300, 131], q_len=2, kv=KV_BF16, idx=IDX_FP8),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_insert_bitexact(name):
    c = CASES[name]
    w = make_workload("ins_" + name, 51, c["ctx"], c["q_len"], 16, 2, 4, c["kv"], c["idx"],
                      table="permute", k_tensor_scale=c.get("k_ts", 1.0), v_tensor_scale=c.get("v_ts", 1.0))
    nk, nv, ni = make_new_tokens(w, 52, extremes=True)
    ref = O.kv_insert(w, nk, nv, ni)
    _, cache, _ = _gpu_insert(w, nk, nv, ni)
    _assert_same_cache(cache, ref, name)


def test_insert_skips_absent_pages():
    w = make_workload("ins_absent", 53, [300, 260], 4, 16, 2, 4, KV_NVFP4, IDX_FP8, table="permute")
    w.block_table[1, 2] = -1            # the block of sequence 1's new tokens
    w.block_table[0, 2] = w.params["num_pages"] + 5  # out of range
    nk, nv, ni = make_new_tokens(w, 54)
    ref = O.kv_insert(w, nk, nv, ni)
    _, cache, _ = _gpu_insert(w, nk, nv, ni)
    _assert_same_cache(cache, ref, "absent")


def test_insert_then_decode():
    w = make_workload("ins_e2e", 55, [3000, 129, 5000], 4, 32, 4, 8, KV_NVFP4, IDX_FP8, table="pool",
                      pool_factor=1.3)
    nk, nv, ni = make_new_tokens(w, 56)
    ref = O.kv_insert(w, nk, nv, ni)
    run = G.Run(w)
    msa.msa_kv_insert(run.params, run.cache, _dev(nk), _dev(nv), _dev(ni))
    torch.cuda.synchronize()
    _assert_same_cache(run.cache, ref, "e2e")
    ties, mx, mean = G.layer_parity(dataclasses.replace(w, **ref), run=run)
    print("insert+decode: ties %d, out max-abs %.2e mean-abs %.2e" % (ties, mx, mean))


def test_insert_config2_shapes():
    # the 32K-context NVFP4 configuration: 8 sequences x 1 new token, 2 KV
    # heads, permuted pages
    w = make_config(2)
    nk, nv, ni = make_new_tokens(w, 57)
    ref = O.kv_insert(w, nk, nv, ni)
    _, cache, _ = _gpu_insert(w, nk, nv, ni)
    _assert_same_cache(cache, ref, "cfg2")


def test_insert_rejects_bad_args():
    w = make_workload("ins_bad", 58, [300], 2, 16, 2, 4, KV_NVFP4, IDX_FP8, table="permute")
    nk, nv, ni = make_new_tokens(w, 59)
    params, cache, _ = msa.to_device(w)
    with pytest.raises(msa.MSAError):
        msa.msa_kv_insert(params, cache, None, _dev(nv), _dev(ni))
    bad = msa.Params.from_dict(dict(w.params, head_dim=64))
    with pytest.raises(msa.MSAError):
        msa.msa_kv_insert(bad, cache, _dev(nk), _dev(nv), _dev(ni))
