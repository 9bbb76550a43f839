"""GPU parity of the NVFP4 indexer-key path (36 bytes per token) against the
float64 oracle, through the C ABI: indexer scores, pooled scores and the
selection, the fused decode layer, and the KV-insert of NVFP4 keys.
Tolerances as in tests/gpu_util.py (the keys decode exactly to fp16, the
queries are scaled into fp16 exactly, products accumulate in fp32)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_kv_amd as msa
from oracle import msa_oracle as O
from tests import gpu_util as G
from workloads import make_workload, make_new_tokens, KV_NVFP4, KV_BF16, IDX_NVFP4

pytestmark = pytest.mark.gpu


def _cases():
    return [
        make_workload("nv_idx_ragged", 61, [300, 2500, 4100, 129], 2, 16, 2, 3, KV_NVFP4, IDX_NVFP4,
                      table="permute", n_planted=2),
        make_workload("nv_idx_tq4", 62, [3000, 5000], 4, 32, 4, 8, KV_NVFP4, IDX_NVFP4, table="pool",
                      pool_factor=1.3),
        make_workload("nv_idx_bf16kv", 63, [2049, 1], 1, 8, 1, 4, KV_BF16, IDX_NVFP4, table="identity",
                      n_planted=1),
    ]


@pytest.mark.parametrize("idx", range(3))
def test_indexer_nvfp4_keys(idx):
    w = _cases()[idx]
    print("%s: ties %d" % (w.name, G.indexer_parity(w)))


def test_indexer_nvfp4_tensor_scale_and_large_queries():
    # a negative tensor scale flips the ReLU side; queries near bf16's top
    # exercise the power-of-two pre-scale into fp16
    w = make_workload("nv_idx_ts", 64, [2000, 700], 2, 16, 2, 4, KV_NVFP4, IDX_NVFP4, table="permute")
    w.idx_k_tensor_scale = -0.375
    q = (w.idx_q.astype(np.uint32) << 16).view(np.float32)
    q[0] *= np.float32(2.0 ** 100)
    w.idx_q = (q.view(np.uint32) >> 16).astype(np.uint16)
    G.indexer_parity(w)


@pytest.mark.parametrize("idx", range(2))
def test_decode_layer_nvfp4_keys(idx):
    w = _cases()[idx]
    ties, mx, mean = G.layer_parity(w)
    print("%s: ties %d, out max-abs %.2e mean-abs %.2e" % (w.name, ties, mx, mean))


def test_insert_nvfp4_keys_bitexact():
    w = make_workload("nv_idx_ins", 65, [300, 129, 5], 4, 16, 2, 4, KV_NVFP4, IDX_NVFP4, table="permute")
    w.idx_k_tensor_scale = 0.75
    nk, nv, ni = make_new_tokens(w, 66, extremes=True)
    ref = O.kv_insert(w, nk, nv, ni)
    params, cache, _ = msa.to_device(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    msa.msa_kv_insert(params, cache, dev(nk), dev(nv), dev(ni))
    torch.cuda.synchronize()
    for f in ("idx_k", "idx_k_scale", "k_data", "k_scale", "v_data", "v_scale"):
        got = getattr(cache, f).cpu().numpy().view(np.uint8).reshape(-1)
        want = np.ascontiguousarray(ref[f]).view(np.uint8).reshape(-1)
        assert np.array_equal(got, want), f
