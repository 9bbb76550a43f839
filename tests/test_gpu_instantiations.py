"""GPU parity against the oracle for every compiled (indexer key format,
indexer heads, query tokens) instantiation of both layer paths, on a small
ragged batch each: the two-kernel layer for FP8, NVFP4 and bf16 indexer keys
with 4 indexer heads (1-8 query tokens) and 8 indexer heads (1-4 query
tokens), on NVFP4 and bf16 K/V, and the single-launch layer for FP8 and
NVFP4 keys (1-4 query tokens), whose selection must also equal the
two-kernel layer's. Tolerances: tests/gpu_util.py."""
import itertools

import numpy as np
import pytest

from tests import gpu_util as G
from workloads import make_workload, KV_NVFP4, KV_BF16, IDX_BF16, IDX_FP8, IDX_NVFP4

pytestmark = pytest.mark.gpu

CTX = [700, 2100, 130]

TWO = [(kv, idx, hi, q)
       for kv, idx in ((KV_NVFP4, IDX_FP8), (KV_NVFP4, IDX_NVFP4), (KV_NVFP4, IDX_BF16), (KV_BF16, IDX_BF16))
       for hi, qmax in ((4, 8), (8, 4)) for q in range(1, qmax + 1)]


@pytest.mark.parametrize("kv,idx,hi,q", TWO)
def test_two_kernel_instantiation(kv, idx, hi, q):
    w = make_workload("inst2_%d_%d_%d_%d" % (kv, idx, hi, q), 80 + 10 * idx + q, CTX, q, 16, 2, hi, kv, idx,
                      table="permute", n_planted=2)
    G.layer_parity(w)


SINGLE = list(itertools.product((IDX_FP8, IDX_NVFP4), (4, 8), (1, 2, 3, 4)))


@pytest.mark.parametrize("idx,hi,q", SINGLE)
def test_single_launch_instantiation(idx, hi, q):
    w = make_workload("inst1_%d_%d_%d" % (idx, hi, q), 120 + 10 * idx + q, CTX, q, 16, 2, hi, KV_NVFP4, idx,
                      table="permute", n_planted=2)
    run = G.Run(w)
    a = run.layer()
    b = run.layer(single=True)
    assert np.array_equal(a["sel"], b["sel"])
    G.layer_parity(w, run=run, single=True)
