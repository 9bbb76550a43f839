"""GPU parity at the full sizes of the large decode configurations, in the
launch configurations bench.py times: the whole batch runs through
msa_decode_layer (every configuration) or msa_decode_layer_single (the 128K
speculative-verify batch, where bench.py's automatic choice takes the
single-launch path), and the oracle recomputes sampled sequences one by one
(selection tie-aware, outputs to the strict max-abs 2e-3 / mean-abs 2e-4)."""
import numpy as np
import pytest

from tests import gpu_util as G
from workloads import make_config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,seqs,single", [(3, [0, 21], False), (3, [10, 31], True), (4, [0, 3], False)])
def test_config_full_size_sampled(cfg, seqs, single):
    w = make_config(cfg)
    ties, mx, mean = G.layer_parity(w, seqs=seqs, strict=True, single=single)
    print("cfg%d%s sampled %s: tie-band selections %d, out max-abs %.2e mean-abs %.2e" % (
        cfg, " single-launch" if single else "", seqs, ties, mx, mean))


def test_config5_ragged_sampled():
    w = make_config(5)
    order = np.argsort(w.ctx_lens)
    seqs = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    ties, mx, mean = G.layer_parity(w, seqs=seqs, strict=True)
    print("cfg5 sampled %s (lens %s): tie-band selections %d, out max-abs %.2e mean-abs %.2e" % (
        seqs, [int(w.ctx_lens[s]) for s in seqs], ties, mx, mean))


@pytest.mark.parametrize("cfg,seqs,single", [(3, [5], True), (4, [1], False)])
def test_config_full_size_nvfp4_index_keys_sampled(cfg, seqs, single):
    # the same workloads with NVFP4 indexer keys (bench.py --idx-dtype nvfp4)
    from workloads import IDX_NVFP4
    w = make_config(cfg, idx_dtype=IDX_NVFP4)
    ties, mx, mean = G.layer_parity(w, seqs=seqs, strict=True, single=single)
    print("cfg%d nvfp4 keys sampled %s: tie-band selections %d, out max-abs %.2e mean-abs %.2e" % (
        cfg, seqs, ties, mx, mean))
