"""CPU pins of the float64 oracle (no GPU). See tests/oracle_pins.py for what
each check is pinned to."""
import math

import numpy as np
import pytest

from oracle import msa_oracle as O
from tests import oracle_pins as pins
from workloads import make_workload, small_cases, make_config, KV_BF16, KV_NVFP4, IDX_BF16, IDX_FP8


def test_e4m3_decoder_exhaustive():
    pins.check_e4m3(O)


def test_e2m1_decoder_table():
    pins.check_e2m1(O)


def test_bf16_decoder():
    pins.check_bf16(O)


def test_layout_golden():
    pins.check_layout_golden(O)


def test_nvfp4_storage_ratio():
    # 64 bytes of 4-bit codes + 8 one-byte scales per 128-element vector is
    # 9/16 of FP8's 128 bytes -- the ratio of the NVFP4 and FP8 bytes/token the
    # ainewsbites page quotes (section "A model built for efficient inference").
    nvfp4 = 128 // 2 + 128 // 16
    assert nvfp4 == 72
    assert nvfp4 * 61440 == 34560 * 128
    assert 1 - 34560 / 61440 == pytest.approx(0.4375)


def test_indexer_bruteforce():
    pins.check_indexer_bruteforce(O)


def test_indexer_relu():
    pins.check_indexer_relu(O)


def test_pool_bruteforce():
    pins.check_pool(O)


def test_select_bruteforce():
    pins.check_select_bruteforce(O)


def test_select_rules():
    pins.check_select_rules(O)


def test_attend_vs_sdpa():
    pins.check_attend_sdpa(O)


def test_dense_equivalence_short_contexts():
    # every context <= 16 blocks: MSA == dense attention (bf16 and NVFP4 caches)
    w = make_workload("dense_nvfp4", 21, [1, 127, 128, 129, 2047, 2048], 1, 16, 2, 4,
                      KV_NVFP4, IDX_FP8, table="permute", outlier_frac=0.02)
    pins.check_dense_equivalence(O, w)
    w = make_workload("dense_bf16", 22, [200, 2048], 2, 8, 1, 3, KV_BF16, IDX_BF16, table="identity")
    pins.check_dense_equivalence(O, w)


@pytest.mark.parametrize("idx", range(4))
def test_sparse_equals_masked_sdpa(idx):
    w = small_cases()[idx]
    pins.check_sparse_masked_sdpa(O, w)


def test_causal_window():
    w = make_workload("causal", 23, [1500, 2500, 130], 4, 16, 2, 4, KV_NVFP4, IDX_FP8,
                      table="permute")
    pins.check_causal_positions(O, w)


def test_edge_contexts_selection_counts():
    lens = [1, 127, 128, 129, 2047, 2048, 2049, 2176]
    w = make_workload("edges", 24, lens, 1, 8, 1, 2, KV_NVFP4, IDX_FP8, table="permute")
    r = O.decode_layer(w)
    for b, L in enumerate(lens):
        nblk = (L + 127) // 128
        assert r["nsel"][b, 0] == min(16, nblk)
        assert r["sel"][b, 0, r["nsel"][b, 0] - 1] == nblk - 1     # last block kept
        assert np.all(r["sel"][b, 0, r["nsel"][b, 0]:] == -1)


def test_short_context_no_keys():
    # ctx_lens < q_len: the earliest tokens have p_t < 0 and attend to nothing
    w = make_workload("neg", 25, [2, 300], 4, 8, 1, 2, KV_NVFP4, IDX_FP8, table="permute")
    r = O.decode_layer(w)
    assert list(r["nsel"][0]) == [0, 0, 1, 1]
    assert np.all(r["out"][0, :2] == 0) and np.all(np.isneginf(r["lse"][0, :2]))


def test_absent_page_is_skipped():
    w = make_workload("absent", 26, [3000], 1, 8, 1, 2, KV_NVFP4, IDX_FP8, table="permute")
    w.block_table = w.block_table.copy()
    w.block_table[0, 5] = -1
    r = O.decode_layer(w)
    assert r["pooled"][0, 0, 5] == -np.inf
    assert 5 not in r["sel"][0, 0]


def test_config1_invariants():
    w = make_config(1)
    r = O.decode_layer(w)
    S = list(r["sel"][0, 0])
    assert len(S) == 16 and 31 in S
    for blk in w.planted[0]:
        assert blk in S
    assert np.max(np.abs(r["out"])) < 0.5   # bf16 half-ulp stays below 2e-3 there


def test_boundary_values_bruteforce():
    pins.check_boundary_bruteforce(O)
