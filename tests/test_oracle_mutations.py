"""Each pin must catch a plausible mistake: plant one in the oracle (on the
CPU, through monkeypatch) and check that the pin then fails."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from tests import oracle_pins as pins
from workloads import make_workload, KV_NVFP4, IDX_FP8


def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_swapped_nibbles_caught(monkeypatch):
    def bad(byte_rows):
        b = np.asarray(byte_rows, dtype=np.uint8)
        out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
        out[..., 0::2] = b >> 4
        out[..., 1::2] = b & 0x0F
        return out
    monkeypatch.setattr(O, "nibbles", bad)
    _fails(pins.check_layout_golden, O)


def test_e4m3_wrong_bias_caught(monkeypatch):
    good = O.e4m3_to_f64
    monkeypatch.setattr(O, "e4m3_to_f64", lambda c: good(c) * 0.5)
    _fails(pins.check_e4m3, O)


def test_e4m3_no_subnormals_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        mag = (1.0 + m / 8.0) * np.exp2(e - 7.0)
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(c >> 7, -mag, mag)
    monkeypatch.setattr(O, "e4m3_to_f64", bad)
    _fails(pins.check_e4m3, O)


def test_e2m1_wrong_mantissa_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes, dtype=np.int64)
        e, m = (c >> 1) & 3, c & 1
        mag = np.where(e == 0, m * 0.5, (1.0 + m / 4.0) * np.exp2(e - 1.0))
        return np.where((c >> 3) & 1, -mag, mag)
    monkeypatch.setattr(O, "e2m1_to_f64", bad)
    _fails(pins.check_e2m1, O)


def test_v_not_transposed_caught(monkeypatch):
    def bad(data, scale):
        vals = O.e2m1_to_f64(O.nibbles(data))
        return vals * np.repeat(O.e4m3_to_f64(scale), 16, axis=0)
    monkeypatch.setattr(O, "nvfp4_v_page", bad)
    _fails(pins.check_layout_golden, O)


def test_missing_relu_caught(monkeypatch):
    monkeypatch.setattr(O, "indexer_scores", lambda qi, w, k: (k @ qi.T) @ w)
    _fails(pins.check_indexer_relu, O)


def test_unweighted_heads_caught(monkeypatch):
    monkeypatch.setattr(O, "indexer_scores", lambda qi, w, k: np.maximum(k @ qi.T, 0).sum(axis=1))
    _fails(pins.check_indexer_bruteforce, O)


def test_mean_pool_caught(monkeypatch):
    def bad(scores, present=None):
        n = scores.shape[0]
        return np.array([scores[i * 128:(i + 1) * 128].mean() for i in range((n + 127) // 128)])
    monkeypatch.setattr(O, "pool_blocks", bad)
    _fails(pins.check_pool, O)


def test_tie_to_higher_index_caught(monkeypatch):
    def bad(P, top_k, keep_last=True):
        n = P.shape[0]
        if n <= top_k:
            return np.arange(n)
        Pk = P.copy()
        if keep_last:
            Pk[-1] = np.inf
        order = np.lexsort((-np.arange(n), -Pk))
        return np.sort(order[:top_k])
    monkeypatch.setattr(O, "select_blocks", bad)
    _fails(pins.check_select_rules, O)


def test_no_keep_last_caught(monkeypatch):
    good = O.select_blocks
    monkeypatch.setattr(O, "select_blocks", lambda P, k, keep_last=True: good(P, k, False))
    _fails(pins.check_select_bruteforce, O)


def test_missing_softmax_scale_caught(monkeypatch):
    good = O.attend
    monkeypatch.setattr(O, "attend", lambda q, K, V, scale: good(q, K, V, 1.0))
    _fails(pins.check_attend_sdpa, O)


def test_position_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(O, "query_position", lambda L, q_len, t, mb: min(int(L), mb * 128) - q_len + t - 1)
    w = make_workload("causal", 23, [1500, 130], 4, 16, 2, 4, KV_NVFP4, IDX_FP8, table="permute")
    _fails(pins.check_causal_positions, O, w)


def test_boundary_off_by_one_caught(monkeypatch):
    def bad(P, top_k, keep_last=True):
        n = P.shape[0]
        if n <= top_k + 1:
            return None, None
        Pk = P.astype(np.float64).copy()
        if keep_last:
            Pk[n - 1] = np.inf
        order = np.lexsort((np.arange(n), -Pk))
        return float(Pk[order[top_k]]), float(Pk[order[top_k + 1]])
    monkeypatch.setattr(O, "boundary_values", bad)
    _fails(pins.check_boundary_bruteforce, O)


def test_boundary_ignoring_keep_last_caught(monkeypatch):
    good = O.boundary_values
    monkeypatch.setattr(O, "boundary_values", lambda P, k, keep_last=True: good(P, k, False))
    _fails(pins.check_boundary_bruteforce, O)
