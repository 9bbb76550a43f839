"""CPU tests of the seeded input generator (workloads/): its quantisers round
to nearest-even as stated, its output is deterministic and independent of the
thread count, and the configurations have the documented shapes."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import torch

from oracle import msa_oracle as O
from workloads import _native, make_workload, make_config, KV_NVFP4, IDX_FP8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _nearest_even_ok(x, code, values, mant_bits):
    finite = [(c, v) for c, v in enumerate(values) if np.isfinite(v)]
    best = min(abs(v - x) for _, v in finite)
    got = values[code]
    if abs(got - x) > best:
        return False
    ties = [c for c, v in finite if abs(v - x) == best and np.signbit(v) == np.signbit(got)]
    if len(ties) > 1:  # exact tie between two codes: the even mantissa wins
        return (code & ((1 << mant_bits) - 1)) % 2 == 0
    return True


def test_e4m3_encoder_rne():
    lib = _native.lib()
    vals = O.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.normal(size=300) * 10, rng.uniform(-0.02, 0.02, size=200),
                         vals[np.isfinite(vals)][:120] * 1.0001,
                         (vals[1:0x7E] + vals[2:0x7F]) / 2])      # exact midpoints
    for x in xs:
        if not np.isfinite(x) or abs(x) >= 448:
            continue
        c = lib.msagen_e4m3_rne(float(x))
        assert _nearest_even_ok(float(x), c, vals, 3), (x, c, vals[c])
    assert vals[lib.msagen_e4m3_rne(1e9)] == 448.0


def test_e2m1_encoder_rne():
    lib = _native.lib()
    vals = O.e2m1_to_f64(np.arange(16))
    for x in np.concatenate([np.linspace(-7, 7, 561), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]]):
        c = lib.msagen_e2m1_rne(float(x))
        if abs(x) > 6:
            assert abs(vals[c]) == 6.0
            continue
        assert _nearest_even_ok(float(x), c, vals, 1), (x, c, vals[c])


def test_bf16_encoder_matches_torch():
    lib = _native.lib()
    xs = np.random.default_rng(1).normal(size=2000).astype(np.float32) * 100
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([lib.msagen_bf16_rne(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _digest(w):
    h = hashlib.sha256()
    for a in (w.q, w.idx_q, w.idx_w, w.k_data, w.k_scale, w.v_data, w.v_scale, w.idx_k,
              w.idx_k_scale, w.block_table, w.ctx_lens):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic_and_thread_independent():
    a = make_workload("d", 7, [700, 3000], 2, 16, 2, 4, KV_NVFP4, IDX_FP8, n_planted=2)
    b = make_workload("d", 7, [700, 3000], 2, 16, 2, 4, KV_NVFP4, IDX_FP8, n_planted=2)
    c = make_workload("d", 8, [700, 3000], 2, 16, 2, 4, KV_NVFP4, IDX_FP8, n_planted=2)
    assert _digest(a) == _digest(b) != _digest(c)
    code = ("import sys; sys.path.insert(0, %r); from tests.test_workloads import _digest;"
            "from workloads import make_workload, KV_NVFP4, IDX_FP8;"
            "print(_digest(make_workload('d', 7, [700, 3000], 2, 16, 2, 4, KV_NVFP4, IDX_FP8, n_planted=2)))" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == _digest(a)


def test_nvfp4_scale_is_amax_over_6():
    w = make_workload("s", 9, [256], 1, 8, 1, 2, KV_NVFP4, IDX_FP8, table="identity")
    # decoded values never exceed 6 * scale and the group amax maps near code 6
    K = O.nvfp4_k_page(w.k_data[0, 0], w.k_scale[0, 0])
    s = np.repeat(O.e4m3_to_f64(w.k_scale[0, 0]), 16, axis=1)
    assert np.all(np.abs(K) <= 6 * s + 1e-12)
    assert np.all((np.abs(K) / np.where(s > 0, s, 1)).reshape(128, 8, 16).max(axis=2) >= 4.0)


def test_config_shapes():
    w = make_config(1)
    assert w.params["num_seqs"] == 1 and w.k_data.dtype == np.uint16 and len(w.planted[0]) == 3
    w = make_config(2)
    assert w.params["num_pages"] == 2048 and w.k_data.shape == (2048, 2, 128, 64)
    assert sorted(np.unique(w.block_table).tolist()) == list(range(2048))
    assert all(len(v) == 8 for v in w.planted.values())
