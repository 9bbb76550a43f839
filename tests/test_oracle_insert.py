"""CPU pins of the oracle's KV-insert quantisers (oracle.kv_insert and its
encoders) against things other than themselves:

  E4M3 encoder   exhaustive round trip of every finite code; torch's
                 float8_e4m3fn cast (a library routine, round to nearest
                 even) on random and midpoint values inside its
                 non-saturating range; hand-worked ties and saturation
  E2M1 encoder   round trip of all 16 codes; hand-worked midpoints (each goes
                 to the even code); the input generator's independent C
                 encoder on random values
  kv_insert      brute force over all codes (every stored scale is the
                 nearest E4M3 value to max|y|/6, every element code the
                 nearest E2M1 value to y/scale), positions, untouched bytes,
                 nibble sharing of the dim-major V page, FP8 key scales
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from workloads import make_workload, make_new_tokens, KV_BF16, KV_NVFP4, IDX_BF16, IDX_FP8
from workloads import _native


def _finite_e4m3_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_e4m3_encode_round_trip():
    c = _finite_e4m3_codes()
    back = O.e4m3_encode(O.e4m3_to_f64(c))
    want = np.where(c == 0x80, 0, c)  # -0 is stored as +0
    assert np.array_equal(back, want)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12, np.log2(460.0), size=20000))
    v = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    vals = np.sort(np.unique(np.abs(O.e4m3_to_f64(_finite_e4m3_codes()))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32 (<= 5 bits)
    v = np.concatenate([v, mids, -mids, vals.astype(np.float32)])
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    t = np.where(t == 0x80, 0, t)  # torch keeps -0 for tiny negatives
    assert np.array_equal(O.e4m3_encode(v.astype(np.float64)), t)


def test_e4m3_encode_worked_values():
    cases = {0.0: 0x00, 1.0: 0x38, 1.0625: 0x38,  # tie 1 | 1.125 -> even code 0x38
             1.1875: 0x3A,                         # tie 1.125 | 1.25 -> 0x3A
             2.0 ** -10: 0x00,                     # tie 0 | 2^-9 -> 0
             1.5 * 2.0 ** -10: 0x01, 448.0: 0x7E, 450.0: 0x7E, 1e9: 0x7E,
             -1e9: 0xFE, -1e-9: 0x00, 0.015625: 0x08}
    for x, c in cases.items():
        assert int(O.e4m3_encode(x)) == c, (x, hex(c))


def test_e2m1_encode_round_trip_and_ties():
    codes = np.arange(16)
    assert np.array_equal(O.e2m1_encode(O.e2m1_to_f64(codes)), np.where(codes == 8, 0, codes))
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in ties.items():
        assert int(O.e2m1_encode(x)) == c and int(O.e2m1_encode(-x)) == (c | 8 if c else 0)
    worked = {0.3: 1, 0.74: 1, 0.76: 2, 5.01: 7, 100.0: 7, -0.1: 0, -6.0: 15, 2.4: 4, 2.6: 5}
    for x, c in worked.items():
        assert int(O.e2m1_encode(x)) == c, (x, c)


def test_e2m1_encode_matches_generator_encoder():
    lib = _native.lib()
    f = lib.msagen_e2m1_rne
    f.restype = ctypes.c_uint8
    f.argtypes = [ctypes.c_double]
    rng = np.random.default_rng(9)
    xs = np.concatenate([rng.normal(0, 3, 5000), rng.uniform(-7, 7, 5000)])
    gen = np.array([f(float(x)) for x in xs])
    assert np.array_equal(O.e2m1_encode(xs), gen)


def _brute_e4m3(a):
    vals = O.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    return int(best[0]) if best.size == 1 else int([c for c in best if c % 2 == 0][0])


def _brute_e2m1(y):
    vals = O.e2m1_to_f64(np.arange(16))
    d = np.abs(vals - y)
    best = np.flatnonzero(d == d.min())
    if best.size > 1:  # a tie (or +0 / -0): the even magnitude, +0 for zero
        mags = [c for c in best if (c & 7) % 2 == 0]
        best = [c for c in mags if c != 8] or mags
    return int(best[0])


def _insert_case(kv_dtype, idx_dtype, ctx, q_len, k_ts=1.0, v_ts=1.0, seed=21):
    w = make_workload("ins", seed, ctx, q_len, 8, 2, 4, kv_dtype, idx_dtype, table="permute",
                      k_tensor_scale=k_ts, v_tensor_scale=v_ts)
    nk, nv, ni = make_new_tokens(w, seed + 1, extremes=True)
    return w, nk, nv, ni, O.kv_insert(w, nk, nv, ni)


def _written(w):
    """(b, t, page, slot) of every new token the insert writes."""
    prm = w.params
    Tq, maxb = int(prm["q_len"]), int(prm["max_blocks_per_seq"])
    res = []
    for b in range(w.B):
        for t in range(Tq):
            pos = int(w.ctx_lens[b]) - Tq + t
            if 0 <= pos < maxb * 128:
                page = int(w.block_table[b, pos // 128])
                if 0 <= page < int(prm["num_pages"]):
                    res.append((b, t, page, pos % 128))
    return res


@pytest.mark.parametrize("ctx,q_len", [([300, 129, 1000], 4), ([257, 64], 3), ([200], 70)])
def test_kv_insert_nvfp4_brute_force(ctx, q_len):
    w, nk, nv, ni, out = _insert_case(KV_NVFP4, IDX_FP8, ctx, q_len, k_ts=0.75)
    G = int(w.params["num_kv_heads"])
    for b, t, page, slot in _written(w):
        for g in range(G):
            for which in ("k", "v"):
                x = O.bf16_to_f64((nk if which == "k" else nv)[b, t, g])
                y = x / (w.k_tensor_scale if which == "k" else w.v_tensor_scale)
                for c in range(8):
                    grp = y[16 * c:16 * c + 16]
                    if which == "k":
                        sc = int(out["k_scale"][page, g, slot, c])
                        codes = O.nibbles(out["k_data"][page, g, slot, 8 * c:8 * c + 8][None])[0]
                    else:
                        sc = int(out["v_scale"][page, g, c, slot])
                        byte = out["v_data"][page, g, 16 * c:16 * c + 16, slot // 2].astype(np.int64)
                        codes = (byte >> 4) if slot % 2 else (byte & 15)
                    assert sc == _brute_e4m3(np.max(np.abs(grp)) / 6.0)
                    s = float(O.e4m3_to_f64(np.uint8(sc)))
                    want = [(_brute_e2m1(v / s) if s > 0 else 0) for v in grp]
                    assert list(codes) == want, (b, t, g, which, c)


def test_kv_insert_fp8_keys_and_untouched_bytes():
    w, nk, nv, ni, out = _insert_case(KV_NVFP4, IDX_FP8, [300, 129, 1000], 4)
    wr = _written(w)
    for b, t, page, slot in wr:
        k = O.bf16_to_f64(ni[b, t])
        s = out["idx_k_scale"][page, slot]
        amax = np.max(np.abs(k))
        assert s == (np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0))
        assert [int(c) for c in out["idx_k"][page, slot]] == \
            [_brute_e4m3(abs(v) / float(s)) | (0x80 if v < 0 and _brute_e4m3(abs(v) / float(s)) else 0) for v in k]
    # nothing else moved: K rows, scales and indexer rows of other slots, and
    # the V nibbles of other tokens
    mask_tok = np.zeros(w.k_data.shape[:1] + (128,), dtype=bool)
    for _, _, page, slot in wr:
        mask_tok[page, slot] = True
    keep = ~mask_tok
    assert np.array_equal(out["k_data"].transpose(0, 2, 1, 3)[keep], w.k_data.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(out["k_scale"].transpose(0, 2, 1, 3)[keep], w.k_scale.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(out["v_scale"].transpose(0, 3, 1, 2)[keep], w.v_scale.transpose(0, 3, 1, 2)[keep])
    assert np.array_equal(out["idx_k"][keep], w.idx_k[keep])
    assert np.array_equal(out["idx_k_scale"][keep], w.idx_k_scale[keep])
    nib_old = np.stack([w.v_data & 15, w.v_data >> 4], axis=-1).reshape(w.v_data.shape[:3] + (128,))
    nib_new = np.stack([out["v_data"] & 15, out["v_data"] >> 4], axis=-1).reshape(nib_old.shape)
    keep_v = np.broadcast_to(keep[:, None, None, :], nib_old.shape)
    assert np.array_equal(nib_new[keep_v], nib_old[keep_v])


def test_kv_insert_positions_round_trip():
    # decode what landed at each new token's slot and bound it by the NVFP4
    # arithmetic: the stored scale s is within E4M3 rounding of max|y|/6 (half
    # a unit in the last place: 1/16 relative, or 2^-10 below the smallest
    # normal), unless max|y|/6 is past 448; each element is within
    # max(s, |y| - 6 s) of y (half an E2M1 gap is at most one scale unit;
    # beyond 6 s it saturates), and is 0 when s is 0
    w, nk, nv, ni, out = _insert_case(KV_NVFP4, IDX_FP8, [1000, 129], 4, seed=33)
    for b, t, page, slot in _written(w):
        for g in range(2):
            K = O.nvfp4_k_page(out["k_data"][page, g], out["k_scale"][page, g])[slot]
            V = O.nvfp4_v_page(out["v_data"][page, g], out["v_scale"][page, g])[slot]
            ks = O.e4m3_to_f64(out["k_scale"][page, g, slot])
            vs = O.e4m3_to_f64(out["v_scale"][page, g, :, slot])
            for x, dec, sc in ((O.bf16_to_f64(nk[b, t, g]), K, ks), (O.bf16_to_f64(nv[b, t, g]), V, vs)):
                for c in range(8):
                    grp, got, s = x[16 * c:16 * c + 16], dec[16 * c:16 * c + 16], float(sc[c])
                    ideal = np.max(np.abs(grp)) / 6.0
                    if ideal <= 448.0:
                        assert abs(s - ideal) <= max(ideal / 16, 2.0 ** -10)
                    else:
                        assert s == 448.0
                    err = np.abs(grp - got)
                    if s == 0:
                        assert np.all(got == 0)
                    else:
                        assert np.all(err <= np.maximum(s, np.abs(grp) - 6 * s) + 1e-12)


def test_kv_insert_bf16_cache_keeps_bits():
    w, nk, nv, ni, out = _insert_case(KV_BF16, IDX_BF16, [300, 129], 4)
    for b, t, page, slot in _written(w):
        assert np.array_equal(out["k_data"][page, 0, slot], nk[b, t, 0])
        assert np.array_equal(out["v_data"][page, 1, :, slot], nv[b, t, 1])
        assert np.array_equal(out["idx_k"][page, slot], ni[b, t])


# ------------------------------------------------ NVFP4 indexer keys

def test_nvfp4_index_keys_decode_worked_page():
    # a page whose slot 3 holds hand-made codes: dims 0/1 = 0.5/1.0 and dims
    # 30/31 = -6/3 under group scales 1.0 (0x38) and 2.0 (0x40), tensor 0.5
    from workloads import IDX_NVFP4
    w = make_workload("nvidx", 71, [256], 1, 8, 1, 4, KV_NVFP4, IDX_NVFP4, table="identity")
    w.idx_k[0, 3, :] = 0
    w.idx_k[0, 3, 0] = 0x21            # dim 0 code 1 (0.5), dim 1 code 2 (1.0)
    w.idx_k[0, 3, 15] = (0x5 << 4) | 0xF  # dim 30 code 15 (-6), dim 31 code 5 (3)
    w.idx_k_scale[0, 3, :] = [0x38, 0x40, 0x38, 0x38]
    w.idx_k_tensor_scale = 0.5
    keys, present = O.seq_indexer_keys(w, 0, 256)
    want = np.zeros(64)
    want[0], want[1] = 0.5 * 0.5, 1.0 * 0.5
    want[30], want[31] = -6 * 2.0 * 0.5, 3 * 2.0 * 0.5
    assert present[3] and np.array_equal(keys[3], want)


def test_nvfp4_index_keys_agree_with_fp8_keys_of_the_same_draws():
    # the generator quantises the same draws to FP8 (3 mantissa bits, one
    # scale per token) or to NVFP4 (one E4M3 scale per 16 dims): both decode
    # to within their own step of the draw, hence of each other
    from workloads import IDX_NVFP4
    wf = make_workload("f8", 72, [700, 300], 1, 8, 1, 4, KV_NVFP4, IDX_FP8, table="permute")
    wn = make_workload("f4", 72, [700, 300], 1, 8, 1, 4, KV_NVFP4, IDX_NVFP4, table="permute")
    for b in range(2):
        n = int(wf.ctx_lens[b])
        kf, _ = O.seq_indexer_keys(wf, b, n)
        kn, _ = O.seq_indexer_keys(wn, b, n)
        for c in range(4):
            gf, gn = kf[:, 16 * c:16 * c + 16], kn[:, 16 * c:16 * c + 16]
            amax = np.max(np.abs(gf), axis=1, keepdims=True)
            # NVFP4 step: one scale unit (amax/6 up to 1/16 rounding, or
            # 2^-10 below the smallest normal E4M3); FP8: 1/16 relative
            bound = np.maximum(amax / 6 * (1 + 1 / 16), 2.0 ** -10) + np.abs(gf) / 16 + 1e-12
            assert np.all(np.abs(gf - gn) <= bound)


def test_kv_insert_nvfp4_index_keys_brute_force():
    from workloads import IDX_NVFP4
    w = make_workload("nvins", 73, [300, 129, 5], 4, 8, 2, 4, KV_NVFP4, IDX_NVFP4, table="permute")
    w.idx_k_tensor_scale = 0.75
    nk, nv, ni = make_new_tokens(w, 74, extremes=True)
    out = O.kv_insert(w, nk, nv, ni)
    for b, t, page, slot in _written(w):
        y = O.bf16_to_f64(ni[b, t]) / 0.75
        codes = O.nibbles(out["idx_k"][page, slot][None])[0]
        for c in range(4):
            grp = y[16 * c:16 * c + 16]
            sc = int(out["idx_k_scale"][page, slot, c])
            assert sc == _brute_e4m3(np.max(np.abs(grp)) / 6.0)
            s = float(O.e4m3_to_f64(np.uint8(sc)))
            assert list(codes[16 * c:16 * c + 16]) == [(_brute_e2m1(v / s) if s > 0 else 0) for v in grp]
