"""Pins of the float64 oracle to things other than itself.

Each check takes the oracle module as an argument so that the mutation tests
can hand it a copy with a planted mistake and show that the check fails.
Nothing here re-types an oracle formula: the pins are library routines
(torch's float8/bfloat16 casts, torch's scaled_dot_product_attention), the
published E2M1 value table, hand-derived bytes (tests/golden), exact brute
force on tiny inputs (math.fsum loops, subset enumeration) and invariants the
method states.
"""
import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# E2M1 magnitudes as printed in the OCP Microscaling Formats spec (FP4 E2M1):
# codes 0..7 -> 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
E2M1_PUBLISHED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _same(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def check_e4m3(O):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    assert _same(got, ref), "E4M3 decode differs from torch.float8_e4m3fn"
    # closed forms of the format: smallest subnormal, smallest normal, 1, max
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and math.isnan(got[0x7F])
    assert got[0x80] == 0.0 and math.copysign(1.0, got[0x80]) == -1.0


def check_e2m1(O):
    got = O.e2m1_to_f64(np.arange(16))
    want = E2M1_PUBLISHED + [-v for v in E2M1_PUBLISHED]
    assert _same(got, want), "E2M1 decode differs from the published table"


def check_bf16(O):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                  # finite values only
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(O.bf16_to_f64(bits), ref), "bf16 decode differs from torch.bfloat16"


def check_layout_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_layout.json")))
    kd = np.zeros((128, 64), dtype=np.uint8)
    ks = np.zeros((128, 8), dtype=np.uint8)
    for tok, i, v in g["k_page"]["data"]:
        kd[tok, i] = v
    for tok, c, v in g["k_page"]["scale"]:
        ks[tok, c] = v
    K = O.nvfp4_k_page(kd, ks)
    for tok, d, v in g["k_page"]["expect"]:
        assert K[tok, d] == v, ("K", tok, d, K[tok, d], v)
    vd = np.zeros((128, 64), dtype=np.uint8)
    vs = np.zeros((8, 128), dtype=np.uint8)
    for d, i, v in g["v_page"]["data"]:
        vd[d, i] = v
    for c, tok, v in g["v_page"]["scale"]:
        vs[c, tok] = v
    V = O.nvfp4_v_page(vd, vs)
    for tok, d, v in g["v_page"]["expect"]:
        assert V[tok, d] == v, ("V", tok, d, V[tok, d], v)
    f = g["fp8_idx"]
    vals = O.e4m3_to_f64(np.array(f["codes"], dtype=np.uint8)) * f["scale"]
    assert list(vals) == f["expect"]


def _fsum_dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def check_indexer_bruteforce(O, seed=0):
    rng = np.random.default_rng(seed)
    for H, n in ((1, 5), (3, 7), (8, 4)):
        qi = rng.integers(-4, 5, size=(H, 64)).astype(np.float64) / 4
        keys = rng.integers(-4, 5, size=(n, 64)).astype(np.float64) / 8
        w = rng.uniform(0, 1, size=H)
        got = O.indexer_scores(qi, w, keys)
        for j in range(n):
            want = math.fsum(w[h] * max(0.0, _fsum_dot(qi[h], keys[j])) for h in range(H))
            assert abs(got[j] - want) <= 1e-12 * max(1.0, abs(want)), (H, n, j, got[j], want)


def check_indexer_relu(O):
    # head 1 is the negation of head 0: exactly one of the two dots is positive,
    # so s_j = w_{sign} * |<q0, k_j>|.
    rng = np.random.default_rng(1)
    q0 = rng.normal(size=64)
    qi = np.stack([q0, -q0])
    keys = rng.normal(size=(9, 64))
    w = np.array([0.25, 0.75])
    got = O.indexer_scores(qi, w, keys)
    for j in range(9):
        d = _fsum_dot(q0, keys[j])
        want = (0.25 if d > 0 else 0.75) * abs(d)
        assert abs(got[j] - want) <= 1e-12 * max(1.0, abs(want))
    assert np.all(O.indexer_scores(-np.abs(qi), w, np.abs(keys)) == 0.0)


def check_pool(O):
    rng = np.random.default_rng(2)
    for n in (1, 127, 128, 129, 300, 513):
        s = rng.normal(size=n)
        P = O.pool_blocks(s)
        assert P.shape[0] == (n + 127) // 128
        for i in range(P.shape[0]):
            assert P[i] == max(s[i * 128:min(n, i * 128 + 128)].tolist())
    s = rng.normal(size=300)
    present = np.ones(300, dtype=bool)
    present[128:256] = False
    P = O.pool_blocks(s, present)
    assert P[1] == -np.inf and P[0] == s[:128].max()


def _dominates(P, i, j):
    return P[i] > P[j] or (P[i] == P[j] and i < j)


def check_select_bruteforce(O, seed=3):
    rng = np.random.default_rng(seed)
    for n in (17, 18, 19, 20):
        for trial in range(3):
            P = rng.integers(0, 6, size=n).astype(np.float64)  # many exact ties
            if trial == 2:
                P = rng.normal(size=n)
            Pk = P.copy()
            Pk[-1] = np.inf
            found = []
            for S in itertools.combinations(range(n), 16):
                rest = set(range(n)) - set(S)
                if all(_dominates(Pk, i, j) for i in S for j in rest):
                    found.append(list(S))
            assert len(found) == 1
            assert list(O.select_blocks(P, 16, True)) == found[0], (P, found[0])


def check_select_rules(O):
    P = np.arange(40, dtype=np.float64)[::-1].copy()         # block 39 is the worst
    S = O.select_blocks(P, 16, True)
    assert 39 in S and len(S) == 16 and list(S) == list(range(15)) + [39]
    S = O.select_blocks(np.zeros(30), 16, True)              # all tied -> lowest indices
    assert list(S) == list(range(15)) + [29]
    assert list(O.select_blocks(np.zeros(30), 16, False)) == list(range(16))
    assert list(O.select_blocks(np.ones(16), 16, True)) == list(range(16))
    assert list(O.select_blocks(np.ones(5), 16, True)) == list(range(5))


def _sdpa(q, K, V, scale, mask=None):
    qt = torch.from_numpy(q)[None]
    Kt = torch.from_numpy(K)[None]
    Vt = torch.from_numpy(V)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m, scale=scale)[0].numpy()


def check_attend_sdpa(O, seed=4):
    rng = np.random.default_rng(seed)
    for n in (1, 5, 300):
        q = rng.normal(size=(6, 128))
        K = rng.normal(size=(n, 128))
        V = rng.normal(size=(n, 128))
        o, lse = O.attend(q, K, V, 0.088)
        assert np.max(np.abs(o - _sdpa(q, K, V, 0.088))) <= 1e-12
        ref_lse = np.array([math.log(math.fsum(math.exp(0.088 * _fsum_dot(q[h], K[j])) for j in range(n)))
                            for h in range(6)])
        assert np.max(np.abs(lse - ref_lse)) <= 1e-11
    # one key: o = v; two keys with equal logits: o = mean
    q = rng.normal(size=(1, 128))
    K = rng.normal(size=(1, 128))
    V = rng.normal(size=(1, 128))
    o, _ = O.attend(q, K, V, 0.1)
    assert np.max(np.abs(o[0] - V[0])) <= 1e-15
    K2 = np.concatenate([K, K])
    V2 = rng.normal(size=(2, 128))
    o, lse = O.attend(q, K2, V2, 0.1)
    assert np.max(np.abs(o[0] - V2.mean(axis=0))) <= 1e-15
    o, lse = O.attend(q, np.zeros((0, 128)), np.zeros((0, 128)), 0.1)
    assert np.all(o == 0) and lse[0] == -np.inf


def _dense_all_keys(w, O, b, t):
    """Dense attention over every visible key of the sequence via SDPA."""
    prm = w.params
    Hq, G = prm["num_q_heads"], prm["num_kv_heads"]
    grp = Hq // G
    Lb = int(w.ctx_lens[b])
    p_t = Lb - prm["q_len"] + t
    scale = 1.0 / math.sqrt(128) if prm["softmax_scale"] <= 0 else prm["softmax_scale"]
    q = torch.from_numpy(w.q[b, t].astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    out = np.zeros((Hq, 128))
    for g in range(G):
        Ks, Vs = [], []
        for blk in range((p_t + 128) // 128):
            page = int(w.block_table[b, blk])
            if prm["kv_dtype"] == 1:
                # decode through the torch float8 cast, not the oracle's decoder
                kc = w.k_data[page, g]
                ksc = torch.from_numpy(w.k_scale[page, g].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                codes = np.stack([kc & 15, kc >> 4], axis=-1).reshape(128, 128)
                mag = np.array(E2M1_PUBLISHED)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
                Ks.append(mag * np.repeat(ksc, 16, axis=1) * w.k_tensor_scale)
                vc = w.v_data[page, g]                      # [d][64]
                vsc = torch.from_numpy(w.v_scale[page, g].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                vcodes = np.stack([vc & 15, vc >> 4], axis=-1).reshape(128, 128)  # [d][tok]
                vmag = np.array(E2M1_PUBLISHED)[vcodes & 7] * np.where(vcodes & 8, -1.0, 1.0)
                Vs.append((vmag * np.repeat(vsc, 16, axis=0)).T * w.v_tensor_scale)
            else:
                kb = torch.from_numpy(w.k_data[page, g].astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
                vb = torch.from_numpy(w.v_data[page, g].astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
                Ks.append(kb)
                Vs.append(vb.T)
        K = np.concatenate(Ks)[:p_t + 1]
        V = np.concatenate(Vs)[:p_t + 1]
        out[g * grp:(g + 1) * grp] = _sdpa(q[g * grp:(g + 1) * grp], K, V, scale)
    return out


def check_dense_equivalence(O, w):
    """Contexts of at most 16 blocks: MSA equals dense attention over all keys."""
    for b in range(w.B):
        for t, r in enumerate(O.decode_sequence(w, b)):
            if r["p"] < 0 or (r["p"] + 128) // 128 > w.params["top_k"]:
                continue
            dense = _dense_all_keys(w, O, b, t)
            assert np.max(np.abs(r["out"] - dense)) <= 1e-12, (b, t)


def check_sparse_masked_sdpa(O, w):
    """Any context: MSA output equals dense SDPA with a boolean mask that keeps
    exactly the keys of the selected blocks (library routine on the torch-decoded
    cache), and the selection obeys the stated invariants."""
    top_k = w.params["top_k"]
    for b in range(w.B):
        for t, r in enumerate(O.decode_sequence(w, b)):
            p_t = r["p"]
            if p_t < 0:
                continue
            nblk = (p_t + 128) // 128
            S = list(r["sel"])
            assert len(S) == min(top_k, nblk)
            assert r["n_keys"] <= top_k * 128
            if w.params["keep_last"]:
                assert nblk - 1 in S
            for blk in w.planted.get(b, []):
                assert blk in S, ("planted block not selected", b, t, blk)
            prm = w.params
            Hq, G = prm["num_q_heads"], prm["num_kv_heads"]
            grp = Hq // G
            scale = 1.0 / math.sqrt(128) if prm["softmax_scale"] <= 0 else prm["softmax_scale"]
            q = torch.from_numpy(w.q[b, t].astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
            for g in range(G):
                K = np.concatenate([O.block_kv(w, b, i, g)[0] for i in range(nblk)])[:p_t + 1]
                V = np.concatenate([O.block_kv(w, b, i, g)[1] for i in range(nblk)])[:p_t + 1]
                keep = np.zeros(p_t + 1, dtype=bool)
                for i in S:
                    keep[i * 128:(i + 1) * 128] = True
                mask = np.broadcast_to(keep, (grp, p_t + 1)).copy()
                ref = _sdpa(q[g * grp:(g + 1) * grp], K, V, scale, mask)
                assert np.max(np.abs(r["out"][g * grp:(g + 1) * grp] - ref)) <= 1e-12


def _single_token_view(w, t):
    """The same cache seen by query token t alone: q_len 1, context cut to the
    token's own position + 1."""
    import copy
    v = copy.copy(w)
    v.params = dict(w.params)
    v.params["q_len"] = 1
    v.q = w.q[:, t:t + 1]
    v.idx_q = w.idx_q[:, t:t + 1]
    v.idx_w = w.idx_w[:, t:t + 1]
    v.ctx_lens = (w.ctx_lens - w.params["q_len"] + t + 1).astype(np.int32)
    return v


def check_causal_positions(O, w):
    """With T_q > 1, query token t behaves exactly like a single-token decode
    over the context cut after its own position (causal inside the window),
    and the last token of a context of at most 16 blocks attends to all L keys
    (the context length counts the new tokens)."""
    Tq = w.params["q_len"]
    assert Tq > 1
    for b in range(w.B):
        res = O.decode_sequence(w, b, want_scores=True)
        for t, r in enumerate(res):
            single = O.decode_sequence(_single_token_view(w, t), b, want_scores=True)[0]
            assert np.array_equal(r["scores"], single["scores"])
            assert list(r["sel"]) == list(single["sel"])
            assert np.array_equal(r["out"], single["out"])
        L = int(w.ctx_lens[b])
        if L <= 16 * 128:
            assert res[-1]["n_keys"] == L


def _rank_by_dominance(Pk):
    """rank[i] = number of blocks that beat block i under (score desc, index
    asc), counted pair by pair (no sort)."""
    n = len(Pk)
    return [sum(1 for j in range(n) if _dominates(Pk, j, i)) for i in range(n)]


def check_boundary_bruteforce(O, seed=6):
    """boundary_values(P, k, keep_last) = (the score ranked k-th, the score
    ranked (k+1)-th) of the keep-last-adjusted pooled scores, ranks counted by
    pairwise dominance; (None, None) when every block is selected. Also: the
    k-th value is the smallest adjusted score inside the selected set and the
    (k+1)-th the largest outside it."""
    rng = np.random.default_rng(seed)
    cases = []
    for n in (2, 5, 16, 17, 18, 23, 40):
        for trial in range(3):
            if trial == 0:
                P = rng.integers(0, 4, size=n).astype(np.float64)     # exact ties
            elif trial == 1:
                P = rng.normal(size=n)
            else:
                P = np.full(n, 0.5)                                    # all tied
            cases.append(P)
    cases.append(np.array([3.0, -1.0, 7.0, 7.0, -np.inf, 2.0, 7.0, 0.0, 1.0, 5.0]))
    for P in cases:
        n = len(P)
        for top_k in (1, 2, 4, 16):
            for keep_last in (True, False):
                got = O.boundary_values(P, top_k, keep_last)
                if n <= top_k:
                    assert got == (None, None), (P, top_k, keep_last, got)
                    continue
                Pk = [float(x) for x in P]
                if keep_last:
                    Pk[-1] = math.inf
                rank = _rank_by_dominance(Pk)
                want_k = [Pk[i] for i in range(n) if rank[i] == top_k - 1]
                want_k1 = [Pk[i] for i in range(n) if rank[i] == top_k]
                assert len(want_k) == 1 and len(want_k1) == 1
                assert got == (want_k[0], want_k1[0]), (list(P), top_k, keep_last, got, want_k, want_k1)
                # values only: the k-th / (k+1)-th of the adjusted scores sorted descending
                srt = sorted(Pk, reverse=True)
                assert got == (srt[top_k - 1], srt[top_k])
                S = set(int(i) for i in O.select_blocks(P, top_k, keep_last))
                assert got[0] == min(Pk[i] for i in S)
                assert got[1] == max(Pk[i] for i in range(n) if i not in S)
