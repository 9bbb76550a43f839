"""Helpers of the GPU parity tests: run the HIP path through the C ABI on a
host workload and compare with the oracle. Tolerances (stated once here):

  dequant             bit-exact (value and sign of zero)
  indexer scores      |gpu - oracle| <= 1e-5 * max_j |oracle score| per query
                      token (fp32 dot products of exact bf16 operands)
  pooled scores       same bound
  selection           bit-exact, except a token whose selected sets differ
                      only in blocks whose oracle pooled score is within 1e-4
                      (relative) of the k-th ranked pooled score; such tokens
                      are counted and reported
  attention output    against the oracle under the GPU's own selection
                      (fp32 accumulate, bf16 output), element by element:
                      |o| < 0.5:  |gpu - o| <= 2e-3
                      |o| >= 0.5: |gpu - o| <= ulp(o)/2 + slack, where ulp
                      is bf16's at |o| (ulp/2 >= 1.95e-3 there: the output
                      format alone cannot hold 2e-3) and slack is the
                      first-order effect of the one rounding the kernel adds
                      before the output: the softmax weights p_j are rounded
                      to the matrix-core operand format (fp16 for NVFP4 K/V,
                      relative error <= u = 2^-11; bf16 for a bf16 cache,
                      u = 2^-9), which moves o_d by at most
                      u * sum_j p_j |v_jd - o_d|, plus 2^-20 times that sum
                      and |o| for the fp32 exp2, accumulation and division.
                      Mean-abs <= 2e-4 over all elements, against the
                      unrounded oracle when strict (the decode workloads,
                      whose outputs are small), else against the oracle
                      rounded to bf16 (short contexts, where outputs are O(1)
                      and bf16 rounding alone exceeds 2e-4 on average).
  lse                 abs 2e-3
"""
import math

import numpy as np
import torch

import block_sparse_attention_kv_amd as msa
from oracle import msa_oracle as O

OUT_MAX_ABS = 2e-3
OUT_MEAN_ABS = 2e-4
LSE_ABS = 2e-3
SCORE_REL = 1e-5
TIE_REL = 1e-4


def bf16_to_np(t):
    return (t.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Run:
    """Device copy of a workload plus output buffers."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.params, self.cache, qs = msa.to_device(w, device)
        self.q, self.idx_q, self.idx_w = qs["q"], qs["idx_q"], qs["idx_w"]
        prm = w.params
        B, Tq, Hq = prm["num_seqs"], prm["q_len"], prm["num_q_heads"]
        self.shape_out = (B, Tq, Hq, 128)
        self.device = device

    def layer(self, want_lse=True, single=False):
        """msa_decode_layer, or msa_decode_layer_single when single."""
        prm = self.w.params
        B, Tq, Hq, K = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["top_k"]
        out = torch.empty(self.shape_out, dtype=torch.int16, device=self.device)
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=self.device) if want_lse else None
        sel = torch.empty((B, Tq, K), dtype=torch.int32, device=self.device)
        ws = msa.alloc_workspace(self.params, self.device)
        fn = msa.msa_decode_layer_single if single else msa.msa_decode_layer
        fn(self.params, self.cache, self.q, self.idx_q, self.idx_w, out, ws, lse=lse, sel_out=sel)
        torch.cuda.synchronize()
        return dict(out=bf16_to_np(out), out_bits=out.cpu().numpy(), lse=None if lse is None else lse.cpu().numpy().astype(np.float64),
                    sel=sel.cpu().numpy())

    def scores(self):
        prm = self.w.params
        B, Tq, maxb = prm["num_seqs"], prm["q_len"], prm["max_blocks_per_seq"]
        sc = torch.empty((B, Tq, maxb * 128), dtype=torch.float32, device=self.device)
        msa.msa_indexer_scores(self.params, self.cache, self.idx_q, self.idx_w, sc)
        torch.cuda.synchronize()
        return sc

    def pool_select(self, scores):
        prm = self.w.params
        B, Tq, maxb, K = prm["num_seqs"], prm["q_len"], prm["max_blocks_per_seq"], prm["top_k"]
        pooled = torch.empty((B, Tq, maxb), dtype=torch.float32, device=self.device)
        sel = torch.empty((B, Tq, K), dtype=torch.int32, device=self.device)
        nsel = torch.empty((B, Tq), dtype=torch.int32, device=self.device)
        msa.msa_pool_select_blocks(self.params, self.cache.ctx_lens, scores, sel, pooled=pooled, nsel=nsel)
        torch.cuda.synchronize()
        return pooled.cpu().numpy().astype(np.float64), sel.cpu().numpy(), nsel.cpu().numpy()

    def attend(self, sel_np, want_lse=True):
        prm = self.w.params
        B, Tq, Hq = prm["num_seqs"], prm["q_len"], prm["num_q_heads"]
        sel = torch.from_numpy(np.ascontiguousarray(sel_np, dtype=np.int32)).to(self.device)
        out = torch.empty(self.shape_out, dtype=torch.int16, device=self.device)
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=self.device) if want_lse else None
        msa.msa_sparse_attn_decode(self.params, self.cache, self.q, sel, out, lse=lse)
        torch.cuda.synchronize()
        return bf16_to_np(out), None if lse is None else lse.cpu().numpy().astype(np.float64)


def check_scores(gpu, ref, label=""):
    """gpu/ref: [n] scores of one query token (ref float64, -inf masked)."""
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin), (label, "finite pattern differs")
    if fin.any():
        scale = max(np.max(np.abs(ref[fin])), 1e-30)
        err = np.max(np.abs(gpu[fin] - ref[fin]))
        assert err <= SCORE_REL * scale, (label, err, scale)


def check_selection(gpu_sel, pooled_ref, sel_ref, top_k, keep_last, label=""):
    """Returns 1 if the sets differ within the tie band, 0 if identical; fails
    otherwise. pooled_ref: oracle pooled scores of the visible blocks."""
    g = [int(x) for x in gpu_sel if x >= 0]
    assert g == sorted(g), (label, "selection not ascending", g)
    assert all(x == -1 for x in gpu_sel[len(g):]), (label, "padding is not -1", gpu_sel)
    o = [int(x) for x in sel_ref]
    if g == o:
        return 0
    assert len(g) == len(o), (label, g, o)
    kth, _ = O.boundary_values(pooled_ref, top_k, keep_last)
    assert kth is not None and np.isfinite(kth), (label, g, o)
    for blk in set(g) ^ set(o):
        v = pooled_ref[blk]
        assert abs(v - kth) <= TIE_REL * max(abs(kth), 1e-30), (label, "selection differs outside the tie band",
                                                                 blk, v, kth, g, o)
    return 1


def bf16_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def bf16_round(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# unit roundoff of the softmax weights' operand format: fp16 (NVFP4 K/V), bf16 (bf16 K/V)
P_ROUND = {1: 2.0 ** -11, 0: 2.0 ** -9}
FP32_SLACK = 2.0 ** -20  # exp2, accumulation and the final division in fp32


def attend_with_slack(w, b, t, blocks, p_t):
    """The oracle's output under `blocks` plus the per-element slack of the
    rounding of the softmax weights: u * sum_j p_j |v_jd - o_d| (u = P_ROUND
    of the cache's K/V format, p_j = the oracle's softmax weights, v_j its
    decoded values)."""
    o, lse = O.attend_token(w, b, t, blocks, p_t)
    prm = w.params
    Hq, G = int(prm["num_q_heads"]), int(prm["num_kv_heads"])
    grp = Hq // G
    q = O.bf16_to_f64(w.q[b, t])
    scale = O.softmax_scale(prm)
    spread = np.zeros_like(o)
    for g in range(G):
        K, V = O.gather_selected(w, b, blocks, g, p_t)
        if K.shape[0] == 0:
            continue
        hs = slice(g * grp, (g + 1) * grp)
        p = np.exp(scale * (q[hs] @ K.T) - lse[hs, None])            # [grp][n]
        spread[hs] = np.stack([p[i] @ np.abs(V - o[g * grp + i]) for i in range(grp)])
    return o, lse, (P_ROUND[int(prm["kv_dtype"])] + FP32_SLACK) * spread + FP32_SLACK * np.abs(o)


def check_out(gpu, ref, slack, label="", strict=False):
    """Returns (max-abs over |o| < 0.5, max-abs overall, mean-abs). slack:
    per-element slack where |o| >= 0.5 (attend_with_slack)."""
    gpu, ref = np.asarray(gpu).ravel(), np.asarray(ref).ravel()
    slack = np.asarray(slack).ravel()
    err = np.abs(gpu - ref)
    big = np.abs(ref) >= 0.5
    bound = np.where(big, 0.5 * bf16_ulp(ref) + slack, OUT_MAX_ABS)
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), (label, "beyond the element bound", float(err[worst]), float(bound[worst]),
                                  float(ref[worst]), float(gpu[worst]))
    small = ~big
    mx_small = float(err[small].max()) if small.any() else 0.0
    if strict:
        assert err.mean() <= OUT_MEAN_ABS, (label, "mean-abs", float(err.mean()))
    else:
        err_r = np.abs(gpu - bf16_round(ref))
        assert err_r.mean() <= OUT_MEAN_ABS, (label, "mean-abs vs bf16-rounded oracle", float(err_r.mean()))
    return mx_small, float(err.max()), float(err.mean())


def check_lse(gpu, ref, label=""):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin), (label, "lse finite pattern differs")
    if fin.any():
        err = np.max(np.abs(gpu[fin] - ref[fin]))
        assert err <= LSE_ABS, (label, "lse", err)


def indexer_parity(w, run=None):
    """Unfused indexer scores, pool and selection vs the oracle for every
    (sequence, token); returns the number of tie-band selection
    differences."""
    run = run or Run(w)
    sc = run.scores()
    pooled, sel, nsel = run.pool_select(sc)
    scn = sc.cpu().numpy().astype(np.float64)
    ref = O.decode_layer(w, want_scores=True)
    prm = w.params
    ties = 0
    for b in range(prm["num_seqs"]):
        for t in range(prm["q_len"]):
            lab = "%s b=%d t=%d" % (w.name, b, t)
            check_scores(scn[b, t], ref["scores"][b, t], lab)
            n = int(ref["nsel"][b, t])
            assert nsel[b, t] == n, lab
            check_scores(pooled[b, t], ref["pooled"][b, t], lab + " pooled")
            p_t = min(int(w.ctx_lens[b]), prm["max_blocks_per_seq"] * 128) - prm["q_len"] + t
            nb = p_t // 128 + 1 if p_t >= 0 else 0
            ties += check_selection(sel[b, t], ref["pooled"][b, t][:nb], ref["sel"][b, t][:n],
                                    prm["top_k"], prm["keep_last"], lab)
    return ties


def oracle_outputs(w, sel, tokens=None):
    """The oracle's outputs, lse and output slack (attend_with_slack) of every
    (sequence, token) under the selection array sel [B][Tq][top_k]
    (-1 padded)."""
    prm = w.params
    B, Tq, Hq = int(prm["num_seqs"]), int(prm["q_len"]), int(prm["num_q_heads"])
    o = np.zeros((B, Tq, Hq, 128))
    lse = np.full((B, Tq, Hq), -np.inf)
    slack = np.zeros((B, Tq, Hq, 128))
    for b in range(B):
        for t in (range(Tq) if tokens is None else tokens):
            p_t = O.query_position(w.ctx_lens[b], Tq, t, prm["max_blocks_per_seq"])
            if p_t < 0:
                continue
            S = [int(x) for x in sel[b, t] if x >= 0]
            o[b, t], lse[b, t], slack[b, t] = attend_with_slack(w, b, t, S, p_t)
    return o, lse, slack


def compare_layer(w, res, refs, seqs=None, strict=False, label=None):
    """Compare one layer call's results `res` (Run.layer) with the oracle's
    per-sequence results refs[b] (decode_sequence lists) for the sequences
    `seqs` (default: all of refs). Returns (tie-band selection differences,
    max-abs where |o| < 0.5, mean-abs)."""
    prm = w.params
    label = label or w.name
    ties, gots, want, slacks = 0, [], [], []
    for b in (sorted(refs) if seqs is None else seqs):
        for r in refs[b]:
            t = r["t"]
            lab = "%s b=%d t=%d" % (label, b, t)
            if r["p"] < 0:
                assert np.all(res["sel"][b, t] == -1), lab
                assert np.all(res["out"][b, t] == 0), lab
                continue
            ties += check_selection(res["sel"][b, t], r["pooled"], r["sel"], prm["top_k"], prm["keep_last"], lab)
            S = [int(x) for x in res["sel"][b, t] if x >= 0]
            if S == [int(x) for x in r["sel"]]:
                o, lse, sl = r["out"], r["lse"], r["slack"]
            else:
                o, lse, sl = attend_with_slack(w, b, t, S, r["p"])
            gots.append(res["out"][b, t].ravel())
            want.append(o.ravel())
            slacks.append(sl.ravel())
            check_lse(res["lse"][b, t], lse, lab)
    mx, mx_all, mean = check_out(np.concatenate(gots), np.concatenate(want), np.concatenate(slacks), label, strict)
    return ties, mx, mean


def oracle_refs(w, seqs=None, tokens=None):
    """decode_sequence of the listed sequences (default all), each token's
    dict extended with its index t and the output slack under the oracle's
    own selection."""
    refs = {}
    for b in (range(w.B) if seqs is None else seqs):
        res = O.decode_sequence(w, b, tokens=tokens)
        for i, r in enumerate(res):
            r["t"] = i if tokens is None else tokens[i]
            r["slack"] = np.zeros_like(r["out"])
            if r["p"] >= 0:
                _, _, r["slack"] = attend_with_slack(w, b, r["t"], [int(x) for x in r["sel"]], r["p"])
        refs[b] = res
    return refs


def layer_parity(w, run=None, seqs=None, tokens=None, strict=False, single=False):
    """Fused layer (the single-launch one when single) vs the oracle for the
    listed sequences (default all). Returns (number of tie-band selection
    differences, max-abs where |o| < 0.5, mean-abs)."""
    run = run or Run(w)
    res = run.layer(single=single)
    return compare_layer(w, res, oracle_refs(w, seqs, tokens), strict=strict)
