"""Float64 CPU oracle of MSA (MiniMax Sparse Attention) decode.

TEST INFRASTRUCTURE ONLY. This module is the reference the HIP kernels are
checked against. Only the tests, the smoke check of __graft_entry__ and the
cpu_baseline leg of bench.py may import it; the library path never does. It
shares no code with the HIP path or with the input generator: it reads the
stored bytes (layouts of include/msa.h) and decodes them with its own
bit-field arithmetic.

What it computes, step by step, for sequence b and query token t
[page "vLLM Adds Day-0 Support for MiniMax-M3.1-Flash on NVIDIA and AMD GPUs"
(ainewsbites.com), section "A model built for efficient inference": the cache
is split into 128-token blocks, an indexer scores every key, the scores are
pooled into one score per block, exact attention runs over the top 16 blocks
only, the most recent block is always kept, so at most 2,048 keys per query]:

 1. decode   NVFP4 K/V  x = e2m1(code) * e4m3(scale of its 16-group) * ts
             FP8 indexer keys  k = e4m3(code) * per-token fp32 scale
             NVFP4 indexer keys  k = e2m1(code) * e4m3(16-group scale) * ts
             bf16 values exactly.
 2. position p_t = L_b - T_q + t; keys 0..p_t are visible.
 3. indexer  s_j = sum_h w_h * max(0, <qi_h, k_j>)           (reading c1)
 4. pool     P_i = max of s_j over the visible keys of block i (reading c2)
 5. select   top_k blocks by (P desc, index asc), the block holding p_t
             first when keep_last (readings c3, c7)
 6. attend   o = softmax(scale * q K^T) V over the visible keys of the
             selected blocks, lse = log sum exp(scale * q K^T)  (exact)

Before the decode, kv_insert (section 0) writes new tokens into the caches:
the NVFP4 quantiser (E4M3 scale of max|y|/6 per 16 elements, E2M1 codes)
and the FP8 indexer-key quantiser (per-token scale max|k|/448), each
rounding to the nearest representable value with ties to the even code
[same page, section "Kernel and serving optimizations": the KV-insert step].

The readings (c1..c17) are listed, with their reasons, in the design notes of
the repository. Every function below is pinned by CPU tests to something
other than itself: exhaustive decoder tables against torch's float8 cast and
the closed-form E2M1 values, special cases that reduce to a plain dot
product, a brute-force subset search for the selection, and PyTorch's
scaled_dot_product_attention for the attention step.
"""
import math

import numpy as np

BLOCK = 128
HEAD_DIM = 128
IDX_DIM = 64


# ---------------------------------------------------------------- 1. decode

def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes):
    """OCP E4M3 (e4m3fn) bytes -> float64 from the bit fields: sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 is
    subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e2m1_to_f64(codes):
    """4-bit E2M1 codes (0..15) -> float64 from the bit fields: sign bit 3,
    exponent bits 2..1 with bias 1, mantissa bit 0; exponent field 0 is
    subnormal (m * 0.5). Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; code 8 is -0."""
    c = np.asarray(codes, dtype=np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(sign == 1, -mag, mag)


def nibbles(byte_rows):
    """u8[..., n] -> int codes[..., 2n]; element 2i is the low nibble of byte i."""
    b = np.asarray(byte_rows, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def nvfp4_k_page(data, scale):
    """One K page of one KV head: data u8[128 tok][64], scale u8[128 tok][8]
    -> float64 [128 tok][128 d] without the tensor scale."""
    vals = e2m1_to_f64(nibbles(data))                      # [tok][128]
    s = e4m3_to_f64(scale)                                  # [tok][8]
    return vals * np.repeat(s, 16, axis=1)


def nvfp4_v_page(data, scale):
    """One V page of one KV head in the dim-major layout: data u8[128 d][64]
    (byte i of row d holds tokens 2i, 2i+1), scale u8[8][128 tok]
    -> float64 [128 tok][128 d] without the tensor scale."""
    vals_dt = e2m1_to_f64(nibbles(data))                    # [d][tok]
    s = e4m3_to_f64(scale)                                  # [c][tok]
    return (vals_dt * np.repeat(s, 16, axis=0)).T          # [tok][d]


def _page_ok(page, num_pages):
    return 0 <= page < num_pages


def seq_indexer_keys(w, b, n_tok):
    """Indexer keys of tokens 0..n_tok-1 of sequence b -> float64 [n_tok][64]
    and a bool mask of tokens whose page is present."""
    P = int(w.params["num_pages"])
    maxb = int(w.params["max_blocks_per_seq"])
    nblk = (n_tok + BLOCK - 1) // BLOCK
    keys = np.zeros((nblk * BLOCK, IDX_DIM))
    present = np.zeros(nblk * BLOCK, dtype=bool)
    fmt = int(w.params["idx_dtype"])
    for i in range(min(nblk, maxb)):
        page = int(w.block_table[b, i])
        if not _page_ok(page, P):
            continue
        sl = slice(i * BLOCK, (i + 1) * BLOCK)
        if fmt == 1:
            keys[sl] = e4m3_to_f64(w.idx_k[page]) * w.idx_k_scale[page].astype(np.float64)[:, None]
        elif fmt == 2:
            vals = e2m1_to_f64(nibbles(w.idx_k[page]))                       # [tok][64]
            keys[sl] = vals * np.repeat(e4m3_to_f64(w.idx_k_scale[page]), 16, axis=1) * \
                float(getattr(w, "idx_k_tensor_scale", 1.0))
        else:
            keys[sl] = bf16_to_f64(w.idx_k[page])
        present[sl] = True
    return keys[:n_tok], present[:n_tok]


def block_kv(w, b, blk, g):
    """K and V of block `blk` of sequence b, KV head g -> float64 [128][128]
    each (tensor scales applied), or None if its page is absent."""
    P = int(w.params["num_pages"])
    page = int(w.block_table[b, blk])
    if not _page_ok(page, P):
        return None
    if int(w.params["kv_dtype"]) == 1:
        K = nvfp4_k_page(w.k_data[page, g], w.k_scale[page, g]) * float(w.k_tensor_scale)
        V = nvfp4_v_page(w.v_data[page, g], w.v_scale[page, g]) * float(w.v_tensor_scale)
    else:
        K = bf16_to_f64(w.k_data[page, g])
        V = bf16_to_f64(w.v_data[page, g]).T
    return K, V


# -------------------------------------------------------------- 2. position

def query_position(L, q_len, t, max_blocks):
    """p_t = L - q_len + t with L clamped to max_blocks*128 (device contract)."""
    L = min(int(L), int(max_blocks) * BLOCK)
    return L - int(q_len) + int(t)


# --------------------------------------------------------------- 3. indexer

def indexer_scores(qi, wts, keys):
    """s_j = sum_h wts[h] * max(0, <qi[h], keys[j]>).
    qi float64 [H][64], wts float64 [H], keys float64 [n][64] -> [n]."""
    dots = keys @ qi.T                                      # [n][H]
    return np.maximum(dots, 0.0) @ wts


# ------------------------------------------------------------------ 4. pool

def pool_blocks(scores, present=None):
    """P_i = max of the scores of block i (the last block may be partial);
    blocks whose page is absent pool to -inf."""
    n = scores.shape[0]
    nblk = (n + BLOCK - 1) // BLOCK
    P = np.full(nblk, -np.inf)
    for i in range(nblk):
        seg = scores[i * BLOCK:min(n, (i + 1) * BLOCK)]
        if present is not None:
            seg = seg[present[i * BLOCK:min(n, (i + 1) * BLOCK)]]
        if seg.size:
            P[i] = seg.max()
    return P


# ---------------------------------------------------------------- 5. select

def select_blocks(P, top_k, keep_last=True):
    """Indices of the top_k blocks by (P desc, index asc), ascending; with
    keep_last the last block ranks first. Fewer than top_k blocks: all."""
    n = P.shape[0]
    if n <= top_k:
        return np.arange(n, dtype=np.int64)
    Pk = P.astype(np.float64).copy()
    if keep_last:
        Pk[n - 1] = np.inf
    order = np.lexsort((np.arange(n), -Pk))                 # primary -P, then index
    return np.sort(order[:top_k])


def boundary_values(P, top_k, keep_last=True):
    """(P'_k, P'_{k+1}): the k-th and (k+1)-th ranked keep-last-adjusted pooled
    scores, or (None, None) when every block is selected."""
    n = P.shape[0]
    if n <= top_k:
        return None, None
    Pk = P.astype(np.float64).copy()
    if keep_last:
        Pk[n - 1] = np.inf
    order = np.lexsort((np.arange(n), -Pk))
    return float(Pk[order[top_k - 1]]), float(Pk[order[top_k]])


# ---------------------------------------------------------------- 6. attend

def attend(q, K, V, scale):
    """Exact softmax attention of the query rows q [H][128] over keys K [n][128]
    and values V [n][128]: o = softmax(scale q K^T) V, lse = log sum exp.
    With n == 0: o = 0, lse = -inf."""
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    z = scale * (q @ K.T)                                   # [H][n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    den = e.sum(axis=1, keepdims=True)
    return (e @ V) / den, (m + np.log(den))[:, 0]


def gather_selected(w, b, blocks, g, p_t):
    """Concatenate K/V of the visible keys (position <= p_t) of the selected
    blocks of sequence b for KV head g. Absent or out-of-range blocks are
    skipped."""
    maxb = int(w.params["max_blocks_per_seq"])
    Ks, Vs = [], []
    for blk in blocks:
        blk = int(blk)
        if blk < 0 or blk >= maxb:
            continue
        kv = block_kv(w, b, blk, g)
        if kv is None:
            continue
        n_vis = min(BLOCK, p_t + 1 - blk * BLOCK)
        if n_vis <= 0:
            continue
        Ks.append(kv[0][:n_vis])
        Vs.append(kv[1][:n_vis])
    if not Ks:
        return np.zeros((0, HEAD_DIM)), np.zeros((0, HEAD_DIM))
    return np.concatenate(Ks), np.concatenate(Vs)


def softmax_scale(params):
    s = float(params["softmax_scale"])
    return s if s > 0 else 1.0 / math.sqrt(HEAD_DIM)


def attend_token(w, b, t, blocks, p_t=None):
    """Attention output of query token t of sequence b over `blocks` for all
    query heads -> (o float64 [Hq][128], lse float64 [Hq])."""
    prm = w.params
    Hq, G = int(prm["num_q_heads"]), int(prm["num_kv_heads"])
    grp = Hq // G
    if p_t is None:
        p_t = query_position(w.ctx_lens[b], prm["q_len"], t, prm["max_blocks_per_seq"])
    q = bf16_to_f64(w.q[b, t])                              # [Hq][128]
    o = np.zeros((Hq, HEAD_DIM))
    lse = np.full(Hq, -np.inf)
    if p_t < 0:
        return o, lse
    sc = softmax_scale(prm)
    for g in range(G):
        K, V = gather_selected(w, b, blocks, g, p_t)
        o[g * grp:(g + 1) * grp], lse[g * grp:(g + 1) * grp] = attend(q[g * grp:(g + 1) * grp], K, V, sc)
    return o, lse


# ------------------------------------------------------- 0. KV-insert

def _nearest_code(a, table):
    """Index of the value of `table` (ascending, non-negative) nearest to each
    a >= 0; a tie between two neighbours goes to the even index (the even
    code: the mantissa's last bit is the code's last bit). Values above the
    table's end go to its last entry (saturation)."""
    a = np.asarray(a, dtype=np.float64)
    n = table.shape[0]
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    dlo, dhi = np.abs(a - table[lo]), np.abs(table[hi] - a)
    return np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))


def e4m3_encode(x):
    """float64 -> OCP E4M3 bytes: the nearest finite E4M3 value, ties to the
    even code, saturating at +-448; a value that rounds to zero is +0."""
    x = np.asarray(x, dtype=np.float64)
    mags = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))    # codes 0..0x7E, ascending
    c = _nearest_code(np.abs(x), mags).astype(np.uint8)
    return np.where((x < 0) & (c != 0), c | 0x80, c).astype(np.uint8)


def e2m1_encode(x):
    """float64 -> 4-bit E2M1 codes: the nearest of 0, .5, 1, 1.5, 2, 3, 4, 6,
    ties to the even code, saturating at +-6; a value that rounds to zero is
    +0."""
    x = np.asarray(x, dtype=np.float64)
    mags = e2m1_to_f64(np.arange(8))
    c = _nearest_code(np.abs(x), mags).astype(np.int64)
    return np.where((x < 0) & (c != 0), c | 8, c)


def nvfp4_quantize_group(y):
    """16 values (already divided by the tensor scale) -> (E4M3 scale code,
    16 E2M1 codes): scale = E4M3(max|y| / 6), codes = E2M1(y / scale),
    all +0 when the scale is 0 (the NVFP4 storage the decode reads: one E4M3
    scale per 16 elements, the largest magnitude mapped to E2M1's 6)."""
    y = np.asarray(y, dtype=np.float64)
    sc = int(e4m3_encode(np.max(np.abs(y)) / 6.0))
    s = float(e4m3_to_f64(np.uint8(sc)))
    codes = e2m1_encode(y / s) if s > 0 else np.zeros(y.shape[0], dtype=np.int64)
    return sc, codes


def kv_insert(w, new_k, new_v, new_idx_k):
    """Write the q_len new tokens into copies of the caches of workload `w`
    and return them as a dict (k_data, k_scale, v_data, v_scale, idx_k,
    idx_k_scale). Token t of sequence b lands at position
    pos = ctx_lens[b] - q_len + t, page block_table[b][pos // 128], slot
    pos % 128; tokens outside [0, max_blocks*128) or on an absent page are
    skipped. NVFP4: per 16-group of y = x / tensor_scale as in
    nvfp4_quantize_group; FP8 indexer keys: s = fp32(max|k| / 448) (1 when
    the max is 0), byte = E4M3(k / s); NVFP4 indexer keys as NVFP4 K with
    the indexer's tensor scale. bf16 caches keep the bits."""
    prm = w.params
    B, Tq, G = int(prm["num_seqs"]), int(prm["q_len"]), int(prm["num_kv_heads"])
    maxb, P = int(prm["max_blocks_per_seq"]), int(prm["num_pages"])
    nvfp4, idx_fmt = int(prm["kv_dtype"]) == 1, int(prm["idx_dtype"])
    out = dict(k_data=w.k_data.copy(), v_data=w.v_data.copy(), idx_k=w.idx_k.copy(),
               k_scale=None if w.k_scale is None else w.k_scale.copy(),
               v_scale=None if w.v_scale is None else w.v_scale.copy(),
               idx_k_scale=None if w.idx_k_scale is None else w.idx_k_scale.copy())
    for b in range(B):
        for t in range(Tq):
            pos = int(w.ctx_lens[b]) - Tq + t
            if pos < 0 or pos >= maxb * BLOCK:
                continue
            page = int(w.block_table[b, pos // BLOCK])
            if not _page_ok(page, P):
                continue
            slot = pos % BLOCK
            for g in range(G):
                if not nvfp4:
                    out["k_data"][page, g, slot, :] = new_k[b, t, g]
                    out["v_data"][page, g, :, slot] = new_v[b, t, g]
                    continue
                yk = bf16_to_f64(new_k[b, t, g]) / float(w.k_tensor_scale)
                yv = bf16_to_f64(new_v[b, t, g]) / float(w.v_tensor_scale)
                for c in range(HEAD_DIM // 16):
                    sc, codes = nvfp4_quantize_group(yk[16 * c:16 * c + 16])
                    out["k_scale"][page, g, slot, c] = sc
                    out["k_data"][page, g, slot, 8 * c:8 * c + 8] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
                    sc, codes = nvfp4_quantize_group(yv[16 * c:16 * c + 16])
                    out["v_scale"][page, g, c, slot] = sc
                    for i in range(16):
                        d = 16 * c + i
                        byte = int(out["v_data"][page, g, d, slot // 2])
                        if slot % 2 == 0:
                            byte = (byte & 0xF0) | int(codes[i])
                        else:
                            byte = (byte & 0x0F) | (int(codes[i]) << 4)
                        out["v_data"][page, g, d, slot // 2] = byte
            if idx_fmt == 0:
                out["idx_k"][page, slot, :] = new_idx_k[b, t]
                continue
            k = bf16_to_f64(new_idx_k[b, t])
            if idx_fmt == 2:
                y = k / float(getattr(w, "idx_k_tensor_scale", 1.0))
                for c in range(IDX_DIM // 16):
                    sc, codes = nvfp4_quantize_group(y[16 * c:16 * c + 16])
                    out["idx_k_scale"][page, slot, c] = sc
                    out["idx_k"][page, slot, 8 * c:8 * c + 8] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
                continue
            amax = np.float32(np.max(np.abs(k)))
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            out["idx_k"][page, slot, :] = e4m3_encode(k / float(s))
            out["idx_k_scale"][page, slot] = s
    return out


# ------------------------------------------------------------ whole decode

def decode_sequence(w, b, tokens=None, want_scores=False):
    """Run steps 1-6 for the query tokens of sequence b. Returns a list of
    per-token dicts: p, scores (optional), pooled, sel, boundary, out, lse,
    n_keys (keys attended per KV head)."""
    prm = w.params
    Tq, maxb = int(prm["q_len"]), int(prm["max_blocks_per_seq"])
    top_k, keep_last = int(prm["top_k"]), bool(prm["keep_last"])
    Lc = min(int(w.ctx_lens[b]), maxb * BLOCK)
    keys, present = seq_indexer_keys(w, b, max(Lc, 0))
    qi = bf16_to_f64(w.idx_q[b])                            # [Tq][Hi][64]
    wt = w.idx_w[b].astype(np.float64)                      # [Tq][Hi]
    res = []
    for t in (range(Tq) if tokens is None else tokens):
        p_t = query_position(w.ctx_lens[b], Tq, t, maxb)
        r = {"p": p_t}
        if p_t < 0:
            r.update(scores=np.zeros(0), pooled=np.zeros(0), sel=np.zeros(0, dtype=np.int64),
                     boundary=(None, None), out=np.zeros((int(prm["num_q_heads"]), HEAD_DIM)),
                     lse=np.full(int(prm["num_q_heads"]), -np.inf), n_keys=0)
            res.append(r)
            continue
        s = indexer_scores(qi[t], wt[t], keys[:p_t + 1])
        s = np.where(present[:p_t + 1], s, -np.inf)
        P = pool_blocks(s, present[:p_t + 1])
        S = select_blocks(P, top_k, keep_last)
        o, lse = attend_token(w, b, t, S, p_t)
        n_keys = sum(max(0, min(BLOCK, p_t + 1 - int(i) * BLOCK)) for i in S)
        r.update(pooled=P, sel=S, boundary=boundary_values(P, top_k, keep_last), out=o, lse=lse,
                 n_keys=n_keys)
        if want_scores:
            r["scores"] = s
        res.append(r)
    return res


def decode_layer(w, want_scores=False):
    """Whole decode step: dict of arrays shaped like the library's outputs
    (out/lse float64, pooled float64 padded with -inf, sel int64 padded with
    -1, nsel) plus per-token boundary values."""
    prm = w.params
    B, Tq, Hq = int(prm["num_seqs"]), int(prm["q_len"]), int(prm["num_q_heads"])
    maxb, top_k = int(prm["max_blocks_per_seq"]), int(prm["top_k"])
    out = np.zeros((B, Tq, Hq, HEAD_DIM))
    lse = np.full((B, Tq, Hq), -np.inf)
    pooled = np.full((B, Tq, maxb), -np.inf)
    sel = np.full((B, Tq, top_k), -1, dtype=np.int64)
    nsel = np.zeros((B, Tq), dtype=np.int64)
    scores = np.full((B, Tq, maxb * BLOCK), -np.inf) if want_scores else None
    boundary = {}
    for b in range(B):
        for t, r in enumerate(decode_sequence(w, b, want_scores=want_scores)):
            out[b, t], lse[b, t] = r["out"], r["lse"]
            n = r["pooled"].shape[0]
            pooled[b, t, :n] = r["pooled"]
            sel[b, t, :len(r["sel"])] = r["sel"]
            nsel[b, t] = len(r["sel"])
            boundary[(b, t)] = r["boundary"]
            if want_scores and r["p"] >= 0:
                scores[b, t, :r["p"] + 1] = r["scores"]
    return dict(out=out, lse=lse, pooled=pooled, sel=sel, nsel=nsel, boundary=boundary,
                scores=scores)
