"""Seeded synthetic MSA decode workloads in the device layout of include/msa.h.

A workload is the full set of buffers one MSA decode step reads (queries,
indexer queries and head weights, the paged NVFP4 or bf16 K/V cache, the FP8
or bf16 indexer-key cache, block table, context lengths) plus the scalar
parameters. Every value is a pure function of (seed, shape): bulk draws come
from the counter-based C generator (workloads/csrc/msagen.c), structural
choices (page permutation, planted blocks, ragged lengths, outlier channels)
from numpy's PCG64.

The shapes follow the five decode configurations this library is measured
on: a tiny bf16 case at 4K context, an NVFP4 case at 32K, the speculative
verify case (4 query tokens) at 128K, a 512K single-sequence-share case with
near-tied pooled scores, and a ragged serving batch with log-uniform lengths.
There is no dataset on the pages for this path; the draws stand in for the
agentic traces and benchmark the pages measure on.

This module holds no part of the decode arithmetic: it only draws values and
quantises them into stored codes.
"""
import ctypes
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import _native

KV_BF16, KV_NVFP4 = 0, 1
IDX_BF16, IDX_FP8, IDX_NVFP4 = 0, 1, 2
BLOCK = 128
HEAD_DIM = 128
IDX_DIM = 64

TAG_Q, TAG_IDXQ, TAG_IDXW, TAG_K, TAG_V, TAG_IDXK = 1, 2, 3, 4, 5, 6
TAG_OUTLIER, TAG_PLANT, TAG_TABLE, TAG_LENS = 7, 8, 9, 10
TAG_NEWK, TAG_NEWV, TAG_NEWIDX = 11, 12, 13


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


@dataclass
class Workload:
    """Host-side buffers of one decode step (numpy, device layout)."""
    name: str
    params: Dict[str, float]
    q: np.ndarray            # uint16 (bf16 bits) [B][Tq][Hq][128]
    idx_q: np.ndarray        # uint16 (bf16 bits) [B][Tq][Hi][64]
    idx_w: np.ndarray        # float32 [B][Tq][Hi]
    k_data: np.ndarray       # uint8 [P][G][128][64] or uint16 [P][G][128][128]
    k_scale: Optional[np.ndarray]
    v_data: np.ndarray       # uint8 [P][G][128][64] (dim-major) or uint16 [P][G][128][128]
    v_scale: Optional[np.ndarray]
    idx_k: np.ndarray        # uint8 [P][128][64] or uint16 [P][128][64]
    idx_k_scale: Optional[np.ndarray]  # FP8 float32 [P][128], NVFP4 uint8 [P][128][4]
    block_table: np.ndarray  # int32 [B][max_blocks]
    ctx_lens: np.ndarray     # int32 [B]
    k_tensor_scale: float = 1.0
    v_tensor_scale: float = 1.0
    idx_k_tensor_scale: float = 1.0
    planted: Dict[int, List[int]] = field(default_factory=dict)
    recipe: str = ""

    @property
    def B(self):
        return int(self.params["num_seqs"])

    @property
    def Tq(self):
        return int(self.params["q_len"])

    def nbytes(self):
        tot = 0
        for a in (self.q, self.idx_q, self.idx_w, self.k_data, self.k_scale, self.v_data,
                  self.v_scale, self.idx_k, self.idx_k_scale, self.block_table, self.ctx_lens):
            if a is not None:
                tot += a.nbytes
        return tot


def _rng(seed, tag):
    return np.random.Generator(np.random.PCG64([int(seed), int(tag)]))


def make_workload(name, seed, ctx_lens, q_len, num_q_heads, num_kv_heads, idx_heads,
                  kv_dtype=KV_NVFP4, idx_dtype=IDX_FP8, max_blocks=None, table="permute",
                  pool_factor=1.0, n_planted=0, idx_sigma=1.0, outlier_frac=0.0,
                  outlier_mul=8.0, top_k=16, keep_last=1, softmax_scale=0.0,
                  k_tensor_scale=1.0, v_tensor_scale=1.0, recipe=""):
    """Build a workload.

    ctx_lens: per-sequence context length L_b (includes the q_len new tokens).
    table: "identity" (pages in order, one sequence after the other),
           "permute" (a random permutation of all pages), or "pool" (a shared
           pool of ceil(pool_factor * total blocks) pages, randomly permuted
           and handed out round-robin across sequences, leaving holes).
    n_planted: non-last blocks per sequence whose indexer keys get
           0.5 * sum_h qi[b, 0, h, :] added, so that they score high.
    outlier_frac: fraction of the 128 channels of each KV head (for K and for V
           separately, fixed across tokens) multiplied by outlier_mul.
    """
    lib = _native.lib()
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    B = int(ctx.size)
    Tq, Hq, G, Hi = int(q_len), int(num_q_heads), int(num_kv_heads), int(idx_heads)
    nblk = (ctx.astype(np.int64) + BLOCK - 1) // BLOCK
    if max_blocks is None:
        max_blocks = int(nblk.max()) if B else 1
    total_blocks = int(nblk.sum())

    # ---- block table
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    if table == "identity":
        num_pages = total_blocks
        nxt = 0
        for b in range(B):
            bt[b, :nblk[b]] = np.arange(nxt, nxt + nblk[b], dtype=np.int32)
            nxt += int(nblk[b])
    elif table == "permute":
        num_pages = total_blocks
        perm = _rng(seed, TAG_TABLE).permutation(num_pages).astype(np.int32)
        nxt = 0
        for b in range(B):
            bt[b, :nblk[b]] = perm[nxt:nxt + nblk[b]]
            nxt += int(nblk[b])
    elif table == "pool":
        num_pages = int(math.ceil(pool_factor * total_blocks))
        perm = _rng(seed, TAG_TABLE).permutation(num_pages).astype(np.int32)
        nxt = 0
        for blk in range(int(nblk.max()) if B else 0):
            for b in range(B):
                if blk < nblk[b]:
                    bt[b, blk] = perm[nxt]
                    nxt += 1
    else:
        raise ValueError(table)
    num_pages = max(num_pages, 1)

    # ---- queries (bf16 bits) and head weights
    key = lambda tag: lib.msagen_stream_key(int(seed), tag)
    q = np.empty((B, Tq, Hq, HEAD_DIM), dtype=np.uint16)
    lib.msagen_normal_bf16(key(TAG_Q), 0, q.size, 1.0, _ptr(q))
    idx_q = np.empty((B, Tq, Hi, IDX_DIM), dtype=np.uint16)
    lib.msagen_normal_bf16(key(TAG_IDXQ), 0, idx_q.size, 1.0, _ptr(idx_q))
    idx_w = np.empty((B, Tq, Hi), dtype=np.float32)
    lib.msagen_uniform_f32(key(TAG_IDXW), 0, idx_w.size, _ptr(idx_w))

    # ---- planted blocks: non-last for every query token of the sequence
    planted = {}
    plant = np.zeros((B, max_blocks), dtype=np.uint8)
    shift = np.zeros((B, IDX_DIM), dtype=np.float32)
    if n_planted > 0:
        r = _rng(seed, TAG_PLANT)
        qf = (idx_q.astype(np.uint32) << 16).view(np.float32)
        for b in range(B):
            first_new = (int(ctx[b]) - Tq) // BLOCK  # block of the earliest query token
            cand = max(first_new, 0)
            k = min(n_planted, cand)
            if k > 0:
                blks = np.sort(r.choice(cand, size=k, replace=False))
                planted[b] = [int(x) for x in blks]
                plant[b, blks] = 1
            shift[b] = 0.5 * qf[b, 0].astype(np.float64).sum(axis=0)

    # ---- outlier channels
    kmul = np.ones((G, HEAD_DIM), dtype=np.float32)
    vmul = np.ones((G, HEAD_DIM), dtype=np.float32)
    if outlier_frac > 0:
        n_out = int(math.ceil(outlier_frac * HEAD_DIM))
        r = _rng(seed, TAG_OUTLIER)
        for g in range(G):
            kmul[g, r.choice(HEAD_DIM, size=n_out, replace=False)] = outlier_mul
            vmul[g, r.choice(HEAD_DIM, size=n_out, replace=False)] = outlier_mul

    # ---- caches
    if kv_dtype == KV_NVFP4:
        k_data = np.zeros((num_pages, G, BLOCK, HEAD_DIM // 2), dtype=np.uint8)
        v_data = np.zeros((num_pages, G, HEAD_DIM, BLOCK // 2), dtype=np.uint8)
        k_scale = np.zeros((num_pages, G, BLOCK, HEAD_DIM // 16), dtype=np.uint8)
        v_scale = np.zeros((num_pages, G, HEAD_DIM // 16, BLOCK), dtype=np.uint8)
    else:
        k_data = np.zeros((num_pages, G, BLOCK, HEAD_DIM), dtype=np.uint16)
        v_data = np.zeros((num_pages, G, HEAD_DIM, BLOCK), dtype=np.uint16)
        k_scale = v_scale = None
    lib.msagen_kv_cache(key(TAG_K), key(TAG_V), B, _ptr(ctx), _ptr(bt), max_blocks, G,
                        _ptr(kmul), _ptr(vmul), 1 if kv_dtype == KV_NVFP4 else 0,
                        _ptr(k_data), _ptr(k_scale), _ptr(v_data), _ptr(v_scale))
    if idx_dtype == IDX_FP8:
        idx_k = np.zeros((num_pages, BLOCK, IDX_DIM), dtype=np.uint8)
        idx_k_scale = np.zeros((num_pages, BLOCK), dtype=np.float32)
    elif idx_dtype == IDX_NVFP4:
        idx_k = np.zeros((num_pages, BLOCK, IDX_DIM // 2), dtype=np.uint8)
        idx_k_scale = np.zeros((num_pages, BLOCK, IDX_DIM // 16), dtype=np.uint8)
    else:
        idx_k = np.zeros((num_pages, BLOCK, IDX_DIM), dtype=np.uint16)
        idx_k_scale = None
    lib.msagen_idx_cache(key(TAG_IDXK), B, _ptr(ctx), _ptr(bt), max_blocks, float(idx_sigma),
                         _ptr(plant), _ptr(shift), int(idx_dtype), _ptr(idx_k), _ptr(idx_k_scale))

    params = dict(num_seqs=B, q_len=Tq, num_q_heads=Hq, num_kv_heads=G, head_dim=HEAD_DIM,
                  idx_heads=Hi, idx_dim=IDX_DIM, block_size=BLOCK, top_k=int(top_k),
                  keep_last=int(keep_last), max_blocks_per_seq=int(max_blocks),
                  num_pages=int(num_pages), softmax_scale=float(softmax_scale),
                  kv_dtype=int(kv_dtype), idx_dtype=int(idx_dtype))
    return Workload(name=name, params=params, q=q, idx_q=idx_q, idx_w=idx_w, k_data=k_data,
                    k_scale=k_scale, v_data=v_data, v_scale=v_scale, idx_k=idx_k,
                    idx_k_scale=idx_k_scale, block_table=bt, ctx_lens=ctx,
                    k_tensor_scale=float(k_tensor_scale), v_tensor_scale=float(v_tensor_scale),
                    planted=planted, recipe=recipe)


def make_new_tokens(w, seed, sigma=1.0, extremes=False):
    """bf16 bits of the q_len new tokens of every sequence of workload `w`:
    K and V [B][q_len][num_kv_heads][128] and indexer keys [B][q_len][64],
    drawn N(0, sigma^2). With `extremes`, token 0 of sequence 0, KV head 0
    (and its indexer key) gets a saturating group (|x| = 3000), an all-zero
    group and a group of tiny values (1e-6 scale), so that the quantiser's
    saturation, zero-scale and subnormal-scale cases occur."""
    lib = _native.lib()
    B, Tq, G = w.B, w.Tq, int(w.params["num_kv_heads"])
    key = lambda tag: lib.msagen_stream_key(int(seed), tag)
    nk = np.empty((B, Tq, G, HEAD_DIM), dtype=np.uint16)
    nv = np.empty((B, Tq, G, HEAD_DIM), dtype=np.uint16)
    ni = np.empty((B, Tq, IDX_DIM), dtype=np.uint16)
    lib.msagen_normal_bf16(key(TAG_NEWK), 0, nk.size, float(sigma), _ptr(nk))
    lib.msagen_normal_bf16(key(TAG_NEWV), 0, nv.size, float(sigma), _ptr(nv))
    lib.msagen_normal_bf16(key(TAG_NEWIDX), 0, ni.size, float(sigma), _ptr(ni))
    if extremes:
        def bf16(x):
            return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        sgn = np.where(np.arange(16) % 2 == 0, 1.0, -1.0)
        for arr in (nk, nv):
            arr[0, 0, 0, 0:16] = bf16(3000.0 * sgn)
            arr[0, 0, 0, 16:32] = 0
            arr[0, 0, 0, 32:48] = bf16(1e-6 * sgn * np.arange(1, 17))
        ni[0, 0, 0:16] = 0
        if Tq > 1:
            ni[0, 1, :] = 0
    return nk, nv, ni


# ----------------------------------------------------------------- configs

CONFIG_NAMES = {
    1: "tiny bf16: 1 seq x 1 token, 4K ctx, 8/1 heads, 4 idx heads, bf16 KV + bf16 idx keys",
    2: "nvfp4: 8 seqs x 1 token, 32K ctx, 32/2 heads, 4 idx heads, NVFP4 KV + FP8 idx keys",
    3: "spec-verify: 32 seqs x 4 tokens, 128K ctx, 64/4 heads, 8 idx heads, NVFP4 KV + FP8 idx keys",
    4: "long: 4 seqs x 1 token, 512K ctx, 64/4 heads, 4 idx heads, NVFP4 KV + FP8 idx keys, near-tied",
    5: "ragged: 64 seqs x 1 token, log-U[1K,256K] ctx, 48/4 heads, 8 idx heads, NVFP4 KV + FP8 idx keys",
}


def ragged_lengths(seed, n, lo=1024, hi=262144):
    """floor(exp(U(ln lo, ln hi))) per sequence."""
    r = _rng(seed, TAG_LENS)
    return np.floor(np.exp(r.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int32)


def make_config(n, seed=None, idx_dtype=None):
    """One of the five decode configurations (seed defaults to 1000 + n).
    idx_dtype overrides the indexer-key format of configurations 2-5 (FP8)."""
    if seed is None:
        seed = 1000 + n
    idx = IDX_FP8 if idx_dtype is None else int(idx_dtype)
    if n == 1:
        return make_workload("cfg1", seed, [4096], 1, 8, 1, 4, KV_BF16, IDX_BF16,
                             table="identity", n_planted=3,
                             recipe="q,k,v,qi,ki ~ N(0,1) bf16; w ~ U(0,1); identity table; "
                                    "3 planted non-last blocks")
    if n == 2:
        return make_workload("cfg2", seed, [32768] * 8, 1, 32, 2, 4, KV_NVFP4, idx,
                             table="permute", n_planted=8,
                             recipe="K/V ~ N(0,1) -> NVFP4 (scale E4M3(amax/6), ts 1.0); "
                                    "ki ~ N(0,1) -> FP8 + per-token amax/448; permuted pages; "
                                    "8 planted blocks per sequence")
    if n == 3:
        return make_workload("cfg3", seed, [131072] * 32, 4, 64, 4, 8, KV_NVFP4, idx,
                             table="permute", outlier_frac=0.01, outlier_mul=8.0,
                             recipe="K/V ~ N(0,1), 2 channels per KV head x8 (K and V), NVFP4; "
                                    "ki ~ N(0,1) FP8; permuted pages; no planting; "
                                    "4 causal query tokens")
    if n == 4:
        return make_workload("cfg4", seed, [524288] * 4, 1, 64, 4, 4, KV_NVFP4, idx,
                             table="permute", n_planted=16, idx_sigma=0.01,
                             recipe="K/V ~ N(0,1) NVFP4; ki ~ N(0, 0.01^2) FP8 (near-tied "
                                    "pooled scores); 16 planted blocks; permuted pages")
    if n == 5:
        lens = ragged_lengths(seed, 64)
        return make_workload("cfg5", seed, lens, 1, 48, 4, 8, KV_NVFP4, idx,
                             max_blocks=2048, table="pool", pool_factor=1.25,
                             recipe="L ~ floor(exp(U(ln 1024, ln 262144))); K/V ~ N(0,1) "
                                    "NVFP4; ki ~ N(0,1) FP8; shared pool of 1.25x pages, "
                                    "permuted, round-robin across sequences (holes)")
    raise ValueError("config must be 1..5")


def small_cases():
    """Small workloads the oracle finishes in seconds that still span several
    blocks, ragged tails, partial last blocks, and both dtypes."""
    cases = []
    cases.append(make_workload("small_nvfp4_ragged", 11, [300, 2500, 4100, 129], 2, 16, 2, 3,
                               KV_NVFP4, IDX_FP8, table="permute", n_planted=2,
                               outlier_frac=0.02))
    cases.append(make_workload("small_bf16", 12, [2049, 2176, 1], 1, 8, 1, 4, KV_BF16, IDX_BF16,
                               table="identity", n_planted=1))
    cases.append(make_workload("small_tq4", 13, [3000, 5000], 4, 32, 4, 8, KV_NVFP4, IDX_FP8,
                               table="pool", pool_factor=1.3))
    cases.append(make_workload("small_g12", 14, [2047, 2048, 6000], 1, 48, 4, 8, KV_NVFP4,
                               IDX_FP8, table="permute", n_planted=3))
    return cases
