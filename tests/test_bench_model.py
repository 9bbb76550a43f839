"""CPU pins of bench.py's byte model (the algorithmic bytes every reported
rate and roofline fraction divides by): the closed forms of the hot-path
scope table for the 32K and 512K decode workloads, and the ratio of MSA's
bytes to dense attention's that the ainewsbites page gives as about 12.5%
(section "A model built for efficient inference")."""
import numpy as np

import bench


def _params(B, Tq, Hq, G, Hi, L, idx_dtype=1, kv_dtype=1):
    return dict(num_seqs=B, q_len=Tq, num_q_heads=Hq, num_kv_heads=G, idx_heads=Hi,
                max_blocks_per_seq=(L + 127) // 128, idx_dtype=idx_dtype, kv_dtype=kv_dtype, top_k=16)


def _sel(B, Tq, nblk, per_token_distinct=False):
    """Selections of 16 blocks per token (ascending), the last block kept."""
    sel = np.full((B, Tq, 16), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            base = 16 * t if per_token_distinct else 0
            sel[b, t, :15] = np.arange(base, base + 15)
            sel[b, t, 15] = nblk - 1
    return sel


def test_nvfp4_32k_bytes():
    # 8 seqs x 32,768 tokens, 32/2 heads, 4 indexer heads, FP8 indexer keys
    p = _params(8, 1, 32, 2, 4, 32768)
    L = np.full(8, 32768)
    sel = _sel(8, 1, 256)
    t = bench.step_byte_terms(p, L, bench.union_blocks(sel))
    assert t["idx_keys"] == 8 * 32768 * 68 == 17_825_792
    assert t["kv"] == 8 * 16 * 2 * 128 * 144 == 4_718_592
    assert sum(t.values()) == 22_687_904
    assert bench.indexer_bytes(p, L) + bench.attention_bytes(p, L, sel) == 22_687_904


def test_long_512k_bytes():
    # 4 seqs x 524,288 tokens, 64/4 heads, 4 indexer heads
    p = _params(4, 1, 64, 4, 4, 524288)
    L = np.full(4, 524288)
    sel = _sel(4, 1, 4096)
    t = bench.step_byte_terms(p, L, bench.union_blocks(sel))
    assert t["idx_keys"] == 142_606_336 and t["kv"] == 4_718_592
    assert sum(t.values()) == 147_523_664
    assert bench.indexer_bytes(p, L) + bench.attention_bytes(p, L, sel) == 147_523_664


def test_union_counts_distinct_blocks_per_sequence():
    # 4 query tokens selecting disjoint blocks but the same last block:
    # 4 x 15 + 1 = 61 distinct blocks per sequence
    sel = _sel(2, 4, 1024, per_token_distinct=True)
    assert bench.union_blocks(sel) == 2 * 61
    sel[0, 1] = sel[0, 0]                      # token 1 repeats token 0
    assert bench.union_blocks(sel) == 46 + 61
    sel[1, 0, 3:] = -1                         # padding is not a block
    assert bench.union_blocks(sel) == 46 + 61 - 13 + 1


def test_ratio_to_dense_attention():
    # (68 L + 16 x 128 x 576) / (576 L) per sequence with 4 KV heads: 13.4% at
    # 128K and 12.2% at 512K, the pages' "about 12.5%"
    for L, want in ((131072, 0.1337), (524288, 0.1220)):
        p = _params(1, 1, 64, 4, 8, L)
        lens = np.array([L])
        t = bench.step_byte_terms(p, lens, 16)
        ratio = (t["idx_keys"] + t["kv"]) / bench.dense_kv_bytes(p, lens)
        assert abs(ratio - (68 * L + 2048 * 576) / (576 * L)) < 1e-15
        assert abs(ratio - want) < 5e-4, ratio


def test_clamped_context_and_bf16_terms():
    # contexts are clamped to max_blocks_per_seq * 128 like the kernels do;
    # bf16 K/V cost 512 B per token and KV head, bf16 indexer keys 128 B
    p = _params(1, 1, 8, 1, 4, 4096, idx_dtype=0, kv_dtype=0)
    t = bench.step_byte_terms(p, np.array([10_000]), 16)
    assert t["idx_keys"] == 4096 * 128 and t["table"] == 32 * 4
    assert t["kv"] == 16 * 128 * 512 == 1_048_576
    assert sum(t.values()) == 1_577_620          # the tiny bf16 workload's total
