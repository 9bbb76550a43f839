"""GPU parity of msa_decode_layer_single (one launch) through the C ABI:
against the oracle on small ragged batches, every split of the attention
items, edge contexts, scales and selection variants (tolerances of
tests/gpu_util.py; the full-size workloads are in test_gpu_configs.py), and
against msa_decode_layer, whose kernels run the same device code: the same
selection everywhere, and the same output bits where both run the attention
with 4 waves and one workgroup per item (batches with at least two items
per compute unit). Also its bounded waits, the give-up query and graph
capture."""
import contextlib
import gc

import numpy as np
import pytest
import torch

import block_sparse_attention_kv_amd as msa
from tests import gpu_util as G
from workloads import make_workload, make_config, small_cases, KV_NVFP4, KV_BF16, IDX_FP8, IDX_NVFP4, IDX_BF16

pytestmark = pytest.mark.gpu


def _same_as_two_kernel(w, run=None):
    """The selection always matches msa_decode_layer's bit for bit (same
    pooled scores). The output and lse match bit for bit when the two-kernel
    attention also runs 4 waves per item, i.e. with at least two items per
    compute unit; for fewer items it spreads an item over 8 waves, whose
    partial softmax states merge in another order (the oracle comparison
    covers those cases)."""
    run = run or G.Run(w)
    a = run.layer()
    b = run.layer(single=True)
    assert np.array_equal(a["sel"], b["sel"]), (w.name, "selection differs from msa_decode_layer")
    prm = w.params
    items = prm["num_seqs"] * prm["q_len"] * prm["num_kv_heads"]
    if items >= 2 * torch.cuda.get_device_properties(0).multi_processor_count:
        assert np.array_equal(a["out_bits"], b["out_bits"]), (w.name, "out differs from msa_decode_layer")
        assert np.array_equal(a["lse"].view(np.uint64), b["lse"].view(np.uint64)), (w.name, "lse differs")
    else:
        print("%s: %d items, out max |single - two-kernel| %.2e" % (w.name, items,
                                                                   np.abs(a["out"] - b["out"]).max()))
    return run


CASES = {
    # ragged contexts: empty visible range for early tokens (ctx 2 < q_len),
    # a single partial block, a block boundary, long ones
    "fp8_q4_ragged": dict(ctx=[2, 100, 129, 3000, 40000, 640], q_len=4, hq=16, hkv=2, hi=8, idx=IDX_FP8),
    "nvfp4_q4_ragged": dict(ctx=[5, 300, 129, 9000, 257], q_len=4, hq=16, hkv=2, hi=8, idx=IDX_NVFP4),
    "fp8_q1_hi4": dict(ctx=[7000, 1, 128, 130], q_len=1, hq=8, hkv=1, hi=4, idx=IDX_FP8),
    "nvfp4_q2_hi4": dict(ctx=[2049, 777], q_len=2, hq=32, hkv=4, hi=4, idx=IDX_NVFP4),
    "fp8_q3_topk5_nokeep": dict(ctx=[5000, 900, 1300], q_len=3, hq=16, hkv=2, hi=8, idx=IDX_FP8, top_k=5,
                                keep_last=0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_single_matches_oracle_and_two_kernel(name):
    c = CASES[name]
    w = make_workload("single_" + name, 61, c["ctx"], c["q_len"], c["hq"], c["hkv"], c["hi"], KV_NVFP4, c["idx"],
                      table="pool", pool_factor=1.2, n_planted=3, top_k=c.get("top_k", 16),
                      keep_last=c.get("keep_last", 1))
    run = _same_as_two_kernel(w)
    ties, mx, mean = G.layer_parity(w, run=run, single=True)
    print("%s: ties %d, out max-abs %.2e mean-abs %.2e" % (name, ties, mx, mean))


def test_single_more_items_than_grid():
    # 160 x 4 x 4 = 2560 items: every workgroup loops over several items
    rng = np.random.default_rng(62)
    ctx = rng.integers(1, 3000, size=160)
    w = make_workload("single_many_items", 63, ctx, 4, 16, 4, 8, KV_NVFP4, IDX_FP8, table="permute")
    run = _same_as_two_kernel(w)
    ties, mx, mean = G.layer_parity(w, run=run, seqs=[0, 1, 77, 159], single=True)
    print("many items: ties %d, out max-abs %.2e mean-abs %.2e" % (ties, mx, mean))


def test_single_more_than_four_selector_ranges():
    # 4,098 to 8,192 blocks per context: 5 to 8 selector records per token in
    # the split shape, so the attention workgroups hold the candidates in two
    # slots per lane; the winners lie in every range
    w = make_workload("single_8rec", 66, [8192 * 128, 6000 * 128 - 37, 4097 * 128 + 5], 1, 16, 1, 4, KV_NVFP4,
                      IDX_FP8, table="permute", n_planted=6)
    run = _same_as_two_kernel(w)
    ties, mx, mean = G.layer_parity(w, run=run, single=True)
    print("8 records: ties %d, out max-abs %.2e mean-abs %.2e" % (ties, mx, mean))


def test_single_absent_pages():
    w = make_workload("single_absent", 64, [3000, 1200], 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    w.block_table[0, 5] = -1
    w.block_table[1, 3] = w.params["num_pages"] + 2
    _same_as_two_kernel(w)


def test_single_repeat_reuses_workspace():
    w = make_workload("single_repeat", 65, [4000, 300, 2500], 4, 16, 2, 8, KV_NVFP4, IDX_NVFP4, table="permute")
    run = G.Run(w)
    first = run.layer(single=True)
    for _ in range(3):
        again = run.layer(single=True)
        assert np.array_equal(first["out_bits"], again["out_bits"])
        assert np.array_equal(first["sel"], again["sel"])


def test_single_workspace_holds_no_stale_scores():
    # Two different batches of one shape alternate through one workspace.
    # The pooled scores a call reads must be its own, not the words the
    # other batch's call left there (they carry another call's tag), so
    # every result equals that batch's run on a fresh zero-filled workspace
    # bit for bit.
    lens = [5000, 2100, 3300, 700]
    wa = make_workload("ws_a", 71, lens, 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    wb = make_workload("ws_b", 72, lens, 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    assert wa.params == wb.params
    ra, rb = G.Run(wa), G.Run(wb)
    prm = wa.params
    B, Tq, Hq, K = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["top_k"]

    def call(r, ws):
        out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
        sel = torch.empty((B, Tq, K), dtype=torch.int32, device="cuda")
        msa.msa_decode_layer_single(r.params, r.cache, r.q, r.idx_q, r.idx_w, out, ws, lse=lse, sel_out=sel)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()

    want = {}
    for key, r in (("a", ra), ("b", rb)):
        fresh = msa.alloc_workspace(r.params, "cuda").zero_()
        want[key] = call(r, fresh)
    assert not np.array_equal(want["a"][2], want["b"][2])  # the batches select differently
    ws = msa.alloc_workspace(ra.params, "cuda")
    for key, r in (("a", ra), ("b", rb), ("a", ra), ("b", rb), ("b", rb)):
        got = call(r, ws)
        for g, x in zip(got, want[key]):
            assert np.array_equal(g.view(np.uint8), x.view(np.uint8)), key
    # the two-kernel layer on the same workspace between single launches
    # leaves its own (fp32) pooled scores, which the single launch must not
    # read: its results stay those of a fresh workspace
    for key, r in (("a", ra), ("b", rb), ("a", ra)):
        out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
        msa.msa_decode_layer(r.params, r.cache, r.q, r.idx_q, r.idx_w, out, ws)
        other = rb if r is ra else ra
        got = call(other, ws)
        okey = "b" if key == "a" else "a"
        for g, x in zip(got, want[okey]):
            assert np.array_equal(g.view(np.uint8), x.view(np.uint8)), okey


def test_single_rejects_unsupported():
    w = make_workload("single_bf16", 66, [300], 4, 16, 2, 4, KV_BF16, IDX_BF16, table="permute")
    run = G.Run(w)
    with pytest.raises(msa.MSAError):
        run.layer(single=True)
    w = make_workload("single_q5", 67, [300], 5, 16, 2, 4, KV_NVFP4, IDX_FP8, table="permute")
    run = G.Run(w)
    with pytest.raises(msa.MSAError):
        run.layer(single=True)


def test_single_traced_matches_plain():
    # the traced entry records the kernel's start and end into two events and
    # computes the same result
    import ctypes
    w = make_workload("single_traced", 68, [3000, 700], 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    run = G.Run(w)
    want = run.layer(single=True)
    prm = w.params
    B, Tq, Hq, K = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["top_k"]
    out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
    sel = torch.empty((B, Tq, K), dtype=torch.int32, device="cuda")
    ws = msa.alloc_workspace(run.params, "cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    arr = (ctypes.c_void_p * 2)(*[e.cuda_event for e in ev])
    c = run.cache.c()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = msa.load().msa_decode_layer_single_traced(
        ctypes.byref(run.params), ctypes.byref(c), vp(run.q), vp(run.idx_q), vp(run.idx_w), vp(out), None, vp(sel),
        vp(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), arr)
    assert st == 0
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    assert np.array_equal(out.cpu().numpy(), want["out_bits"])
    assert np.array_equal(sel.cpu().numpy(), want["sel"])


@pytest.mark.parametrize("shape,ctx,nseq", [(0, 20000, 24), (1, 20000, 24), (0, 140000, 6)])
def test_single_bounded_wait_gives_up_cleanly(shape, ctx, nseq):
    # With a poll limit of 1 a workgroup that finds the data it waits for
    # unpublished at the first poll gives up at once: the kernel still ends,
    # every (token, KV head) item is either the normal result or marked
    # invalid (NaN output and lse; the token's selection either the normal
    # one or all -1 when the workgroup writing it gave up), the give-up
    # query counts the workgroups
    # that stopped, and the default limit restores the normal result (and a
    # zero count) on the next call.
    # shapes: split items selecting themselves (contexts of at most 1,024
    # blocks), fused, and split items reading selector records (1,094 blocks)
    w = make_workload("single_spin", 69, [ctx] * nseq, 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    run = G.Run(w)
    prm = w.params
    B, Tq, Hkv, grp = prm["num_seqs"], prm["q_len"], prm["num_kv_heads"], prm["num_q_heads"] // prm["num_kv_heads"]
    Hq, K = prm["num_q_heads"], prm["top_k"]
    ws = msa.alloc_workspace(run.params, "cuda")

    def call():
        out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
        sel = torch.empty((B, Tq, K), dtype=torch.int32, device="cuda")
        msa.msa_decode_layer_single(run.params, run.cache, run.q, run.idx_q, run.idx_w, out, ws, lse=lse, sel_out=sel)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()

    msa.msa_debug_layer_splits(shape)  # 0: the automatic shape (split, for these few items); 1: fused
    try:
        want = call()
        assert msa.msa_decode_layer_gave_up(run.params, ws) == 0
        try:
            msa.msa_debug_layer_spin_limit(1)
            got = call()
        finally:
            msa.msa_debug_layer_spin_limit(0)
    finally:
        msa.msa_debug_layer_splits(0)
    n_gave_up = msa.msa_decode_layer_gave_up(run.params, ws)
    invalid = 0
    for b in range(B):
        for t in range(Tq):
            sel_ok = np.array_equal(got[2][b, t], want[2][b, t])
            assert sel_ok or np.all(got[2][b, t] == -1), (b, t)
            for g in range(Hkv):
                heads = slice(g * grp, (g + 1) * grp)
                o = got[0][b, t, heads]
                if np.all(o.view(np.uint16) == 0x7FC0):
                    assert np.all(np.isnan(got[1][b, t, heads]))
                    invalid += 1
                else:
                    assert np.array_equal(o, want[0][b, t, heads]), (b, t, g)
                    assert np.array_equal(got[1][b, t, heads].view(np.uint32),
                                          want[1][b, t, heads].view(np.uint32)), (b, t, g)
    print("with a poll limit of 1: %d of %d items invalid, %d workgroups gave up" % (invalid, B * Tq * Hkv, n_gave_up))
    assert (invalid > 0) == (n_gave_up > 0)
    msa.msa_debug_layer_splits(shape)
    try:
        again = call()
    finally:
        msa.msa_debug_layer_splits(0)
    assert msa.msa_decode_layer_gave_up(run.params, ws) == 0
    for g_, w_ in zip(again, want):
        assert np.array_equal(g_.view(np.uint8), w_.view(np.uint8))


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_single_forced_splits(splits):
    # every split count on batches whose automatic choice differs: against
    # the oracle, and deterministic over repeated calls
    w = make_workload("single_split%d" % splits, 74, [5000, 129, 2100, 300, 40000], 4, 16, 2, 8, KV_NVFP4, IDX_FP8,
                      table="pool", pool_factor=1.2, n_planted=3)
    run = G.Run(w)
    try:
        msa.msa_debug_layer_splits(splits)
        first = run.layer(single=True)
        again = run.layer(single=True)
        ties, mx, mean = G.layer_parity(w, run=run, single=True)
    finally:
        msa.msa_debug_layer_splits(0)
    assert np.array_equal(first["out_bits"], again["out_bits"])
    assert np.array_equal(first["lse"].view(np.uint64), again["lse"].view(np.uint64))
    assert np.array_equal(first["sel"], again["sel"])
    print("splits %d: ties %d, out max-abs %.2e mean-abs %.2e" % (splits, ties, mx, mean))


def test_single_split_counts_agree_on_selection():
    # the selection does not depend on how the attention is split; the
    # outputs agree to rounding
    w = make_workload("single_split_sel", 75, [9000, 3000], 4, 32, 4, 8, KV_NVFP4, IDX_NVFP4, table="permute")
    run = G.Run(w)
    res = {}
    try:
        for s in (1, 2, 4):
            msa.msa_debug_layer_splits(s)
            res[s] = run.layer(single=True)
    finally:
        msa.msa_debug_layer_splits(0)
    for s in (2, 4):
        assert np.array_equal(res[s]["sel"], res[1]["sel"])
        assert np.max(np.abs(res[s]["out"] - res[1]["out"])) <= 2 * G.OUT_MAX_ABS


@contextlib.contextmanager
def _no_gc_capture():
    """Objects left by earlier tests (tensors, graphs) must not be destroyed
    while a stream is being captured: their destructors make HIP calls that a
    capture does not permit, and HIP aborts the process. Collect them first
    and keep the collector off during the capture."""
    gc.collect()
    torch.cuda.synchronize()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def test_single_rejects_graph_capture():
    # the call's epoch is drawn on the host: a captured launch would replay
    # it, so the single launch refuses to be captured (before enqueueing)
    w = make_workload("single_capture", 76, [3000, 700], 4, 16, 2, 8, KV_NVFP4, IDX_FP8, table="permute")
    run = G.Run(w)
    prm = w.params
    B, Tq, Hq = prm["num_seqs"], prm["q_len"], prm["num_q_heads"]
    out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
    ws = msa.alloc_workspace(run.params, "cuda")
    graph = torch.cuda.CUDAGraph()
    err = None
    with _no_gc_capture():
        try:
            with torch.cuda.graph(graph):
                try:
                    msa.msa_decode_layer_single(run.params, run.cache, run.q, run.idx_q, run.idx_w, out, ws)
                except msa.MSAError as e:
                    err = e
        except RuntimeError:
            pass  # an empty capture may be refused by torch; the library's answer is what is checked
    torch.cuda.synchronize()
    # the refused graph is released here, outside any capture: its destructor
    # makes HIP calls that a capture in progress would not permit
    del graph
    gc.collect()
    assert err is not None and err.status == msa.MSA_ERR_UNSUPPORTED, err
    # and the next uncaptured call works
    G.layer_parity(w, run=run, single=True)


def test_two_kernel_layer_graph_replays():
    # msa_decode_layer needs no per-call tag when its stream is captured (the
    # split bf16 attention falls back to one workgroup per item): a captured
    # step replays correctly, with eager work and synchronisations between
    # the replays, and every replay matches the oracle
    w = small_cases()[1]                              # bf16 cache: split attention when eager
    run = G.Run(w)
    prm = w.params
    B, Tq, Hq, K = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["top_k"]
    out = torch.zeros((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
    lse = torch.zeros((B, Tq, Hq), dtype=torch.float32, device="cuda")
    sel = torch.zeros((B, Tq, K), dtype=torch.int32, device="cuda")
    ws = msa.alloc_workspace(run.params, "cuda")
    msa.msa_decode_layer(run.params, run.cache, run.q, run.idx_q, run.idx_w, out, ws, lse=lse, sel_out=sel)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with _no_gc_capture():
        with torch.cuda.graph(graph):
            msa.msa_decode_layer(run.params, run.cache, run.q, run.idx_q, run.idx_w, out, ws, lse=lse, sel_out=sel)
    torch.cuda.synchronize()
    refs = G.oracle_refs(w)
    for i in range(3):
        out.zero_()
        lse.zero_()
        sel.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        res = dict(out=G.bf16_to_np(out), out_bits=out.cpu().numpy(), lse=lse.cpu().numpy().astype(np.float64),
                   sel=sel.cpu().numpy())
        G.compare_layer(w, res, refs, label="%s replay %d" % (w.name, i))


def test_single_spin_limit_rejects_negative():
    with pytest.raises(msa.MSAError):
        msa.msa_debug_layer_spin_limit(-1)


def test_single_edge_contexts():
    # an empty sequence, 1 token, partial blocks, exactly 16 blocks, 16 blocks
    # + 1 token, ctx < q_len, and a context longer than the block table
    # (clamped to max_blocks * 128)
    w = make_workload("single_edges", 71, [0, 1, 127, 128, 129, 2047, 2048, 2049, 2176, 2, 3000], 2, 16, 2, 8,
                      KV_NVFP4, IDX_FP8, table="permute")
    w.ctx_lens[-1] = w.params["max_blocks_per_seq"] * 128 + 700
    run = _same_as_two_kernel(w)
    ties, mx, mean = G.layer_parity(w, run=run, single=True)
    print("edges: ties %d, out max-abs %.2e mean-abs %.2e" % (ties, mx, mean))


@pytest.mark.parametrize("k_ts,v_ts,sm", [(0.75, 1.5, 0.05), (-0.5, 1.0, 0.0)])
def test_single_tensor_and_softmax_scales(k_ts, v_ts, sm):
    w = make_workload("single_scales", 72, [1000, 4000, 300], 2, 16, 2, 8, KV_NVFP4, IDX_NVFP4, table="permute",
                      k_tensor_scale=k_ts, v_tensor_scale=v_ts, softmax_scale=sm)
    run = _same_as_two_kernel(w)
    G.layer_parity(w, run=run, single=True)


@pytest.mark.parametrize("k,keep", [(4, 1), (16, 0), (1, 1)])
def test_single_top_k_and_keep_last(k, keep):
    w = make_workload("single_k%d_keep%d" % (k, keep), 73, [3000, 700], 1, 8, 1, 4, KV_NVFP4, IDX_FP8,
                      table="permute", top_k=k, keep_last=keep, n_planted=2)
    run = _same_as_two_kernel(w)
    G.layer_parity(w, run=run, single=True)
