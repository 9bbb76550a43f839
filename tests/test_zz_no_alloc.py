"""GPU test of msa_decode_layer_single_static, the decode-layer entry point
that allocates nothing (its scratch is the library's static per-GPU array):
through the C ABI, two calls in a row -- a few-item batch over long
contexts (selectors and items split over several workgroups) and then a
smaller batch -- each bit for bit equal to msa_decode_layer_single on a
workspace, and the second also against the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_kv_amd as msa
from tests import gpu_util as G
from workloads import make_workload, KV_NVFP4, IDX_FP8, IDX_NVFP4

pytestmark = pytest.mark.gpu


def _call_static(run):
    prm = run.w.params
    B, Tq, Hq, K = prm["num_seqs"], prm["q_len"], prm["num_q_heads"], prm["top_k"]
    out = torch.empty((B, Tq, Hq, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Tq, K), dtype=torch.int32, device="cuda")
    msa.msa_decode_layer_single_static(run.params, run.cache, run.q, run.idx_q, run.idx_w, out, lse=lse, sel_out=sel)
    torch.cuda.synchronize()
    return dict(out=G.bf16_to_np(out), out_bits=out.cpu().numpy(), lse=lse.cpu().numpy().astype(np.float64),
                sel=sel.cpu().numpy())


def test_static_scratch_matches_workspace_entry():
    big = make_workload("static_big", 81, [150000, 140000], 1, 32, 2, 4, KV_NVFP4, IDX_FP8, table="permute",
                        n_planted=4)
    small = make_workload("static_small", 82, [3000, 129, 700], 4, 16, 2, 8, KV_NVFP4, IDX_NVFP4, table="permute")
    runs = [G.Run(big), G.Run(small)]
    got = [_call_static(r) for r in runs]          # two calls in a row on the same static scratch
    for r, g in zip(runs, got):
        want = r.layer(single=True)
        assert np.array_equal(g["out_bits"], want["out_bits"]), r.w.name
        assert np.array_equal(g["lse"].view(np.uint64), want["lse"].view(np.uint64)), r.w.name
        assert np.array_equal(g["sel"], want["sel"]), r.w.name
    G.compare_layer(small, got[1], G.oracle_refs(small), label="static_small")
    # and again after the workspace calls: the static words of the first
    # calls carry older tags and are not read
    again = _call_static(runs[0])
    assert np.array_equal(again["out_bits"], got[0]["out_bits"])
