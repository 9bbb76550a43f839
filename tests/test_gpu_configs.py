"""GPU parity at the full sizes of the decode workloads, every sequence and
every query token, through both layer entry points (the launch
configurations bench.py times): the whole batch runs on the GPU and the
oracle recomputes every (sequence, token): selection tie-aware, outputs
element by element to max-abs 2e-3 where |o| < 0.5 (half a bf16 ulp plus
the fp16-weight slack above), mean-abs 2e-4 against the unrounded oracle,
lse to 2e-3. The tie-band selection count of every workload is printed and,
when MSA_PARITY_LOG names a file, appended to it as one JSON line."""
import json
import os
import time

import numpy as np
import pytest

from tests import gpu_util as G
from workloads import make_config, IDX_NVFP4

pytestmark = pytest.mark.gpu


def _record(name, entry, ties, tokens, mx, mean, secs):
    line = dict(workload=name, entry=entry, tie_band_tokens=ties, tokens=tokens, out_max_abs_small=mx,
                out_mean_abs=mean, seconds=round(secs, 1))
    print(json.dumps(line))
    path = os.environ.get("MSA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def _full(cfg, idx_dtype=None):
    t0 = time.time()
    w = make_config(cfg, idx_dtype=idx_dtype)
    refs = G.oracle_refs(w)
    run = G.Run(w)
    tokens = sum(len(r) for r in refs.values())
    name = w.name + ("" if idx_dtype is None else "/nvfp4-idx")
    sels = []
    for single in (False, True):
        res = run.layer(single=single)
        sels.append(res["sel"])
        ties, mx, mean = G.compare_layer(w, res, refs, strict=True, label=name)
        _record(name, "msa_decode_layer_single" if single else "msa_decode_layer", ties, tokens, mx, mean,
                time.time() - t0)
    # both entry points select from the same pooled scores
    assert np.array_equal(sels[0], sels[1]), (name, "the layer entry points select differently")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_config_full_size_every_token(cfg):
    _full(cfg)


@pytest.mark.parametrize("cfg", [3, 4])
def test_config_full_size_nvfp4_index_keys(cfg):
    # the same workloads with NVFP4 indexer keys (bench.py --idx-dtype nvfp4)
    _full(cfg, IDX_NVFP4)
