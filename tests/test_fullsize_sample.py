"""Host checks of the token sample the full-size GPU parity tests check (no GPU): the
sample reaches every active expert, and every unit of the hottest experts of the skewed
fp8 workload has its first and last row among the sampled tokens' rows."""
import os

import numpy as np
import pytest

import moe_expert_layer_top_amd as M
from moe_expert_layer_top_amd import _lib
from oracle import moe as O
from synth import configs, inputs
from tests.test_gpu_fullsize import block_rows, sample_tokens, slice_bounds, unit_bounds


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return M.lib()


def test_unit_bounds_on_a_small_table():
    # experts of 0, 5, 300 (one unit of 320) and 700 rows (three units of 240, 240, 220)
    offs = np.cumsum([0, 0, 5, 300, 700])
    assert unit_bounds(offs, 320) == [0, 4, 5, 304, 305, 544, 545, 784, 785, 1004]
    assert slice_bounds(1000, 320) == [0, 255, 256, 511, 512, 767, 768, 999]


def test_c5_hot_expert_units_are_sampled(L):
    """The three hottest experts of the skewed fp8 layer span several units each, and the
    first and last row of every one of their units is a row of a sampled token (the GPU
    test then checks those tokens' outputs against the oracle).  Routing from the
    oracle's own logits."""
    cfg = configs.get("c5_skewed_fp8")
    x = O.to_f64(inputs.tokens(cfg), cfg.act)
    l32 = O.gate_logits(x, O.to_f64(inputs.gate_weight(cfg), cfg.act)).astype(np.float32)
    del x
    idx, _ = O.route_topk(l32, inputs.expert_bias(cfg), cfg.k)
    rt = O.init_routing(idx, cfg.E)
    bm, bm_sh = block_rows(M, cfg)
    S = sample_tokens(cfg, rt, bm, bm_sh)
    assert len(S) < cfg.T // 4
    sampled_rows = set(rt["expanded_row_idx"].reshape(cfg.T, cfg.k)[S].reshape(-1).tolist())
    assert set(idx[S].reshape(-1).tolist()) == set(np.nonzero(rt["tokens_per_expert"])[0].tolist())
    hot = np.argsort(-rt["tokens_per_expert"], kind="stable")[:3]
    offs = rt["expert_offsets"]
    for e in hot:
        sub = np.array([0, offs[e + 1] - offs[e]])
        bounds = [int(offs[e]) + r for r in unit_bounds(sub, bm)]
        assert len(bounds) >= 8, (e, len(bounds))          # several units
        assert set(bounds) <= sampled_rows, e
