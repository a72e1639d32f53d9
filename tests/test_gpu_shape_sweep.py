"""Grouped FFN at exact per-expert row counts around every boundary the kernels cut
rows at: 8-row load chunks (a chunk wholly past a unit's rows is not loaded), 16-row
MFMA tiles, and 32-, 256- and 320-row units (short, fp8 and tall tiles), for every
expert dtype, against the oracle.  Rows are pretagged with their expert, so the counts
are exact; shapes include partial N tiles (H = 384, 640) and the decode-sized grids that
split K.  Same tolerances as the other parity tests.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe as O
from synth import configs, inputs
from synth.device import to_dev
from tests.gpu_helpers import act_to_f64, check_close, empty_act, poison_, say, tol_of

pytestmark = pytest.mark.gpu

# (expert dtype, H, I, rows of each expert)
CASES = [
    ("bf16", 640, 256, [0, 1, 7, 8, 9, 319, 320, 321, 640, 17]),     # tall 320-row tiles
    ("fp8", 384, 256, [255, 256, 257, 0, 512, 1, 129, 8]),           # fp8 256-row tiles
    ("int8", 384, 128, [320, 321, 0, 7, 641, 16]),
    ("int4", 512, 256, [319, 1, 0, 322, 33, 9]),
    ("bf16", 384, 384, [31, 32, 33, 0, 1, 5, 64, 65]),               # short 32-row tiles
    ("fp8", 256, 128, [1, 2, 31, 32, 33, 0, 0, 3]),
    ("int8", 256, 256, [1, 0, 2, 3, 33, 31, 8, 9]),
]


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


def sweep_case(i, wt, H, I, counts):
    G, R = len(counts), int(sum(counts))
    cfg = replace(configs.get("p3_ep_rank_bf16"), name=f"sweep{i}_{wt}", cid=900 + i, T=R, H=H, E=G,
                  k=1, I=I, I_shared=I, wt=wt, e_base=0, E_total=G, T_local=min(R, 64))
    d = inputs.layer_inputs(cfg)
    # rows tagged with exact counts, in a seeded random row order
    ids = np.repeat(np.arange(G, dtype=np.int32), counts)
    ids = ids[np.random.default_rng(cfg.cid).permutation(R)].reshape(R, 1)
    d["ids"] = ids
    return cfg, d


@pytest.mark.parametrize("i", range(len(CASES)))
def test_grouped_ffn_row_count_sweep(M, i):
    wt, H, I, counts = CASES[i]
    cfg, d = sweep_case(i, wt, H, I, counts)
    say("grouped_ffn sweep", f"{cfg.name} H={H} I={I} rows={counts}")
    rt = O.init_routing(d["ids"], cfg.E, cfg.e_base)
    assert np.array_equal(rt["tokens_per_expert"], np.asarray(counts))
    x32 = O.to_f64(d["x"], cfg.act).astype(np.float32)
    if wt == "fp8":
        xq, xs = O.quant_1x128(x32)
        a_bytes = O.expand_rows(xq, rt["sorted_src"], 1)
        a_scale = O.expand_rows(xs, rt["sorted_src"], 1)
        a64 = O.dequant_1x128(a_bytes, a_scale)
    elif wt in ("int8", "int4"):
        xq, xs = O.quant_per_token_int8(x32)
        a_bytes = O.expand_rows(xq, rt["sorted_src"], 1)
        a_scale = np.ascontiguousarray(xs[rt["sorted_src"]])
        a64 = O.dequant_rows(a_bytes, a_scale)
    else:
        a_bytes = O.expand_rows(d["x"], rt["sorted_src"], 1)
        a_scale = None
        a64 = O.expand_rows(O.to_f64(d["x"], cfg.act), rt["sorted_src"], 1)
    R = a_bytes.shape[0]
    s = M.shape_of(cfg)
    y = poison_(empty_act((R, H), cfg.act))
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, R), dtype=torch.uint8, device="cuda")
    keys = ("w13", "w13_scale", "w2", "w2_scale")
    g = {k: to_dev(d[k]) for k in keys if k in d}
    M.moe_grouped_ffn(s, cfg.E, R, to_dev(a_bytes), to_dev(a_scale), to_dev(rt["expert_offsets"]),
                      g["w13"], g.get("w13_scale"), g["w2"], g.get("w2_scale"), y, ws)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(a64, rt["expert_offsets"], O.expert_weights_f64(d),
                        quant_h="int8" if wt in ("int8", "int4") else wt == "fp8")
    got = act_to_f64(y, cfg.act)
    assert np.isfinite(got).all()
    check_close(f"grouped_ffn sweep {cfg.name}", got, ref, tol_of(cfg))
