"""GPU parity of the router variants ([MND §MoE Router]: group-limited top-k, softmax
scoring, no renormalization, a routed scaling factor) against the oracle's
route_grouped.  As for the plain router, the ids must match bit for bit given the
GPU's float32 logits, and the weights within 1e-6 (times the scaling factor)."""
import numpy as np
import pytest
import torch

from oracle import moe as O
from synth import configs
from tests.gpu_helpers import act_to_f64, check_close, empty_act, host, poison_, say, tol_of
from tests.test_gpu_parity import case, ws_for

pytestmark = pytest.mark.gpu

ROUTERS = {
    "softmax": dict(scoring="softmax"),
    "softmax_raw": dict(scoring="softmax", renormalize=False),
    "grouped_top2": dict(n_group=8, topk_group=4, group_topn=2),
    "grouped_softmax_scaled": dict(scoring="softmax", n_group=4, topk_group=2, group_topn=1, scale=2.5),
    "sigmoid_raw_scaled": dict(renormalize=False, scale=2.5),
    "one_group_kept": dict(n_group=4, topk_group=1, group_topn=2),
}
CONFIGS = ["p2_prefill_bf16", "p2b_prefill_bf16", "p4_decode_bf16", "p1_small_fp32"]


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


def fits(cfg, r):
    G, TG = r.get("n_group", 1), r.get("topk_group", 1)
    return cfg.E % G == 0 and cfg.k <= TG * (cfg.E // G) and r.get("group_topn", 1) <= cfg.E // G


def gate(M, cfg, g, r, T=None):
    T = cfg.T if T is None else T
    s = M.shape(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    logits = poison_(torch.empty((T, cfg.E), dtype=torch.float32, device="cuda"))
    idx = poison_(torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"))
    w = poison_(torch.empty((T, cfg.k), dtype=torch.float32, device="cuda"))
    M.moe_gate_topk_ex(s, M.router(**r), g["x"], g["w_gate"], g.get("bias"), logits, idx, w, ws_for(M, s))
    torch.cuda.synchronize()
    return host(logits), host(idx), host(w)


@pytest.mark.parametrize("rname", list(ROUTERS))
@pytest.mark.parametrize("name", CONFIGS)
def test_gate_topk_router(M, name, rname):
    cfg, d, g = case(name)
    r = ROUTERS[rname]
    if not fits(cfg, r):
        pytest.skip(f"{rname} needs k <= kept experts and n_group | E")
    say("router", name, rname)
    l_gpu, i_gpu, w_gpu = gate(M, cfg, g, r)
    ref_idx, ref_w = O.route_grouped(l_gpu, d["bias"], cfg.k, r)
    assert np.array_equal(i_gpu, ref_idx)
    assert np.abs(w_gpu - ref_w).max() <= 1e-6 * max(1.0, r.get("scale", 1.0))
    ref_l = O.gate_logits(O.to_f64(d["x"], cfg.act), O.to_f64(d["w_gate"], cfg.act))
    assert (np.abs(l_gpu - ref_l).max(axis=1) / np.abs(ref_l).max(axis=1)).max() <= 1e-5


def test_gate_topk_router_full_c2(M):
    """DeepSeek-V3-shaped grouping at the full c2 size: 256 experts in 8 groups, 4 kept,
    groups scored by their best two, weights scaled by 2.5."""
    from synth.device import to_dev
    from synth import inputs
    cfg = configs.get("c2_prefill_bf16")
    r = dict(n_group=8, topk_group=4, group_topn=2, scale=2.5)
    say("router full c2")
    g = {"x": to_dev(inputs.tokens(cfg)), "w_gate": to_dev(inputs.gate_weight(cfg)), "bias": None}
    l_gpu, i_gpu, w_gpu = gate(M, cfg, g, r)
    ref_idx, ref_w = O.route_grouped(l_gpu, None, cfg.k, r)
    assert np.array_equal(i_gpu, ref_idx)
    assert np.abs(w_gpu - ref_w).max() <= 2.5e-6
    # every selected expert lies in one of the 4 kept groups of 32
    assert (np.array([len(set(row // 32)) for row in i_gpu]) <= 4).all()


@pytest.mark.parametrize("rname", ["grouped_softmax_scaled", "grouped_top2", "softmax"])
@pytest.mark.parametrize("name", ["p2_prefill_bf16", "p5_skewed_fp8", "p1_small_fp32"])
def test_layer_router(M, name, rname):
    cfg, d, g = case(name)
    r = ROUTERS[rname]
    if not fits(cfg, r):
        pytest.skip(f"{rname} does not fit {name}")
    say("layer router", name, rname)
    s = M.shape_of(cfg)
    out = poison_(empty_act((cfg.T, cfg.H), cfg.act))
    idx = poison_(torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda"))
    w = poison_(torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda"))
    logits = poison_(torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda"))
    W = M.weights_of(g)
    M.moe_layer_ex(s, M.router(**r), W, g["x"], out, idx, w, logits, ws_for(M, s), side=torch.cuda.Stream())
    torch.cuda.synchronize()
    ref = O.moe_layer(d, logits32_override=host(logits), router=r)
    assert np.array_equal(host(idx), ref["topk_idx"])
    # the combine's weights sum to `scale` instead of 1: the tolerance is relative to the
    # output rows, which scale with it
    check_close(f"router layer {cfg.name} {sorted(r.items())}", act_to_f64(out, cfg.act), ref["out"],
                tol_of(cfg))


def test_layer_ex_default_router_is_moe_layer(M):
    cfg, d, g = case("p2_prefill_bf16")
    s = M.shape_of(cfg)
    W = M.weights(g["w_gate"], g["w13"], g["w2"], g["sh_w13"], g["sh_w2"], None, None, g.get("bias"))
    outs = []
    for ex in (False, True):
        out = poison_(empty_act((cfg.T, cfg.H), cfg.act))
        if ex:
            M.moe_layer_ex(s, None, W, g["x"], out, None, None, None, ws_for(M, s))
        else:
            M.moe_layer(s, W, g["x"], out, None, None, None, ws_for(M, s))
        torch.cuda.synchronize()
        outs.append(host(out).copy())
    assert np.array_equal(outs[0], outs[1])
