"""GPU parity of every C-ABI call against the CPU oracle on the reduced workloads.

Integers (routing ids, counts, permutations, copied rows, fp8 codes and scales of
the routed activations) must match bit for bit; floats within the tolerance of
the workload's dtype (max over rows of max|gpu - oracle| / max|oracle|):
2e-2 bf16, 6e-2 fp8, 1e-5 fp32.  Routing is compared given identical float32
logits: the oracle routes on the logits the GPU produced, and those logits are
checked against the oracle's own within 1e-5 of the row maximum.
"""
import numpy as np
import pytest
import torch

from oracle import moe as O
from synth import configs, inputs
from synth.device import to_dev
from tests.gpu_helpers import (act_to_f64, check_close, empty_act, host, max_row_rel_err, poison_,
                               round_bf16_bits, say, tol_of)

pytestmark = pytest.mark.gpu

GATED = [n for n in configs.SMALL_CONFIGS if not configs.get(n).pretagged]
ALL = list(configs.SMALL_CONFIGS)


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


_cache = {}


def case(name):
    if name not in _cache:
        cfg = configs.get(name)
        d = inputs.layer_inputs(cfg)
        _cache[name] = (cfg, d, {k: to_dev(v) for k, v in d.items() if isinstance(v, np.ndarray)})
    return _cache[name]


def ws_for(M, s):
    n = M.moe_workspace_bytes(s)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def routing_ids(cfg, d):
    """Ids the routing tests start from: the oracle's own top-k, or the pretagged ids."""
    if cfg.pretagged:
        return d["ids"]
    x = O.to_f64(d["x"], cfg.act)
    idx, _ = O.route_topk(O.gate_logits(x, O.to_f64(d["w_gate"], cfg.act)).astype(np.float32),
                          d["bias"], cfg.k)
    return idx


# ----------------------------------------------------------------------------- gate + router

@pytest.mark.parametrize("name", GATED)
def test_gate_topk(M, name):
    cfg, d, g = case(name)
    say("gate_topk", name)
    s = M.shape_of(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    logits = poison_(torch.empty((T, E), dtype=torch.float32, device="cuda"))
    idx = poison_(torch.empty((T, k), dtype=torch.int32, device="cuda"))
    w = poison_(torch.empty((T, k), dtype=torch.float32, device="cuda"))
    M.moe_gate_topk(s, g["x"], g["w_gate"], g.get("bias"), logits, idx, w, ws_for(M, s))
    torch.cuda.synchronize()
    l_gpu = host(logits)
    l_ref = O.gate_logits(O.to_f64(d["x"], cfg.act), O.to_f64(d["w_gate"], cfg.act))
    assert np.isfinite(l_gpu).all()
    err = np.abs(l_gpu - l_ref).max(axis=1) / np.abs(l_ref).max(axis=1)
    assert err.max() <= 1e-5, err.max()
    ridx, rw = O.route_topk(l_gpu, d["bias"], k)     # the router's definition on the GPU logits
    assert np.array_equal(host(idx), ridx)
    assert np.abs(host(w) - rw).max() <= 1e-6
    assert np.abs(host(w).sum(axis=1) - 1).max() <= 1e-6
    # without a logits buffer (they stay in the workspace) the routing is the same, bit for bit
    idx2 = poison_(torch.empty((T, k), dtype=torch.int32, device="cuda"))
    w2 = poison_(torch.empty((T, k), dtype=torch.float32, device="cuda"))
    M.moe_gate_topk(s, g["x"], g["w_gate"], g.get("bias"), None, idx2, w2, ws_for(M, s))
    torch.cuda.synchronize()
    assert np.array_equal(host(idx2), host(idx)) and np.array_equal(host(w2), host(w))


# ----------------------------------------------------------------------------- init routing

def run_init_routing(M, cfg, g, ids_dev, T, k, E, e_base, with_rows=True):
    s = M.shape(T, cfg.H, E, k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    R = T * k
    fp8 = cfg.wt == "fp8"
    i8 = cfg.wt in ("int8", "int4")
    ex = None
    exs = None
    if with_rows:
        if fp8 or i8:
            ex = poison_(torch.empty((R, cfg.H), dtype=torch.uint8 if fp8 else torch.int8, device="cuda"))
            exs = poison_(torch.empty((R, cfg.H // 128) if fp8 else (R,), dtype=torch.float32, device="cuda"))
        else:
            ex = poison_(empty_act((R, cfg.H), cfg.act))
    eri = poison_(torch.empty(R, dtype=torch.int32, device="cuda"))
    ssrc = poison_(torch.empty(R, dtype=torch.int32, device="cuda"))
    tpe = poison_(torch.empty(E, dtype=torch.int32, device="cuda"))
    offs = poison_(torch.empty(E + 1, dtype=torch.int32, device="cuda"))
    ws = ws_for(M, s)
    M.moe_init_routing(s, g["x"] if with_rows else None, ids_dev, e_base, ex, exs, eri, ssrc, tpe, offs, ws)
    torch.cuda.synchronize()
    return dict(ex=ex, exs=exs, eri=eri, ssrc=ssrc, tpe=tpe, offs=offs, ws=ws)


@pytest.mark.parametrize("name", ALL)
def test_init_routing(M, name):
    cfg, d, g = case(name)
    say("init_routing", name)
    ids = routing_ids(cfg, d)
    k = ids.shape[1]
    out = run_init_routing(M, cfg, g, to_dev(np.ascontiguousarray(ids, dtype=np.int32)), cfg.T, k, cfg.E,
                           cfg.e_base)
    ref = O.init_routing(ids, cfg.E, cfg.e_base)
    assert np.array_equal(host(out["tpe"]), ref["tokens_per_expert"])
    assert np.array_equal(host(out["offs"]), ref["expert_offsets"])
    assert np.array_equal(host(out["eri"]), ref["expanded_row_idx"])
    assert np.array_equal(host(out["ssrc"]), ref["sorted_src"])
    if cfg.wt == "fp8":
        xq, xs = O.quant_1x128(O.to_f64(d["x"], cfg.act).astype(np.float32))
        assert np.array_equal(host(out["ex"]), O.expand_rows(xq, ref["sorted_src"], k))
        assert np.array_equal(host(out["exs"]), O.expand_rows(xs, ref["sorted_src"], k))
    elif cfg.wt in ("int8", "int4"):
        # per-token int8 codes and row scales, bit for bit
        xq, xs = O.quant_per_token_int8(O.to_f64(d["x"], cfg.act).astype(np.float32))
        assert np.array_equal(host(out["ex"]), O.expand_rows(xq, ref["sorted_src"], k))
        assert np.array_equal(host(out["exs"]), xs[ref["sorted_src"] // k])
    else:
        want = O.expand_rows(d["x"], ref["sorted_src"], k)
        got = host(out["ex"])
        if cfg.act == "bf16":
            got = got.view(np.uint16)
        assert np.array_equal(got, want)
    assert M.moe_get_error(out["ws"]) == M.MOE_OK


# ----------------------------------------------------------------------------- grouped FFN

def oracle_sorted_inputs(cfg, d):
    ids = routing_ids(cfg, d)
    k = ids.shape[1]
    rt = O.init_routing(ids, cfg.E, cfg.e_base)
    if cfg.wt == "fp8":
        xq, xs = O.quant_1x128(O.to_f64(d["x"], cfg.act).astype(np.float32))
        a_bytes = O.expand_rows(xq, rt["sorted_src"], k)
        a_scale = O.expand_rows(xs, rt["sorted_src"], k)
        a64 = O.dequant_1x128(a_bytes, a_scale)
    elif cfg.wt in ("int8", "int4"):
        xq, xs = O.quant_per_token_int8(O.to_f64(d["x"], cfg.act).astype(np.float32))
        a_bytes = O.expand_rows(xq, rt["sorted_src"], k)
        a_scale = np.ascontiguousarray(xs[rt["sorted_src"] // k])
        a64 = O.dequant_rows(a_bytes, a_scale)
    else:
        a_bytes = O.expand_rows(d["x"], rt["sorted_src"], k)
        a_scale = None
        a64 = O.expand_rows(O.to_f64(d["x"], cfg.act), rt["sorted_src"], k)
    return ids, k, rt, a_bytes, a_scale, a64


@pytest.mark.parametrize("name", ALL)
def test_grouped_ffn(M, name):
    cfg, d, g = case(name)
    say("grouped_ffn", name)
    ids, k, rt, a_bytes, a_scale, a64 = oracle_sorted_inputs(cfg, d)
    R = a_bytes.shape[0]
    s = M.shape_of(cfg)
    y = poison_(empty_act((R, cfg.H), cfg.act))
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, R), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn(s, cfg.E, R, to_dev(a_bytes), to_dev(a_scale), to_dev(rt["expert_offsets"]),
                      g["w13"], g.get("w13_scale"), g["w2"], g.get("w2_scale"), y, ws)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(a64, rt["expert_offsets"], O.expert_weights_f64(d),
                        quant_h="int8" if cfg.wt in ("int8", "int4") else cfg.wt == "fp8")
    got = act_to_f64(y, cfg.act)
    assert np.isfinite(got).all()
    check_close(f"grouped_ffn {name}", got, ref, tol_of(cfg))


# ----------------------------------------------------------------------------- finalize

@pytest.mark.parametrize("name", GATED)
def test_finalize(M, name):
    cfg, d, g = case(name)
    say("finalize", name)
    rng = np.random.default_rng(cfg.cid)
    ids = routing_ids(cfg, d)
    rt = O.init_routing(ids, cfg.E)
    R, T, H, k = cfg.R, cfg.T, cfg.H, cfg.k
    w = rng.random((T, k)).astype(np.float32)
    if cfg.act == "bf16":
        y_bits = round_bf16_bits(rng.standard_normal((R, H)))
        s_bits = round_bf16_bits(rng.standard_normal((T, H)))
        y64, s64 = O.bf16_bits_to_f64(y_bits), O.bf16_bits_to_f64(s_bits)
        yd, sd = to_dev(y_bits), to_dev(s_bits)
    else:
        y64 = rng.standard_normal((R, H)).astype(np.float32).astype(np.float64)
        s64 = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
        yd, sd = to_dev(y64.astype(np.float32)), to_dev(s64.astype(np.float32))
    out = poison_(empty_act((T, H), cfg.act))
    s = M.shape_of(cfg)
    M.moe_finalize_routing(s, yd, sd, to_dev(w), to_dev(rt["expanded_row_idx"]), out)
    torch.cuda.synchronize()
    ref = O.finalize(y64, rt["expanded_row_idx"], k, w, s64)
    # fp32 accumulation then one rounding to the output dtype
    bound = 2.0 ** -8 if cfg.act == "bf16" else 1e-6
    check_close(f"finalize {name}", act_to_f64(out, cfg.act), ref, bound)


@pytest.mark.parametrize("name", ["p3_ep_rank_bf16", "p2_prefill_bf16"])
def test_unsort_is_exact(M, name):
    """k = 1, no weights, no skip: the un-sort of re-routed rows, bit-exact."""
    cfg, d, g = case(name)
    say("unsort", name)
    T, H = cfg.T, cfg.H
    ids = np.random.default_rng(5).integers(0, cfg.E, size=(T, 1)).astype(np.int32)
    rt = O.init_routing(ids, cfg.E)
    y_bits = round_bf16_bits(np.random.default_rng(6).standard_normal((T, H)))
    out = poison_(empty_act((T, H), "bf16"))
    s = M.shape(T, H, cfg.E, 1, cfg.I, cfg.I_shared, "bf16", "bf16")
    M.moe_finalize_routing(s, to_dev(y_bits), None, None, to_dev(rt["expanded_row_idx"]), out)
    torch.cuda.synchronize()
    want = O.unsort(y_bits, rt["sorted_src"])
    assert np.array_equal(host(out).view(np.uint16), want)


# ----------------------------------------------------------------------------- whole layer

def run_layer(M, cfg, g, T=None):
    T = cfg.T if T is None else T
    s = M.shape(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    out = poison_(empty_act((T, cfg.H), cfg.act))
    idx = poison_(torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"))
    w = poison_(torch.empty((T, cfg.k), dtype=torch.float32, device="cuda"))
    logits = poison_(torch.empty((T, cfg.E), dtype=torch.float32, device="cuda"))
    W = M.weights_of(g)
    M.moe_layer(s, W, g["x"], out, idx, w, logits, ws_for(M, s))
    torch.cuda.synchronize()
    return out, idx, w, logits


@pytest.mark.parametrize("name", GATED)
def test_layer(M, name):
    cfg, d, g = case(name)
    say("layer", name)
    out, idx, w, logits = run_layer(M, cfg, g)
    l_gpu = host(logits)
    ref = O.moe_layer(d, logits32_override=l_gpu)
    assert np.array_equal(host(idx), ref["topk_idx"])
    assert np.abs(host(w) - ref["topk_w"]).max() <= 1e-6
    check_close(f"layer {name}", act_to_f64(out, cfg.act), ref["out"], tol_of(cfg))
    # the oracle's own logits select the same experts except at near-ties
    l_ref = ref["logits"].astype(np.float32)
    own, _ = O.route_topk(l_ref, d["bias"], cfg.k)
    flips = np.nonzero((own != ref["topk_idx"]).any(axis=1))[0]
    for t in flips:
        z = np.sort(l_ref[t] + (0 if d["bias"] is None else d["bias"]))[::-1]
        assert z[cfg.k - 1] - z[cfg.k] <= 1e-5 * np.abs(l_ref[t]).max()


def test_layer_is_deterministic(M):
    cfg, d, g = case("p2_prefill_bf16")
    say("layer determinism")
    a = [host(t).copy() for t in run_layer(M, cfg, g)]
    b = [host(t).copy() for t in run_layer(M, cfg, g)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_ep_rank_share(M):
    """Re-routing of pretagged received rows, grouped experts, un-sort back to arrival
    order and the shared expert on the local tokens, composed from the C-ABI calls."""
    cfg, d, g = case("p3_ep_rank_bf16")
    say("ep rank share")
    R, H = cfg.T, cfg.H
    # the re-routing writes no sorted copy: the expert GEMM reads the received rows in place
    rr = run_init_routing(M, cfg, g, g["ids"], cfg.T, 1, cfg.E, cfg.e_base, with_rows=False)
    s = M.shape_of(cfg)
    y = poison_(empty_act((R, H), cfg.act))
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, R), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn_gathered(s, cfg.E, R, g["x"], R, None, rr["ssrc"], 1, rr["offs"], g["w13"], None,
                               g["w2"], None, y, ws)
    y_arr = poison_(empty_act((R, H), cfg.act))
    M.moe_finalize_routing(s, y, None, None, rr["eri"], y_arr)
    # shared expert: one group of T_local rows
    s_sh = M.shape(cfg.T_local, H, 1, 1, cfg.I_shared, cfg.I_shared, cfg.act, cfg.act)
    sh = poison_(empty_act((cfg.T_local, H), cfg.act))
    ws2 = torch.empty(M.moe_grouped_ffn_workspace_bytes(s_sh, 1, cfg.T_local), dtype=torch.uint8,
                      device="cuda")
    offs1 = torch.tensor([0, cfg.T_local], dtype=torch.int32, device="cuda")
    M.moe_grouped_ffn(s_sh, 1, cfg.T_local, g["x_local"], None, offs1, g["sh_w13"], None, g["sh_w2"], None,
                      sh, ws2)
    torch.cuda.synchronize()
    ref = O.moe_layer(d)
    assert np.array_equal(host(rr["ssrc"]), ref["sorted_src"])
    assert np.array_equal(host(rr["tpe"]), ref["tokens_per_expert"])
    check_close(f"ep rank share routed {cfg.name}", act_to_f64(y_arr, cfg.act), ref["y_arrival"], tol_of(cfg))
    check_close(f"ep rank share shared {cfg.name}", act_to_f64(sh, cfg.act), ref["shared"], tol_of(cfg))
    # the arrival-order output is the page's index_select(y_sorted, argsort(gathered_ids_unsort))
    y_sorted_bits = host(y).view(np.uint16)
    assert np.array_equal(host(y_arr).view(np.uint16), O.unsort(y_sorted_bits, host(rr["ssrc"])))


# Tall and short tiles, split-K, several down-projection tiles per workgroup, and every
# weight type.
GATHERED = ["p2_prefill_bf16", "p4_decode_bf16", "p5_skewed_fp8", "p5b_decode_fp8", "p6_prefill_w8a8",
            "p8_prefill_w4a8", "p9_decode_w4a8", "p10_split_bf16", "p11_split_fp8", "p12_split_w8a8",
            "p14_multi_bf16", "p15_multi_w8a8", "p16_multi_w4a8"]


@pytest.mark.parametrize("name", GATHERED)
def test_grouped_ffn_gathered_matches_copied_rows(M, name):
    """The gathered grouped FFN reads sorted row r as row row_of[r] / row_div of its input.
    On the same rows it equals moe_grouped_ffn on the sorted copy, bit for bit: for tokens in
    token order (row_of = sorted_src, row_div = k) and for the sorted rows shuffled
    (row_of = the inverse shuffle, row_div = 1)."""
    cfg, d, g = case(name)
    say("gathered ffn", name)
    ids = routing_ids(cfg, d)
    T, k = ids.shape
    R = T * k
    rr = run_init_routing(M, cfg, g, to_dev(np.ascontiguousarray(ids, dtype=np.int32)), T, k, cfg.E, cfg.e_base)
    s = M.shape(T, cfg.H, cfg.E, k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    ex, exs = rr["ex"], rr["exs"]
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, R), dtype=torch.uint8, device="cuda")
    w = (g["w13"], g.get("w13_scale"), g["w2"], g.get("w2_scale"))
    want = poison_(empty_act((R, cfg.H), cfg.act))
    M.moe_grouped_ffn(s, cfg.E, R, ex, exs, rr["offs"], w[0], w[1], w[2], w[3], want, ws)
    torch.cuda.synchronize()
    want = host(want).view(np.uint8)
    # each token's row (codes and scales for quantized activations) is its first slot's row
    first = rr["eri"].view(T, k)[:, 0].long()
    tok, tok_s = ex[first].contiguous(), (exs[first].contiguous() if exs is not None else None)
    y = poison_(empty_act((R, cfg.H), cfg.act))
    M.moe_grouped_ffn_gathered(s, cfg.E, R, tok, T, tok_s, rr["ssrc"], k, rr["offs"], *w, y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint8), want)
    # sorted rows in a shuffled order: shuffled row i is sorted row p[i]
    p = torch.randperm(R, generator=torch.Generator().manual_seed(cfg.cid)).to("cuda")
    inv = torch.argsort(p).to(torch.int32)
    sh, sh_s = ex[p].contiguous(), (exs[p].contiguous() if exs is not None else None)
    y = poison_(empty_act((R, cfg.H), cfg.act))
    M.moe_grouped_ffn_gathered(s, cfg.E, R, sh, R, sh_s, inv, 1, rr["offs"], *w, y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint8), want)


def test_grouped_ffn_gathered_no_rows(M):
    """No rows at all (every group empty): the call succeeds without a row pointer or a
    row map and leaves the output as it was."""
    cfg, d, g = case("p4_decode_bf16")
    say("gathered ffn, no rows")
    s = M.shape(0, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    offs = torch.zeros(cfg.E + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, 0), dtype=torch.uint8, device="cuda")
    y = poison_(empty_act((4, cfg.H), cfg.act))
    torch.cuda.synchronize()
    before = host(y).copy()
    M.moe_grouped_ffn_gathered(s, cfg.E, 0, None, 0, None, None, 1, offs, g["w13"], None, g["w2"], None, y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint8), before.view(np.uint8))


# ----------------------------------------------------------------------------- edge cases

def test_all_tokens_to_one_expert(M):
    """Maximum skew: every slot to expert 3 -> one group of T*k rows split into units."""
    cfg, d, g = case("p2_prefill_bf16")
    say("one expert")
    T, k = cfg.T, 1
    ids = np.full((T, 1), 3, dtype=np.int32)
    out = run_init_routing(M, cfg, g, to_dev(ids), T, k, cfg.E, 0)
    tpe = host(out["tpe"])
    assert tpe[3] == T and tpe.sum() == T
    assert np.array_equal(host(out["ssrc"]), np.arange(T))
    s = M.shape(T, cfg.H, cfg.E, 1, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    y = poison_(empty_act((T, cfg.H), cfg.act))
    ws = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, cfg.E, T), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn(s, cfg.E, T, out["ex"], None, out["offs"], g["w13"], None, g["w2"], None, y, ws)
    torch.cuda.synchronize()
    ref = O.swiglu_ffn(O.to_f64(d["x"], cfg.act), O.to_f64(d["w13"][3], cfg.wt), O.to_f64(d["w2"][3], cfg.wt))
    check_close("all tokens to one expert", act_to_f64(y, cfg.act), ref, tol_of(cfg))


# Routing runs in one launch for up to 16 segments of 1024 slots whose per-segment counts
# fit in 60 KB of LDS, and in three launches otherwise: both sides of each boundary, with a
# skewed expert popularity (one expert takes a quarter of the slots) and two invalid ids.
@pytest.mark.parametrize("T,k,E", [(2048, 8, 256), (2049, 8, 256), (900, 16, 1024),
                                   (1000, 16, 1024), (3, 5, 7), (5000, 1, 1), (40000, 1, 1)])
def test_routing_single_and_three_launch(M, T, k, E):
    cfg, _, g = case("p4_decode_bf16")
    say("routing paths", T, k, E)
    rng = np.random.default_rng(1000 + T * 31 + k * 7 + E)
    ids = rng.integers(0, E, (T, k))
    ids[rng.random(T) < 0.25, 0] = 0                 # a quarter of the tokens pick expert 0
    ids[T // 2, k - 1] = E                            # two slots outside the local experts
    ids[T - 1, 0] = -1
    ids = np.ascontiguousarray(ids + cfg.e_base, dtype=np.int32)
    out = run_init_routing(M, cfg, g, to_dev(ids), T, k, E, cfg.e_base, with_rows=False)
    ref = O.init_routing(ids, E, cfg.e_base)
    assert ref["n_invalid"] == (1 if (T // 2, k - 1) == (T - 1, 0) else 2)
    assert np.array_equal(host(out["tpe"]), ref["tokens_per_expert"])
    assert np.array_equal(host(out["offs"]), ref["expert_offsets"])
    assert np.array_equal(host(out["eri"]), ref["expanded_row_idx"])
    n = int(ref["expert_offsets"][-1])
    assert np.array_equal(host(out["ssrc"])[:n], ref["sorted_src"])
    assert M.moe_get_error(out["ws"]) == M.MOE_EDEVICE
    assert M.moe_get_error(out["ws"]) == M.MOE_OK


def test_invalid_ids_are_flagged_and_dropped(M):
    cfg, d, g = case("p3_ep_rank_bf16")
    say("invalid ids")
    ids = d["ids"].copy()
    ids[5, 0] = 3            # below e_base
    ids[77, 0] = 10_000      # above e_base + E
    out = run_init_routing(M, cfg, g, to_dev(ids), cfg.T, 1, cfg.E, cfg.e_base)
    ref = O.init_routing(ids, cfg.E, cfg.e_base)
    assert ref["n_invalid"] == 2
    assert np.array_equal(host(out["eri"]), ref["expanded_row_idx"])
    n = int(ref["expert_offsets"][-1])
    assert np.array_equal(host(out["ssrc"])[:n], ref["sorted_src"])
    assert np.array_equal(host(out["tpe"]), ref["tokens_per_expert"])
    assert M.moe_get_error(out["ws"]) == M.MOE_EDEVICE
    assert M.moe_get_error(out["ws"]) == M.MOE_OK          # read-and-clear


# p4 keeps the unsplit decode tiles; the split workloads at one or two tokens take the
# split-K expert GEMMs (and an unmerged, split shared expert) for every dtype
@pytest.mark.parametrize("name,T", [("p4_decode_bf16", 0), ("p4_decode_bf16", 1), ("p4_decode_bf16", 17),
                                    ("p10_split_bf16", 1), ("p11_split_fp8", 1),
                                    ("p12_split_w8a8", 2), ("p13_split_w4a8", 1)])
def test_small_token_counts(M, name, T):
    cfg, d, g = case(name)
    say("small T", name, T)
    if T == 0:
        s = M.shape(0, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
        W = M.weights(g["w_gate"], g["w13"], g["w2"], g["sh_w13"], g["sh_w2"], None, None, g["bias"])
        ws = ws_for(M, s)
        M.moe_layer(s, W, None, None, None, None, None, ws)
        torch.cuda.synchronize()
        return
    sub = dict(d)
    sub["x"] = d["x"][:T]
    gs = dict(g)
    gs["x"] = g["x"][:T].contiguous()
    out, idx, w, logits = run_layer(M, cfg, gs, T=T)
    ref = O.moe_layer(sub, logits32_override=host(logits))
    assert np.array_equal(host(idx), ref["topk_idx"])
    check_close(f"small T {name} T={T}", act_to_f64(out, cfg.act), ref["out"], tol_of(cfg))


def test_library_is_the_hip_build():
    """The process runs the in-tree HIP library on torch's HIP runtime (one runtime mapped)."""
    import moe_expert_layer_top_amd as m
    m.lib()
    maps = open("/proc/self/maps").read()
    assert "moe_expert_layer_top_amd/libmoe.so" in maps
    runtimes = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes
