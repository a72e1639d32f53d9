"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle function against brute force on tiny inputs, a
closed form, an invariant the pages or the mathematics fix, or an independent
library routine -- never against a retyped copy of its own formula.
"""
import itertools
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import moe
from synth import configs, inputs


# ----------------------------------------------------------------------------- fp8 format

def _all_bf16_values():
    v = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return v[np.isfinite(v)]


def test_fp8_encode_matches_library_cast_on_every_bf16_value():
    """Independent routine: torch's float8_e4m3fn cast (round-to-nearest-even) agrees
    with the oracle encoder on every finite bf16 value inside the format's range."""
    v = _all_bf16_values()
    v = v[np.abs(v) <= 464.0]            # beyond 464 the library cast gives NaN, the oracle saturates
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(moe.fp8_e4m3fn_encode(v), ref)


def test_fp8_encode_random_float32_matches_library_cast():
    r = np.random.default_rng(7).standard_normal(200_000).astype(np.float32)
    r = np.concatenate([r * np.float32(0.01), r * np.float32(3.0), r * np.float32(100.0)])
    r = r[np.abs(r) <= 464.0]
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(moe.fp8_e4m3fn_encode(r), ref)


def test_fp8_decode_matches_library_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = moe.fp8_e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("value,code", [
    (448.0, 0x7E), (-448.0, 0xFE),          # largest finite magnitude 1.75 * 2^8
    (1.0, 0x38), (2.0 ** -6, 0x08),         # smallest normal
    (2.0 ** -9, 0x01),                      # smallest subnormal
    (1.0625, 0x38),                         # tie between 1 and 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),                         # tie between 1.125 and 1.25 -> even mantissa (1.25)
    (1000.0, 0x7E), (-1e30, 0xFE),          # saturation
    (2.0 ** -11, 0x00), (-0.0, 0x80),       # underflow to zero keeps the sign
])
def test_fp8_encode_closed_form_points(value, code):
    assert int(moe.fp8_e4m3fn_encode(np.array([value], np.float32))[0]) == code


def test_quant_1x128_amax_maps_to_448_and_zero_block():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 384)).astype(np.float32)
    x[2, 128:256] = 0.0
    q, s = moe.quant_1x128(x)
    # [MND §Quantization]: one scale per 128-element activation vector, shape M x ceil(K/128)
    assert q.shape == (5, 384) and s.shape == (5, 3) and s.dtype == np.float32
    blocks = x.reshape(5, 3, 128)
    for m in range(5):
        for b in range(3):
            if m == 2 and b == 1:
                assert s[m, b] == 1.0 and (q[m, 128 * b:128 * b + 128] == 0).all()
                continue
            i = int(np.argmax(np.abs(blocks[m, b])))
            c = int(q[m, 128 * b + i])
            assert c in (0x7E, 0xFE)                     # amax element is exactly +-448
            assert (c == 0xFE) == (blocks[m, b, i] < 0)


def test_quant_1x128_error_bound():
    """e4m3 has 3 mantissa bits: relative error of a normal value <= 2^-4."""
    x = np.random.default_rng(2).standard_normal((64, 256)).astype(np.float32)
    q, s = moe.quant_1x128(x)
    d = moe.dequant_1x128(q, s)
    normal = np.abs(x) >= np.repeat(s, 128, axis=1) * 2.0 ** -6
    err = np.abs(d - x)
    assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)).all()
    # subnormal range: absolute error <= half the subnormal spacing times the scale
    assert (err[~normal] <= 0.5 * 2.0 ** -9 * np.repeat(s, 128, axis=1)[~normal] * (1 + 1e-6)).all()


def test_dequant_block128_scale_layout():
    """[MND §Quantization]: a weight [N, K] carries ceil(K/128) x ceil(N/128) scales,
    one per 128x128 tile.  Put a distinct power of two in each tile and check that
    exactly that tile is scaled."""
    N, K = 256, 384
    q = np.full((N, K), 0x38, dtype=np.uint8)       # every code = 1.0
    s = np.exp2(np.arange(6, dtype=np.float32)).reshape(2, 3)
    d = moe.dequant_block128(q, s)
    for nb in range(2):
        for kb in range(3):
            assert (d[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128] == 2.0 ** (3 * nb + kb)).all()


# ----------------------------------------------------------------------------- router

def _brute_topk(z, k):
    """Enumerate every k-subset; keep the one in which every member beats every
    non-member (higher score, or equal score and lower id); order it."""
    E = len(z)
    beats = lambda a, b: z[a] > z[b] or (z[a] == z[b] and a < b)
    winners = [S for S in itertools.combinations(range(E), k)
               if all(beats(a, b) for a in S for b in range(E) if b not in S)]
    assert len(winners) == 1
    S = list(winners[0])
    # order: selection by repeated "best remaining"
    out = []
    while S:
        best = S[0]
        for c in S[1:]:
            if beats(c, best):
                best = c
        out.append(best)
        S.remove(best)
    return out


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 6), st.integers(1, 6), st.data())
def test_topk_selection_brute_force(T, E, data):
    k = data.draw(st.integers(1, E))
    # a small value alphabet forces ties
    vals = data.draw(st.lists(st.sampled_from([-1.5, -0.25, 0.0, 0.25, 0.5, 2.0]),
                              min_size=T * E, max_size=T * E))
    z = np.array(vals, dtype=np.float32).reshape(T, E)
    idx, w = moe.route_topk(z, None, k)
    for t in range(T):
        assert list(idx[t]) == _brute_topk(list(z[t]), k)
        assert abs(float(w[t].sum()) - 1.0) <= 1e-6     # weights sum to 1
        assert (w[t] > 0).all()
        assert len(set(idx[t])) == k                    # k distinct experts


def test_topk_weights_closed_form():
    """sigma(ln 3) = 3/4 and sigma(0) = 1/2, so renormalized weights are 0.6 / 0.4."""
    z = np.array([[0.0, math.log(3.0), -5.0]], dtype=np.float32)
    idx, w = moe.route_topk(z, None, 2)
    assert list(idx[0]) == [1, 0]
    assert abs(w[0, 0] - 0.6) < 1e-6 and abs(w[0, 1] - 0.4) < 1e-6


def test_topk_k_equals_E_and_k_one():
    z = np.random.default_rng(3).standard_normal((10, 7)).astype(np.float32)
    idx, w = moe.route_topk(z, None, 7)
    assert (np.sort(idx, axis=1) == np.arange(7)).all()          # every expert selected
    assert (np.diff(np.take_along_axis(z, idx, 1), axis=1) <= 0).all()
    idx1, w1 = moe.route_topk(z, None, 1)
    assert (idx1[:, 0] == np.argmax(z, axis=1)).all() and (w1 == 1.0).all()


def test_topk_bias_shifts_selection():
    z = np.zeros((1, 4), dtype=np.float32)
    b = np.array([0.0, 0.0, 1.0, 0.5], dtype=np.float32)
    idx, w = moe.route_topk(z, b, 2)
    assert list(idx[0]) == [2, 3]
    s = [1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(-0.5))]
    assert np.allclose(w[0], np.array(s) / sum(s), atol=1e-7)


# ----------------------------------------------------------------------------- router variants

def test_router_default_is_the_workload_router():
    """Default router (sigmoid, renormalized, one group) = route_topk bit for bit."""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((40, 16)).astype(np.float32)
    b = rng.standard_normal(16).astype(np.float32) * 0.3
    for k in (1, 3, 8, 16):
        i0, w0 = moe.route_topk(z, b, k)
        i1, w1 = moe.route_grouped(z, b, k)
        assert np.array_equal(i0, i1) and np.array_equal(w0, w1)


@pytest.mark.parametrize("scoring", ["sigmoid", "softmax"])
def test_router_all_groups_kept_is_ungrouped(scoring):
    """[MND §MoE Router]: the ungrouped (Mixtral) routing is the special case in which the
    top-K group is every expert: keeping all G groups selects like one group."""
    rng = np.random.default_rng(12)
    z = rng.standard_normal((30, 24)).astype(np.float32)
    flat = moe.route_grouped(z, None, 5, dict(scoring=scoring))
    for G, GN in ((4, 1), (6, 2), (24, 1)):
        grp = moe.route_grouped(z, None, 5, dict(scoring=scoring, n_group=G, topk_group=G, group_topn=GN))
        assert np.array_equal(flat[0], grp[0]) and np.array_equal(flat[1], grp[1])


def _brute_grouped(z, k, G, TG, GN):
    """Group scores by explicit sorting; the kept groups are the TG-subset whose every
    member beats every other group (higher score, or equal and lower id); the experts are
    the brute-force top-k of the kept groups' experts."""
    E = len(z)
    gsz = E // G
    score = []
    for g in range(G):
        vals = sorted((np.float32(v) for v in z[g * gsz:(g + 1) * gsz]), reverse=True)
        score.append(vals[0] if GN == 1 else np.float32(vals[0] + vals[1]))
    beats = lambda a, b: score[a] > score[b] or (score[a] == score[b] and a < b)
    kept = [S for S in itertools.combinations(range(G), TG)
            if all(beats(a, b) for a in S for b in range(G) if b not in S)]
    assert len(kept) == 1
    cand = [e for g in kept[0] for e in range(g * gsz, (g + 1) * gsz)]
    sub = [z[e] for e in cand]
    return [cand[i] for i in _brute_topk(sub, k)]


@settings(max_examples=200, deadline=None)
@given(st.sampled_from([(4, 2), (6, 3), (6, 2), (8, 4), (8, 2), (9, 3)]), st.data())
def test_grouped_selection_brute_force(EG, data):
    E, G = EG
    gsz = E // G
    TG = data.draw(st.integers(1, G))
    GN = data.draw(st.integers(1, min(2, gsz)))
    k = data.draw(st.integers(1, TG * gsz))
    vals = data.draw(st.lists(st.sampled_from([-1.5, -0.25, 0.0, 0.25, 0.5, 2.0]), min_size=E, max_size=E))
    z = np.array([vals], dtype=np.float32)
    idx, w = moe.route_grouped(z, None, k, dict(n_group=G, topk_group=TG, group_topn=GN))
    assert list(idx[0]) == _brute_grouped(list(z[0]), k, G, TG, GN)
    assert abs(float(w.sum()) - 1.0) <= 1e-6


def test_group_score_top1_vs_top2():
    """Groups of 2: [3, -5], [2, 1.9], [0, 0], [1, 0.5].  By the best expert, group 0 wins;
    by the best two, group 1 (3.9 > 1.5 > 0 > -2)."""
    z = np.array([[3.0, -5.0, 2.0, 1.9, 0.0, 0.0, 1.0, 0.5]], dtype=np.float32)
    i1, _ = moe.route_grouped(z, None, 2, dict(n_group=4, topk_group=1, group_topn=1))
    i2, _ = moe.route_grouped(z, None, 2, dict(n_group=4, topk_group=1, group_topn=2))
    assert list(i1[0]) == [0, 1] and list(i2[0]) == [2, 3]
    i3, _ = moe.route_grouped(z, None, 3, dict(n_group=4, topk_group=2, group_topn=2))
    assert list(i3[0]) == [2, 3, 6]


def test_softmax_weights_library_and_closed_form():
    from scipy.special import softmax
    rng = np.random.default_rng(13)
    z = rng.standard_normal((20, 10)).astype(np.float32)
    # k = E without renormalization: the weights are the softmax over all experts
    idx, w = moe.route_grouped(z, None, 10, dict(scoring="softmax", renormalize=False))
    ref = softmax(z.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx, axis=1), rtol=0, atol=1e-7)
    # top-2 renormalized (Mixtral): w0 = 1 / (1 + exp(z1 - z0))
    idx, w = moe.route_grouped(z, None, 2, dict(scoring="softmax"))
    z0 = np.take_along_axis(z, idx[:, :1], 1)[:, 0].astype(np.float64)
    z1 = np.take_along_axis(z, idx[:, 1:2], 1)[:, 0].astype(np.float64)
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(z1 - z0)), atol=1e-7)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    # without renormalization the selected mass is below 1
    _, w = moe.route_grouped(z, None, 3, dict(scoring="softmax", renormalize=False))
    assert (w.sum(axis=1) < 1.0).all()


def test_sigmoid_without_renormalization_and_scale():
    z = np.array([[0.0, math.log(3.0), -5.0, 1.0]], dtype=np.float32)
    idx, w = moe.route_grouped(z, None, 2, dict(renormalize=False, scale=2.0))
    assert list(idx[0]) == [1, 3]
    assert abs(w[0, 0] - 2.0 * 0.75) < 1e-6
    assert abs(w[0, 1] - 2.0 / (1.0 + math.exp(-1.0))) < 1e-6
    _, w = moe.route_grouped(z, None, 3, dict(scale=2.5))
    assert abs(float(w.sum()) - 2.5) < 1e-6


def test_router_rejects_bad_grouping():
    z = np.zeros((1, 8), dtype=np.float32)
    for r, k in ((dict(n_group=3), 1), (dict(n_group=4, topk_group=5), 1), (dict(n_group=8, group_topn=2), 1),
                 (dict(n_group=4, topk_group=1), 3), (dict(scoring="tanh"), 1)):
        with pytest.raises(ValueError):
            moe.route_grouped(z, None, k, r)


# ----------------------------------------------------------------------------- routing

def _brute_routing(ids, E, e_base):
    flat = [int(v) - e_base for v in np.asarray(ids).reshape(-1)]
    R = len(flat)
    counts = [0] * E
    sorted_src = []
    for e in range(E):                    # expert by expert, slots in ascending order
        for s in range(R):
            if flat[s] == e:
                counts[e] += 1
                sorted_src.append(s)
    eri = [-1] * R
    for r, s in enumerate(sorted_src):
        eri[s] = r
    return counts, sorted_src, eri


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 7), st.integers(1, 5), st.integers(1, 3), st.integers(0, 3), st.data())
def test_init_routing_brute_force(T, E, k, e_base, data):
    ids = np.array(data.draw(st.lists(st.integers(e_base - 1, e_base + E), min_size=T * k,
                                      max_size=T * k)), dtype=np.int32).reshape(T, k)
    r = moe.init_routing(ids, E, e_base)
    counts, sorted_src, eri = _brute_routing(ids, E, e_base)
    assert list(r["tokens_per_expert"]) == counts
    assert list(r["sorted_src"]) == sorted_src
    assert list(r["expanded_row_idx"]) == eri
    assert list(r["expert_offsets"]) == [sum(counts[:e]) for e in range(E + 1)]


def _distinct_topk_ids(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 300), st.integers(1, 40), st.data())
def test_init_routing_invariants(T, E, data):
    k = data.draw(st.integers(1, min(E, 8)))
    rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 31)))
    ids = _distinct_topk_ids(rng, T, E, k)
    r = moe.init_routing(ids, E)
    ss, eri, tpe = r["sorted_src"], r["expanded_row_idx"], r["tokens_per_expert"]
    assert tpe.sum() == T * k                                    # sums to T*k
    assert np.array_equal(np.bincount(ss // k, minlength=T), np.full(T, k))   # each token k times
    assert np.array_equal(eri[ss], np.arange(T * k))             # round trip to identity
    assert np.array_equal(ss[eri], np.arange(T * k))
    e_of_row = ids.reshape(-1)[ss]
    assert (np.diff(e_of_row) >= 0).all()                        # grouped by expert
    same = np.diff(e_of_row) == 0
    assert (np.diff(ss)[same] > 0).all()                         # stable inside an expert


def test_init_routing_base_offset_and_invalid():
    ids = np.array([[96, 99], [97, 40], [127, 96]], dtype=np.int32)
    r = moe.init_routing(ids, 32, 96)
    assert r["n_invalid"] == 1
    assert r["expanded_row_idx"][3] == -1
    assert list(r["tokens_per_expert"][:4]) == [2, 1, 0, 1] and r["tokens_per_expert"][31] == 1
    assert list(r["sorted_src"]) == [0, 5, 2, 1, 4]


def test_expand_rows_and_unsort_round_trip():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 8))
    ids = rng.integers(0, 6, size=(50, 1)).astype(np.int32)
    r = moe.init_routing(ids, 6)
    ex = moe.expand_rows(x, r["sorted_src"], 1)
    for rr, s in enumerate(r["sorted_src"]):
        assert np.array_equal(ex[rr], x[s])
    # [R1P] un-sort through argsort(gathered_ids_unsort) restores arrival order exactly,
    # and equals finalize with k = 1, no weights, no skip
    assert np.array_equal(moe.unsort(ex, r["sorted_src"]), x)
    assert np.array_equal(moe.finalize(ex, r["expanded_row_idx"], 1), x)


# ----------------------------------------------------------------------------- experts

def _loop_swiglu(a, w13, w2):
    I = len(w13) // 2
    H = len(w2)
    out = []
    for row in a:
        h = []
        for i in range(I):
            g = sum(row[c] * w13[i][c] for c in range(len(row)))
            u = sum(row[c] * w13[I + i][c] for c in range(len(row)))
            h.append(g / (1.0 + math.exp(-g)) * u)
        out.append([sum(h[i] * w2[o][i] for i in range(I)) for o in range(H)])
    return np.array(out)


def test_swiglu_ffn_matches_explicit_loops():
    rng = np.random.default_rng(5)
    a, w13, w2 = rng.standard_normal((3, 5)), rng.standard_normal((6, 5)), rng.standard_normal((5, 3))
    assert np.allclose(moe.swiglu_ffn(a, w13, w2), _loop_swiglu(a.tolist(), w13.tolist(), w2.tolist()),
                       rtol=1e-12, atol=1e-12)


def test_swiglu_zero_gate_or_up_gives_zero():
    rng = np.random.default_rng(6)
    a, w13, w2 = rng.standard_normal((4, 8)), rng.standard_normal((6, 8)), rng.standard_normal((8, 3))
    wz = w13.copy(); wz[:3] = 0.0                   # silu(0) = 0
    assert np.all(moe.swiglu_ffn(a, wz, w2) == 0.0)
    wz = w13.copy(); wz[3:] = 0.0                   # up projection 0
    assert np.all(moe.swiglu_ffn(a, wz, w2) == 0.0)


def test_grouped_ffn_single_group_is_dense_ffn():
    rng = np.random.default_rng(8)
    a, w13, w2 = rng.standard_normal((9, 8)), rng.standard_normal((6, 8)), rng.standard_normal((8, 3))
    y = moe.grouped_ffn(a, np.array([0, 9]), lambda e: (w13, w2))
    assert np.array_equal(y, moe.swiglu_ffn(a, w13, w2))


def test_finalize_matches_explicit_loops():
    rng = np.random.default_rng(9)
    T, k, H = 4, 2, 3
    y = rng.standard_normal((T * k, H))
    eri = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k))
    skip = rng.standard_normal((T, H))
    out = moe.finalize(y, eri, k, w, skip)
    for t in range(T):
        for h in range(H):
            ref = skip[t, h] + sum(w[t, j] * y[eri[t * k + j], h] for j in range(k))
            assert abs(out[t, h] - ref) < 1e-12


def _layer_with(cfg_name, mutate):
    cfg = configs.get(cfg_name)
    d = inputs.layer_inputs(cfg)
    mutate(d)
    return cfg, d, moe.moe_layer(d)


def test_identical_experts_make_output_independent_of_routing():
    """Sum of weights = 1, so if every expert has the same weights the routed part is
    FFN(x) whatever the routing: out = shared(x) + FFN(x)."""
    def same(d):
        d["w13"][:] = d["w13"][0]
        d["w2"][:] = d["w2"][0]
    cfg, d, r = _layer_with("p1_small_fp32", same)
    x = moe.to_f64(d["x"], cfg.act)
    ffn = moe.swiglu_ffn(x, moe.to_f64(d["w13"][0], cfg.wt), moe.to_f64(d["w2"][0], cfg.wt))
    # the float32 weights sum to 1 within a few float32 ulps
    assert np.abs(r["out"] - (r["shared"] + ffn)).max() <= 1e-6 * np.abs(ffn).max()


def test_zero_down_projection_leaves_shared_expert():
    def zero(d):
        d["w2"][:] = 0
    cfg, d, r = _layer_with("p2_prefill_bf16", zero)
    assert np.array_equal(r["out"], r["shared"])


def test_identity_ffn_combine_returns_tokens():
    """With y = expanded_x (an identity 'FFN'), the combine returns sum_j w_j x_t = x_t."""
    cfg = configs.get("p2_prefill_bf16")
    d = inputs.layer_inputs(cfg, with_experts=False)
    x = moe.to_f64(d["x"], cfg.act)
    idx, w = moe.route_topk(moe.gate_logits(x, moe.to_f64(d["w_gate"], cfg.act)).astype(np.float32),
                            None, cfg.k)
    rt = moe.init_routing(idx, cfg.E)
    y = moe.expand_rows(x, rt["sorted_src"], cfg.k)
    out = moe.finalize(y, rt["expanded_row_idx"], cfg.k, w)
    assert np.allclose(out, x, rtol=1e-6, atol=1e-6)


def test_fp8_layer_dequantized_operands_close_to_exact():
    """The fp8 layer's expanded rows dequantize to the bf16 tokens within the e4m3 bound."""
    cfg = configs.get("p5_skewed_fp8")
    d = inputs.layer_inputs(cfg)
    r = moe.moe_layer(d)
    a = moe.dequant_1x128(r["expanded_x"], r["expanded_scale"])
    x = moe.to_f64(d["x"], cfg.act)[r["sorted_src"] // cfg.k]
    assert np.all(np.abs(a - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * np.repeat(r["expanded_scale"], 128, 1))


def test_int8_quant_amax_maps_to_127_and_zero_row():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 300)).astype(np.float32)
    x[3] = 0.0
    q, s = moe.quant_per_token_int8(x)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (6,)
    assert s[3] == 1.0 and (q[3] == 0).all()
    for m in (0, 1, 2, 4, 5):
        i = int(np.argmax(np.abs(x[m])))
        assert int(q[m, i]) == (127 if x[m, i] > 0 else -127)
    assert np.abs(q.astype(np.int32)).max() <= 127


def test_int8_quant_round_half_even_closed_form():
    """amax 127 gives scale 1 and factor 1: the codes are the values rounded half to even."""
    x = np.array([[127.0, 0.5, 1.5, 2.5, -2.5, -0.49, 3.5]], dtype=np.float32)
    q, s = moe.quant_per_token_int8(x)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 0, 2, 2, -2, 0, 4]


def test_int8_quant_error_bound():
    """Round to nearest: |q * scale - x| <= scale / 2 (plus float32 rounding of x * inv)."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((50, 512)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    q, s = moe.quant_per_token_int8(x)
    err = np.abs(moe.dequant_rows(q, s) - x.astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-6)).all()


def test_int8_gemm_is_integer_product_times_scales():
    """The identity a W8A8 GEMM relies on: with per-row activation and per-channel weight
    scales, the dequantized product equals the exact integer product times s_a s_w."""
    rng = np.random.default_rng(23)
    qa = rng.integers(-127, 128, (9, 640)).astype(np.int8)
    qw = rng.integers(-127, 128, (13, 640)).astype(np.int8)
    sa = rng.uniform(0.001, 0.1, 9).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, 13).astype(np.float32)
    deq = moe.dequant_rows(qa, sa) @ moe.dequant_rows(qw, sw).T
    exact = qa.astype(np.int64) @ qw.astype(np.int64).T          # integers, no rounding
    assert np.abs(exact).max() < 2 ** 31                             # fits an int32 accumulator
    assert np.allclose(deq, exact * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :],
                       rtol=1e-13, atol=0)


def _shared_unquantized(d, x):
    """The int8 shared expert on exact activations: dequantized weights, no token or h
    quantization (a plain SwiGLU FFN)."""
    w13 = d["sh_w13"].astype(np.float64) * d["sh_w13_scale"].astype(np.float64)[:, None]
    w2 = d["sh_w2"].astype(np.float64) * d["sh_w2_scale"].astype(np.float64)[:, None]
    I = w13.shape[0] // 2
    g, u = x @ w13[:I].T, x @ w13[I:].T
    return (g / (1.0 + np.exp(-g)) * u) @ w2.T


@pytest.mark.parametrize("name", ["p6_prefill_w8a8", "p9_decode_w4a8"])
def test_shared_expert_is_w8a8_beside_int8_and_int4_experts(name):
    """[V32 §quantization strategy]: the shared expert is W8A8 whether the routed experts
    are W8A8 or W4A8.  Its weights are int8 codes with one scale per output channel, and
    its output stays within the int8 tolerance of the same FFN on exact activations; the
    quantization does change it (the error is not zero)."""
    cfg = configs.get(name)
    d = inputs.layer_inputs(cfg)
    assert cfg.sh_wt == "int8"
    assert d["sh_w13"].dtype == np.int8 and d["sh_w13"].shape == (2 * cfg.I_shared, cfg.H)
    assert d["sh_w2"].dtype == np.int8 and d["sh_w2"].shape == (cfg.H, cfg.I_shared)
    assert d["sh_w13_scale"].shape == (2 * cfg.I_shared,) and d["sh_w2_scale"].shape == (cfg.H,)
    x = moe.to_f64(d["x"], cfg.act)
    got = moe.shared_expert(x, d)
    ref = _shared_unquantized(d, x)
    rel = (np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1))
    assert rel.max() < 6e-2 and rel.max() > 1e-4, rel.max()


def test_shared_expert_stays_in_activation_dtype_elsewhere():
    for name in ("p2_prefill_bf16", "p5_skewed_fp8", "p1_small_fp32"):
        cfg = configs.get(name)
        assert cfg.sh_wt == cfg.act
        assert "sh_w13_scale" not in inputs.shared_weights(cfg)


def test_w8a8_layer_expanded_rows_and_tolerance():
    """The W8A8 layer's expanded rows are each token's per-token codes, and the layer's
    output stays within the int8 tolerance of the same layer on unquantized
    activations (only the activation and h quantizations differ)."""
    cfg = configs.get("p6_prefill_w8a8")
    d = inputs.layer_inputs(cfg)
    r = moe.moe_layer(d)
    xq, xs = moe.quant_per_token_int8(moe.to_f64(d["x"], cfg.act).astype(np.float32))
    tok = r["sorted_src"] // cfg.k
    assert np.array_equal(r["expanded_x"], xq[tok]) and np.array_equal(r["expanded_scale"], xs[tok])
    # the same layer with exact activations (dequantized int8 weights, no quantization)
    x = moe.to_f64(d["x"], cfg.act)
    a = x[tok]
    y = moe.grouped_ffn(a, r["expert_offsets"], moe.expert_weights_f64(d), quant_h=False)
    out = moe.finalize(y, r["expanded_row_idx"], cfg.k, r["topk_w"], _shared_unquantized(d, x))
    rel = (np.abs(out - r["out"]).max(axis=1) / np.abs(out).max(axis=1)).max()
    assert rel < 6e-2, rel


def test_int4_unpack_closed_form():
    """Byte i of a group: element i in the low nibble, element 8 + i in the high nibble,
    both 4-bit two's complement: 0x0F -> (-1, 0), 0x87 -> (7, -8), 0x78 -> (-8, 7)."""
    packed = np.array([[0x0F, 0x87, 0x78, 0x00, 0x11, 0xF1, 0x1F, 0x88]], dtype=np.uint8)
    codes = moe.int4_unpack(packed, 16)
    assert codes[0, :8].tolist() == [-1, 7, -8, 0, 1, 1, -1, -8]
    assert codes[0, 8:].tolist() == [0, -8, 7, 0, 1, -1, 1, -8]


def test_int4_pack_unpack_round_trip():
    """A packer written with explicit loops, then the oracle's unpack, is the identity."""
    rng = np.random.default_rng(31)
    N, K = 5, 64
    codes = rng.integers(-8, 8, (N, K))
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    for n in range(N):
        for g in range(K // 16):
            for i in range(8):
                lo = codes[n, 16 * g + i] & 0xF
                hi = codes[n, 16 * g + 8 + i] & 0xF
                packed[n, 8 * g + i] = lo | (hi << 4)
    assert np.array_equal(moe.int4_unpack(packed, K), codes.astype(np.int8))


def test_w4a8_layer_weights_and_tolerance():
    """The W4A8 workload's weights unpack to symmetric codes in [-7, 7]; its layer stays
    within the quantized-layer tolerance of the same layer on unquantized activations."""
    cfg = configs.get("p8_prefill_w4a8")
    d = inputs.layer_inputs(cfg)
    c = moe.int4_unpack(d["w13"][0], cfg.H)
    assert c.shape == (2 * cfg.I, cfg.H) and np.abs(c.astype(np.int32)).max() <= 7
    r = moe.moe_layer(d)
    x = moe.to_f64(d["x"], cfg.act)
    y = moe.grouped_ffn(x[r["sorted_src"] // cfg.k], r["expert_offsets"], moe.expert_weights_f64(d), quant_h=False)
    out = moe.finalize(y, r["expanded_row_idx"], cfg.k, r["topk_w"], _shared_unquantized(d, x))
    rel = (np.abs(out - r["out"]).max(axis=1) / np.abs(out).max(axis=1)).max()
    assert rel < 6e-2, rel


def test_gate_logits_is_plain_product():
    rng = np.random.default_rng(10)
    x, wg = rng.standard_normal((3, 4)), rng.standard_normal((5, 4))
    l = moe.gate_logits(x, wg)
    for t in range(3):
        for e in range(5):
            assert abs(l[t, e] - sum(x[t, h] * wg[e, h] for h in range(4))) < 1e-12


def test_bf16_decode_exact():
    # 0x7F7F is the largest finite bf16: (2 - 2^-7) * 2^127
    assert moe.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x7F7F], np.uint16)).tolist() == \
        [1.0, -2.0, 0.0, (2.0 - 2.0 ** -7) * 2.0 ** 127]


# ----------------------------------------------------------------------------- group -> expert mapping

def _expert_of_row(offsets, r):
    """The group that holds sorted row r, found by scanning the offsets (no search routine)."""
    for e in range(len(offsets) - 1):
        if offsets[e] <= r < offsets[e + 1]:
            return e
    raise AssertionError(f"row {r} outside every group")


def _row_swiglu(a_row, w13, w2):
    I = w13.shape[0] // 2
    g = np.array([np.dot(w13[i], a_row) for i in range(I)])
    u = np.array([np.dot(w13[I + i], a_row) for i in range(I)])
    h = g / (1.0 + np.exp(-g)) * u
    return np.array([np.dot(w2[o], h) for o in range(w2.shape[0])])


# uneven groups with an empty one in the middle and one at the end
_GROUP_SIZES = [3, 0, 5, 1, 2, 0]


def test_grouped_ffn_uses_each_groups_own_weights():
    """[MND §Roofline / GroupGEMM]: group i multiplies its own m_i rows by its own
    weights.  Distinct random weights per group and uneven group sizes (two empty
    groups): every output row equals the SwiGLU FFN of that row with the weights of
    the group whose offset range holds the row, found by scanning the offsets."""
    rng = np.random.default_rng(31)
    G, H, I = len(_GROUP_SIZES), 6, 4
    offs = np.concatenate([[0], np.cumsum(_GROUP_SIZES)]).astype(np.int32)
    a = rng.standard_normal((int(offs[-1]), H))
    w13 = rng.standard_normal((G, 2 * I, H))
    w2 = rng.standard_normal((G, H, I))
    asked = []

    def weights(e):
        asked.append(e)
        return w13[e], w2[e]
    y = moe.grouped_ffn(a, offs, weights)
    # only non-empty groups are asked for their weights, each once
    assert asked == [e for e, n in enumerate(_GROUP_SIZES) if n > 0]
    for r in range(a.shape[0]):
        e = _expert_of_row(offs, r)
        assert np.allclose(y[r], _row_swiglu(a[r], w13[e], w2[e]), rtol=1e-12, atol=1e-12), (r, e)
    # a wrong mapping is visible: the rows of group 2 differ from group 3's FFN of them
    assert not np.allclose(y[3:8], np.stack([_row_swiglu(a[r], w13[3], w2[3]) for r in range(3, 8)]))


def _fp8_dequant_by_index(codes, scale):
    """Independent dequantization: torch's e4m3fn decode times the scale of the 128x128
    block holding each element, picked by integer index arrays."""
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()
    N, K = codes.shape
    rows = np.arange(N) // 128
    cols = np.arange(K) // 128
    return v.astype(np.float64) * scale.astype(np.float64)[rows][:, cols]


def _int4_unpack_loops(packed, K):
    """Per 16 elements of K: byte i holds element i (low nibble) and 8 + i (high nibble);
    each nibble is a 4-bit two's-complement code."""
    out = np.zeros((packed.shape[0], K), dtype=np.int64)
    for n in range(packed.shape[0]):
        for b in range(K // 2):
            byte = int(packed[n, b])
            grp, i = divmod(b, 8)
            lo, hi = byte & 0xF, byte >> 4
            out[n, 16 * grp + i] = lo - 16 if lo >= 8 else lo
            out[n, 16 * grp + 8 + i] = hi - 16 if hi >= 8 else hi
    return out


@pytest.mark.parametrize("wt", ["fp8", "int8", "int4"])
def test_expert_weights_adapter_maps_each_expert(wt):
    """The per-expert float64 weights that the layer hands to the grouped FFN are expert
    e's own codes times expert e's own scales, for every quantized weight type; with
    them the grouped FFN of uneven groups (two empty) matches the per-row FFN of each
    row's own expert."""
    rng = np.random.default_rng({"fp8": 41, "int8": 42, "int4": 43}[wt])
    G, H, I = len(_GROUP_SIZES), 128, 128
    cfg = configs.get("c1_tiny_fp32", H=H, I=I, E=G, wt=wt, act="bf16")
    inp = {"cfg": cfg}
    ref = {}
    if wt == "fp8":
        # codes of finite values only (0x7F / 0xFF are NaN); scales differ per block and expert
        def codes(shape):
            c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
            return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)
        w13 = codes((G, 2 * I, H))
        w2 = codes((G, H, I))
        s13 = np.exp2(rng.integers(-12, -6, size=(G, 2 * I // 128, H // 128))).astype(np.float32)
        s2 = np.exp2(rng.integers(-12, -6, size=(G, H // 128, I // 128))).astype(np.float32)
        for e in range(G):
            ref[e] = (_fp8_dequant_by_index(w13[e], s13[e]), _fp8_dequant_by_index(w2[e], s2[e]))
    else:
        if wt == "int8":
            w13 = rng.integers(-127, 128, size=(G, 2 * I, H)).astype(np.int8)
            w2 = rng.integers(-127, 128, size=(G, H, I)).astype(np.int8)
            u13 = w13.astype(np.int64)
            u2 = w2.astype(np.int64)
        else:
            w13 = rng.integers(0, 256, size=(G, 2 * I, H // 2)).astype(np.uint8)
            w2 = rng.integers(0, 256, size=(G, H, I // 2)).astype(np.uint8)
            u13 = [_int4_unpack_loops(w13[e], H) for e in range(G)]
            u2 = [_int4_unpack_loops(w2[e], I) for e in range(G)]
        s13 = (rng.random((G, 2 * I)) * 0.01 + 0.001).astype(np.float32)
        s2 = (rng.random((G, H)) * 0.01 + 0.001).astype(np.float32)
        for e in range(G):
            ref[e] = (u13[e] * s13[e].astype(np.float64)[:, None], u2[e] * s2[e].astype(np.float64)[:, None])
    inp.update(w13=w13, w2=w2, w13_scale=s13, w2_scale=s2)
    get = moe.expert_weights_f64(inp)
    for e in range(G):
        g13, g2 = get(e)
        assert np.array_equal(g13, ref[e][0]), e
        assert np.array_equal(g2, ref[e][1]), e
    offs = np.concatenate([[0], np.cumsum(_GROUP_SIZES)]).astype(np.int32)
    a = rng.standard_normal((int(offs[-1]), H)) * 0.5
    y = moe.grouped_ffn(a, offs, get)
    for r in range(a.shape[0]):
        e = _expert_of_row(offs, r)
        want = _row_swiglu(a[r], *ref[e])
        assert np.allclose(y[r], want, rtol=1e-10, atol=1e-10 * np.abs(want).max()), (r, e)


# ----------------------------------------------------------------------------- bf16 rounding

def test_round_to_bf16_matches_library_cast():
    """Independent routine: torch's float32 -> bfloat16 cast (round to nearest even) on
    random float32 values over many binades and on exact ties."""
    rng = np.random.default_rng(51)
    v = (rng.standard_normal(300_000) * np.exp2(rng.integers(-60, 60, 300_000))).astype(np.float32)
    # exact halfway cases: low 16 bits 0x8000 with even and odd kept halves
    ties = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, ties.view(np.float32)])
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(moe.round_to_bf16(v), ref)


def test_round_to_bf16_closed_form_points():
    one_plus_tie = np.array([1.0 + 2.0 ** -8], dtype=np.float32)      # halfway between 1 and 1 + 2^-7
    assert moe.round_to_bf16(one_plus_tie)[0] == 1.0                   # even kept half
    three_tie = np.array([1.0 + 3 * 2.0 ** -8], dtype=np.float32)     # between 1 + 2^-7 and 1 + 2^-6
    assert moe.round_to_bf16(three_tie)[0] == np.float32(1.0 + 2.0 ** -6)
    assert moe.round_to_bf16(np.array([-0.0], dtype=np.float32)).view(np.uint32)[0] == 0x80000000
    bf = np.arange(0, 65536, 7, dtype=np.uint32) << 16                 # bf16 values stay put
    bf = bf.view(np.float32)[np.isfinite(bf.view(np.float32))]
    assert np.array_equal(moe.round_to_bf16(bf), bf)


def test_w8a8_h_codes_come_from_bf16_h():
    """The W8A8 down projection's input codes are the per-row int8 quantization of h
    rounded to bf16 (the precision the GPU holds h in when it takes that decision)."""
    rng = np.random.default_rng(52)
    a = rng.standard_normal((5, 32))
    w13 = rng.standard_normal((16, 32)) * 0.3
    w2 = np.eye(8)                                   # y = dequantized h
    I = 8
    g, u = a @ w13[:I].T, a @ w13[I:].T
    h = g / (1.0 + np.exp(-g)) * u
    hb = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).float().numpy()
    amax = np.abs(hb).max(axis=1)
    scale = (amax / np.float32(127)).astype(np.float32)
    codes = np.rint(hb * (np.float32(127) / amax)[:, None].astype(np.float32))
    want = codes * scale.astype(np.float64)[:, None]
    assert np.array_equal(moe.swiglu_ffn(a, w13, w2, quant_h="int8"), want)
