"""GPU parity at the full workload sizes, in the launch configuration the bench times.

The whole layer runs on the GPU at full size; the oracle then recomputes a sample of
tokens (every step of the layer is separable per token, so the sample's outputs equal
the full layer's outputs for those tokens).  Routing integers (top-k ids, counts,
offsets, both permutations) are compared bit for bit at full size, and the expanded
rows of the sampled tokens byte for byte.

The sample reaches every active expert: it holds the tokens of the first and the last
row of every work unit the grouped GEMMs cut each expert's rows into (a prefill expert
of up to one tile of rows is one unit; a hot expert is several), the first and last
token of every row slice of the shared expert, and the first and last token.  Decode
batches (at most 128 tokens) are checked on every token.  The oracle computes the
sample expert by expert: each expert's weights are drawn and converted to float64 on a
thread pool a few experts ahead of the grouped FFN that consumes them, so host memory
holds a bounded number of experts at a time.
"""
import dataclasses
from collections import deque
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import moe as O
from synth import configs, inputs
from synth.device import upload_layer
from tests.gpu_helpers import act_to_f64, check_close, empty_act, host, say, tol_of

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

ALL_TOKENS_UP_TO = 128       # batches this small are checked on every token
WORKERS = 16                 # host threads drawing / converting expert weights


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


def unit_bounds(offsets, bm):
    """First and last sorted row of every work unit of the grouped GEMM: an expert of n
    rows is cut into ceil(n / bm) near-equal slices of a multiple of 16 rows."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        n = hi - lo
        if n == 0:
            continue
        nu = -(-n // bm)
        per = (-(-n // nu) + 15) & ~15
        for i in range(nu):
            r0 = lo + i * per
            if r0 >= hi:
                break
            rows += [r0, min(r0 + per, hi) - 1]
    return rows


def slice_bounds(T, bm):
    """First and last row of each of the near-equal row slices of a dense T-row GEMM."""
    nx = -(-T // bm)
    per = (-(-T // nx) + 15) & ~15
    out = []
    for i in range(nx):
        r0 = i * per
        if r0 < T:
            out += [r0, min(r0 + per, T) - 1]
    return out


def sample_tokens(cfg, rt, block_m, shared_block_m):
    """Tokens whose rows cover every unit's first and last row (hence every active
    expert), every shared-expert slice's first and last token, and tokens 0 and T-1."""
    T, k = cfg.T, cfg.k
    if T <= ALL_TOKENS_UP_TO:
        return np.arange(T)
    rows = unit_bounds(rt["expert_offsets"], block_m)
    picks = {0, T - 1}
    picks |= {int(rt["sorted_src"][r]) // k for r in rows}
    picks |= set(slice_bounds(T, shared_block_m))
    return np.array(sorted(picks))


def block_rows(M, cfg):
    """Rows per unit of the routed expert GEMMs and of the shared expert's GEMMs, from the
    library's own launch plan (the shared expert alone is a one-group FFN over T rows)."""
    p = M.moe_layer_plan_of(M.shape_of(cfg))
    if p["shared_merged"]:
        return p["block_m"], p["block_m"]
    sh = M.moe_layer_plan_of(M.shape(cfg.T, cfg.H, 1, 1, cfg.I_shared, cfg.I_shared, cfg.act, cfg.sh_wt))
    return p["block_m"], sh["block_m"]


def weights_one(cfg, e):
    """Expert e's weights as the oracle's per-expert float64 (w13, w2)."""
    w13 = inputs.expert_w13(cfg, e)
    w2 = inputs.expert_w2(cfg, e)
    d = {"cfg": cfg}
    if cfg.wt in ("fp8", "int8", "int4"):
        d.update(w13={e: w13[0]}, w13_scale={e: w13[1]}, w2={e: w2[0]}, w2_scale={e: w2[1]})
    else:
        d.update(w13={e: w13}, w2={e: w2})
    return O.expert_weights_f64(d)(e)


class ExpertStream:
    """e -> float64 (w13, w2) for the oracle's grouped FFN, which asks for the non-empty
    experts in increasing order: each is drawn and converted on a thread pool, at most
    `ahead` experts in advance."""

    def __init__(self, cfg, experts, ahead=WORKERS):
        self.cfg = cfg
        self.order = list(experts)
        self.pool = ThreadPoolExecutor(WORKERS)
        self.pending = deque()
        self.next = 0
        for _ in range(ahead):
            self._submit()

    def _submit(self):
        if self.next < len(self.order):
            e = self.order[self.next]
            self.pending.append((e, self.pool.submit(weights_one, self.cfg, e)))
            self.next += 1

    def __call__(self, e):
        want, fut = self.pending.popleft()
        assert want == e, (want, e)
        self._submit()
        return fut.result()

    def close(self):
        self.pool.shutdown(wait=True)


def oracle_on_sample(cfg, S, logits_s, bias):
    """The oracle layer on tokens S, routed on the given float32 logits of those tokens."""
    idx, _ = O.route_topk(logits_s, bias, cfg.k)
    experts = sorted(set(idx.reshape(-1).tolist()))
    d = {"cfg": dataclasses.replace(cfg, T=len(S)), "x": inputs.tokens(cfg)[S], "w_gate": inputs.gate_weight(cfg),
         "bias": bias, **inputs.shared_weights(cfg)}
    stream = ExpertStream(cfg, experts)
    try:
        ref = O.moe_layer(d, logits32_override=logits_s, expert_weights=stream)
    finally:
        stream.close()
    assert not stream.pending and stream.next == len(experts)    # every expert drawn once
    return ref, experts


FULL = ["c1_tiny_fp32", "c2_prefill_bf16", "c4_decode_bf16", "c5_skewed_fp8", "c6_prefill_w8a8",
        "c7_decode_w8a8", "c8_decode_w4a8", "c9_decode1_bf16", "c10_decode_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_layer_sampled(M, name):
    cfg = configs.get(name)
    say("full layer", name, "upload")
    g = upload_layer(cfg)
    s = M.shape_of(cfg)
    T, E, k, H = cfg.T, cfg.E, cfg.k, cfg.H
    out = empty_act((T, H), cfg.act)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    W = M.weights_of(g)
    say("full layer", name, "run")
    M.moe_layer(s, W, g["x"], out, idx, w, logits, ws)
    torch.cuda.synchronize()
    l_gpu, i_gpu, w_gpu = host(logits), host(idx), host(w)
    bias = inputs.expert_bias(cfg)
    # routing at full size, given the GPU's float32 logits
    ridx, rw = O.route_topk(l_gpu, bias, k)
    assert np.array_equal(i_gpu, ridx)
    assert np.abs(w_gpu - rw).max() <= 1e-6
    # counting sort at full size through the same kernels
    say("full layer", name, "routing")
    R = T * k
    fp8 = cfg.wt == "fp8"
    i8 = cfg.wt in ("int8", "int4")
    ex = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.int8 if i8 else g["x"].dtype, device="cuda")
    exs = torch.empty((R, H // 128), dtype=torch.float32, device="cuda") if fp8 else \
        torch.empty(R, dtype=torch.float32, device="cuda") if i8 else None
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    ssrc = torch.empty(R, dtype=torch.int32, device="cuda")
    tpe = torch.empty(E, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    M.moe_init_routing(s, g["x"], idx, 0, ex, exs, eri, ssrc, tpe, offs, ws)
    torch.cuda.synchronize()
    rt = O.init_routing(i_gpu, E)
    assert np.array_equal(host(tpe), rt["tokens_per_expert"])
    assert np.array_equal(host(offs), rt["expert_offsets"])
    assert np.array_equal(host(eri), rt["expanded_row_idx"])
    assert np.array_equal(host(ssrc), rt["sorted_src"])
    # sampled tokens through the oracle
    bm, bm_sh = block_rows(M, cfg)
    S = sample_tokens(cfg, rt, bm or 64, bm_sh or 64)
    active = np.nonzero(rt["tokens_per_expert"])[0]
    covered = set(i_gpu[S].reshape(-1).tolist())
    assert covered >= set(active.tolist())            # every active expert has a checked row
    xs = inputs.tokens(cfg)[S]
    rows = rt["expanded_row_idx"].reshape(T, k)[S].reshape(-1)
    if fp8:
        q, sc = O.quant_1x128(O.to_f64(xs, cfg.act).astype(np.float32))
        assert np.array_equal(host(ex)[rows], np.repeat(q, k, axis=0))
        assert np.array_equal(host(exs)[rows], np.repeat(sc, k, axis=0))
    elif i8:
        q, sc = O.quant_per_token_int8(O.to_f64(xs, cfg.act).astype(np.float32))
        assert np.array_equal(host(ex)[rows], np.repeat(q, k, axis=0))
        assert np.array_equal(host(exs)[rows], np.repeat(sc, k, axis=0))
    else:
        got = host(ex)[rows]
        if cfg.act == "bf16":
            got = got.view(np.uint16)
        assert np.array_equal(got, np.repeat(xs, k, axis=0))
    del ex, exs
    say("full layer", name, f"oracle on {len(S)} of {T} tokens ({len(active)} active experts, "
        f"{len(unit_bounds(rt['expert_offsets'], bm or 64)) // 2} units)")
    ref, experts = oracle_on_sample(cfg, S, l_gpu[S], bias)
    assert len(experts) == len(active)
    check_close(f"full layer {name} ({len(S)} tokens)", act_to_f64(out, cfg.act)[S], ref["out"], tol_of(cfg))
    lerr = np.abs(l_gpu[S] - ref["logits"]).max(axis=1) / np.abs(ref["logits"]).max(axis=1)
    assert lerr.max() <= 1e-5
    del g, ws
    torch.cuda.empty_cache()


def test_ep_rank_share_full(M):
    """One expert-parallel rank at ep=8: 8192 received rows tagged with experts 96..127,
    re-routed, run through the 32 local experts, un-sorted back to arrival order; plus
    the shared expert on the 1024 local tokens.  Checked rows: the first and last row of
    every unit of every local expert, and the first and last local token of every row
    slice of the shared expert."""
    cfg = configs.get("c3_ep_rank_bf16")
    say("ep share full upload")
    g = upload_layer(cfg)
    s = M.shape_of(cfg)
    R, H, E = cfg.T, cfg.H, cfg.E
    ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    ssrc = torch.empty(R, dtype=torch.int32, device="cuda")
    tpe = torch.empty(E, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    say("ep share full run")
    # re-routing without a sorted copy: the expert GEMM reads the received rows in place
    M.moe_init_routing(s, None, g["ids"], cfg.e_base, None, None, eri, ssrc, tpe, offs, ws)
    y = empty_act((R, H), cfg.act)
    wsf = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, E, R), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn_gathered(s, E, R, g["x"], R, None, ssrc, 1, offs, g["w13"], None, g["w2"], None, y,
                               wsf)
    y_arr = empty_act((R, H), cfg.act)
    M.moe_finalize_routing(s, y, None, None, eri, y_arr)
    s_sh = M.shape(cfg.T_local, H, 1, 1, cfg.I_shared, cfg.I_shared, cfg.act, cfg.act)
    sh = empty_act((cfg.T_local, H), cfg.act)
    ws2 = torch.empty(M.moe_grouped_ffn_workspace_bytes(s_sh, 1, cfg.T_local), dtype=torch.uint8,
                      device="cuda")
    offs1 = torch.tensor([0, cfg.T_local], dtype=torch.int32, device="cuda")
    M.moe_grouped_ffn(s_sh, 1, cfg.T_local, g["x_local"], None, offs1, g["sh_w13"], None, g["sh_w2"],
                      None, sh, ws2)
    torch.cuda.synchronize()
    ids = inputs.pretagged_ids(cfg)
    rt = O.init_routing(ids, E, cfg.e_base)
    assert np.array_equal(host(tpe), rt["tokens_per_expert"])
    assert np.array_equal(host(offs), rt["expert_offsets"])
    assert np.array_equal(host(eri), rt["expanded_row_idx"])
    assert np.array_equal(host(ssrc), rt["sorted_src"])
    # un-sort is exact: arrival row a is sorted row expanded_row_idx[a]
    assert np.array_equal(host(y_arr), host(y)[rt["expanded_row_idx"]])
    bm = M.moe_layer_plan_of(M.shape(R, H, E, 1, cfg.I, cfg.I, cfg.act, cfg.wt))["block_m"]
    sorted_rows = unit_bounds(rt["expert_offsets"], bm)
    S = np.array(sorted({int(rt["sorted_src"][r]) for r in sorted_rows} | {0, R - 1}))
    assert set((ids[S, 0] - cfg.e_base).tolist()) == set(range(E))    # every local expert
    x = inputs.tokens(cfg)
    # the oracle's grouped FFN on the sampled arrival rows, routed by their own ids
    sub_rt = O.init_routing(ids[S], E, cfg.e_base)
    stream = ExpertStream(cfg, [e for e in range(E) if sub_rt["tokens_per_expert"][e] > 0])
    try:
        y_sorted = O.grouped_ffn(O.to_f64(x[S], cfg.act)[sub_rt["sorted_src"]], sub_rt["expert_offsets"], stream)
    finally:
        stream.close()
    ref = O.finalize(y_sorted, sub_rt["expanded_row_idx"], 1)
    say("ep share full", f"{len(S)} of {R} rows, {E} experts")
    check_close(f"ep rank share full routed ({len(S)} rows)", act_to_f64(y_arr, cfg.act)[S], ref, tol_of(cfg))
    L = np.array(sorted(set(slice_bounds(cfg.T_local, bm))))
    xl = inputs.local_tokens(cfg)[L]
    sref = O.swiglu_ffn(O.to_f64(xl, cfg.act), O.to_f64(inputs.shared_w13(cfg), cfg.act),
                        O.to_f64(inputs.shared_w2(cfg), cfg.act))
    check_close(f"ep rank share full shared ({len(L)} tokens)", act_to_f64(sh, cfg.act)[L], sref, tol_of(cfg))
    del g, ws, wsf
    torch.cuda.empty_cache()
