"""Bench of the MI355X MoE expert layer: tokens/s of one full layer call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]

A step is one ``moe_layer`` call (gate + top-k, init-routing, grouped SwiGLU
experts, shared expert, finalize-routing) over T tokens whose inputs are already
resident in HBM.  The default workload is the DeepSeek-V3-shaped prefill layer
(T=8192, H=7168, 256 routed experts of I=2048, top-8, one shared expert, bf16).
Every launch boundary of every timed step is marked with a HIP event on the
launch stream, which gives the per-kernel-class times and the roofline of the
dominant kernel.  The CPU oracle is timed on a bounded token sample of the same
workload.  One JSON line goes to stdout (last line).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "int8": 5000.0, "f32": 157.3}   # int8: TOP/s

METRIC = "MoE-layer tokens/sec on 1 MI355X; % MFMA peak (FFN), % HBM BW (permute)"


# ----------------------------------------------------------------------------- accounting
# [MND §Roofline / GroupGEMM]: a grouped GEMM of g groups of [m, k] x [k, n] does
# 2*g*m*k*n FLOPs and moves g*(m*k + n*k + m*n) elements; [MND §Roofline / GEMM]:
# a dense GEMM does 2*m*k*n FLOPs over m*k + n*k + m*n elements.

def group_gemm_flops(g, m, k, n):
    return 2 * g * m * k * n


def group_gemm_elems(g, m, k, n):
    return g * (m * k + n * k + m * n)


def gemm_flops(m, k, n):
    return 2 * m * k * n


def gemm_elems(m, k, n):
    return m * k + n * k + m * n


def rows_per_expert(batch, qlen, topk, ep, experts):
    """[MND §Roofline / GroupGEMM]: mean rows per expert m = batch*qlen*topk*EP/experts."""
    return batch * qlen * topk * ep / experts


def _bytes(dt):
    return {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}[dt]


def account(cfg, tpe) -> dict:
    """Algorithmic FLOPs and HBM bytes of every kernel class of one layer call.

    Bytes count what the method must move, each once: the weights of the experts
    that received rows (never of empty ones), the activations read and written.
    ``tpe`` is the realized tokens-per-expert histogram."""
    T, H, E, k, I, Is = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared
    R = int(np.sum(tpe))
    active = int(np.count_nonzero(tpe))
    ab = _bytes(cfg.act)
    fp8 = cfg.wt == "fp8"
    i8 = cfg.wt in ("int8", "int4")               # W8A8 / W4A8: row and channel scales
    wb = _bytes(cfg.wt)
    eb = 1 if (fp8 or i8) else ab                 # expanded-row bytes
    hb = 1 if (fp8 or i8) else ab
    sc_a = R * (H // 128) * 4 if fp8 else R * 4 if i8 else 0
    sc_h = R * (I // 128) * 4 if fp8 else R * 4 if i8 else 0
    sc_w13 = active * (2 * I // 128) * (H // 128) * 4 if fp8 else active * 2 * I * 4 if i8 else 0
    sc_w2 = active * (H // 128) * (I // 128) * 4 if fp8 else active * H * 4 if i8 else 0
    mfma_dt = "fp8" if fp8 else "int8" if i8 else ("f32" if cfg.act == "f32" else "bf16")
    acc = {
        "gate": dict(flops=gemm_flops(T, H, E), bytes=T * H * ab + E * H * ab + T * E * 4, dt=cfg.act),
        "topk": dict(flops=0, bytes=T * E * 4 + T * E * 4 + T * k * 8, dt=None),
        "route": dict(flops=0, bytes=R * 4 + 2 * R * 4 + E * 8, dt=None),
        "expand": dict(flops=0, bytes=T * H * ab + R * H * eb + sc_a, dt=None),
        "plan": dict(flops=0, bytes=E * 4, dt=None),
        "ffn1": dict(flops=2 * R * H * 2 * I,
                     bytes=active * 2 * I * H * wb + sc_w13 + R * H * eb + sc_a + R * I * hb + sc_h,
                     dt=mfma_dt),
        "ffn2": dict(flops=2 * R * I * H,
                     bytes=active * H * I * wb + sc_w2 + R * I * hb + sc_h + R * H * ab, dt=mfma_dt),
        "finalize": dict(flops=0, bytes=R * H * ab + 2 * T * H * ab + T * k * 8, dt=None),
    }
    # the shared expert's two GEMMs (x -> h_s, h_s -> s); W8A8 beside int8 / int4 experts:
    # int8 tokens and weights with their row and channel scales, h_s counted once as int8
    swb = _bytes(cfg.sh_wt)
    sq = cfg.sh_wt == "int8"
    xb, shb = (1, 1) if sq else (ab, ab)
    sdt = "int8" if sq else cfg.act
    acc["shared1"] = dict(flops=2 * T * H * 2 * Is,
                          bytes=2 * Is * H * swb + T * H * xb + T * Is * shb
                          + ((2 * Is + 2 * T) * 4 if sq else 0), dt=sdt)
    acc["shared2"] = dict(flops=2 * T * Is * H,
                          bytes=Is * H * swb + T * Is * shb + T * H * ab + ((H + T) * 4 if sq else 0),
                          dt=sdt)
    acc["shared"] = dict(flops=acc["shared1"]["flops"] + acc["shared2"]["flops"],
                         bytes=acc["shared1"]["bytes"] + acc["shared2"]["bytes"], dt=sdt)
    return acc


def layer_plan(cfg) -> dict:
    """The library's own launch plan for the workload's shape (moe_layer_plan_of)."""
    import moe_expert_layer_top_amd as M
    return M.moe_layer_plan_of(M.shape_of(cfg))


def shared_is_merged(cfg) -> bool:
    """moe_layer runs the shared expert as one more group of the routed grouped-GEMM
    launches (same shape and dtype, routed GEMMs not split along K)."""
    return bool(layer_plan(cfg)["shared_merged"])


def gathers_rows(cfg) -> bool:
    """bf16 layers never write the expanded rows: the first expert GEMM reads each routed
    row from x through the sort's slot order."""
    return bool(layer_plan(cfg)["rows_gathered"])


def launch_accounting(cfg, acc: dict) -> dict:
    """Work per timed launch class: with the shared expert merged, the ffn1 / ffn2
    launches also do the shared expert's two GEMMs and there is no shared stage; with
    gathered rows ffn1 reads T token rows instead of R expanded rows, and the expand
    stage writes nothing (bf16) or each token's codes once (fp8 / int8 activations:
    x read, T x H codes and their scales written)."""
    out = {k: dict(v) for k, v in acc.items() if k not in ("shared1", "shared2")}
    if gathers_rows(cfg):
        T, H, R = cfg.T, cfg.H, cfg.R
        ab = _bytes(cfg.act)
        fp8 = cfg.wt == "fp8"
        q = fp8 or cfg.wt in ("int8", "int4")
        eb = 1 if q else ab
        sc_row = (H // 128) * 4 if fp8 else 4 if q else 0     # activation scale bytes per row
        out["expand"] = dict(flops=0, bytes=(T * H * ab + T * H * eb + T * sc_row) if q else 0, dt=None)
        out["ffn1"]["bytes"] += (T - R) * (H * eb + sc_row)
    if shared_is_merged(cfg):
        for k, sk in (("ffn1", "shared1"), ("ffn2", "shared2")):
            out[k] = dict(flops=out[k]["flops"] + acc[sk]["flops"],
                          bytes=out[k]["bytes"] + acc[sk]["bytes"], dt=out[k]["dt"])
        del out["shared"]
    return out


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` measured by the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes recorded in profiles/<stage>_<workload>_hbm_traffic.txt, scaled by the copy
    calibration; None when there is no record or when the kernel sources listed in it
    have changed since (the sha256 no longer matches), so a stale count is never shown."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        rec[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in rec["sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def roofline_entry(acc_k: dict, ms: float) -> dict:
    t = ms / 1e3
    gbs = acc_k["bytes"] / t / 1e9 if t > 0 else 0.0
    e = {"ms": ms, "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    if acc_k["flops"]:
        peak = PEAK_TFLOPS[acc_k["dt"]]
        tf = acc_k["flops"] / t / 1e12 if t > 0 else 0.0
        e.update({"TFLOP/s": tf, "mfma_frac": tf / peak,
                  "bound": "mfma" if acc_k["flops"] / (peak * 1e12) > acc_k["bytes"] / (PEAK_HBM_GBS * 1e9)
                  else "hbm"})
    else:
        e["bound"] = "hbm"
    return e


# ----------------------------------------------------------------------------- GPU run

def run_gpu(cfg, steps, warmup, two_streams=True, flush=False):
    import torch

    import moe_expert_layer_top_amd as M
    from synth.device import upload_layer

    dev = torch.device("cuda:0")
    t0 = time.time()
    g = upload_layer(cfg, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    s = M.shape_of(cfg)
    act_dt = torch.float32 if cfg.act == "f32" else torch.int16
    out = torch.empty((cfg.T, cfg.H), dtype=act_dt, device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    W = M.weights_of(g)
    nev = len(M.EV_NAMES)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for row in events:              # create the underlying HIP events
        for e in row:
            e.record(stream)
    # the shared expert's own launches (when it is not a group of the routed launches)
    # go to a second stream, where they overlap the routing kernels
    side = torch.cuda.Stream() if two_streams else None
    for _ in range(warmup):
        M.moe_layer_overlap(s, W, g["x"], out, idx, w, logits, ws, side)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        M.moe_layer_profiled(s, W, g["x"], out, idx, w, logits, ws, events[i], side=side)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    stage_ms = {}
    for j in range(1, nev):
        stage_ms[M.EV_NAMES[j]] = float(np.mean([events[i][j - 1].elapsed_time(events[i][j])
                                                 for i in range(steps)]))
    tpe = np.bincount(idx.cpu().numpy().reshape(-1), minlength=cfg.E)
    cold_ms = None
    if flush:
        # cold layers: before each one, a 512 MB write evicts the L2s and the 256 MB
        # last-level cache, so nothing of the previous layer is re-read from cache; each
        # layer is timed alone by its own start/finalize events
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        lay = []
        for i in range(steps):
            scratch.zero_()
            M.moe_layer_profiled(s, W, g["x"], out, idx, w, logits, ws, events[i], side=side)
            torch.cuda.synchronize()
            lay.append(events[i][0].elapsed_time(events[i][nev - 1]))
        cold_ms = float(np.median(lay))
        del scratch
    return dict(total_ms=total_ms, wall_s=wall, stage_ms=stage_ms, tpe=tpe, setup_s=setup_s, cold_ms=cold_ms,
                logits=logits.cpu().numpy(), idx=idx.cpu().numpy())


EP_STAGES = ["route", "ffn", "unsort", "shared"]


def run_gpu_ep(cfg, steps, warmup):
    """One expert-parallel rank's share (pretagged rows): the re-routing sort
    (moe_init_routing, k = 1, no row copy), the grouped experts over the rank's experts
    reading the received rows in place through the sort's slot order
    (moe_grouped_ffn_gathered), the un-sort back to arrival order (moe_finalize_routing,
    k = 1) and
    the shared expert on the rank's local tokens (moe_grouped_ffn, G = 1).  The shared
    expert needs none of the routed work, so it runs on a second stream beside it
    ([MND §Computation and communication overlap], Dispatch Overlap); the stages are
    marked by HIP events on the main stream ("shared" is the wait for the side stream)."""
    import torch

    import moe_expert_layer_top_amd as M
    from synth.device import upload_layer

    dev = torch.device("cuda:0")
    t0 = time.time()
    g = upload_layer(cfg, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    s = M.shape_of(cfg)
    R, H, E = cfg.T, cfg.H, cfg.E
    act_dt = torch.float32 if cfg.act == "f32" else torch.int16
    ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    eri = torch.empty(R, dtype=torch.int32, device=dev)
    ssrc = torch.empty(R, dtype=torch.int32, device=dev)
    tpe = torch.empty(E, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    y = torch.empty((R, H), dtype=act_dt, device=dev)
    y_arr = torch.empty((R, H), dtype=act_dt, device=dev)
    wsf = torch.empty(M.moe_grouped_ffn_workspace_bytes(s, E, R), dtype=torch.uint8, device=dev)
    s_sh = M.shape(cfg.T_local, H, 1, 1, cfg.I_shared, cfg.I_shared, cfg.act, cfg.act)
    sh = torch.empty((cfg.T_local, H), dtype=act_dt, device=dev)
    ws2 = torch.empty(M.moe_grouped_ffn_workspace_bytes(s_sh, 1, cfg.T_local), dtype=torch.uint8, device=dev)
    offs1 = torch.tensor([0, cfg.T_local], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def step(ev=None):
        mark = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        mark(0)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            M.moe_grouped_ffn(s_sh, 1, cfg.T_local, g["x_local"], None, offs1, g["sh_w13"], None,
                              g["sh_w2"], None, sh, ws2)
        M.moe_init_routing(s, None, g["ids"], cfg.e_base, None, None, eri, ssrc, tpe, offs, ws)
        mark(1)
        M.moe_grouped_ffn_gathered(s, E, R, g["x"], R, None, ssrc, 1, offs, g["w13"], None, g["w2"],
                                   None, y, wsf)
        mark(2)
        M.moe_finalize_routing(s, y, None, None, eri, y_arr)
        mark(3)
        stream.wait_stream(side)
        mark(4)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(events[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    stage_ms = {name: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(steps)]))
                for j, name in enumerate(EP_STAGES)}
    return dict(total_ms=start.elapsed_time(end), wall_s=wall, stage_ms=stage_ms,
                tpe=tpe.cpu().numpy(), setup_s=setup_s)


def account_ep(cfg, tpe) -> dict:
    """Algorithmic FLOPs and bytes of the rank-share stages (as account())."""
    T, H, E, I, Is, TL = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_shared, cfg.T_local
    ab = _bytes(cfg.act)
    active = int(np.count_nonzero(tpe))
    R = int(np.sum(tpe))
    return {
        "route": dict(flops=0, bytes=T * 4 + 2 * R * 4 + E * 8, dt=None),   # ids in, maps out
        "ffn": dict(flops=2 * R * H * 2 * I + 2 * R * I * H,
                    bytes=active * 3 * I * H * ab + R * H * ab + 2 * R * I * ab + R * H * ab, dt=cfg.act),
        "unsort": dict(flops=0, bytes=2 * R * H * ab + R * 4, dt=None),
        "shared": dict(flops=2 * TL * H * 2 * Is + 2 * TL * Is * H,
                       bytes=3 * Is * H * ab + 2 * TL * H * ab + 2 * TL * Is * ab, dt=cfg.act),
    }


EP_SIDE = ("shared",)   # stages whose time is a wait for the side stream (no rates)


# ----------------------------------------------------------------------------- CPU oracle baseline

def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def _expert_f64(cfg, e):
    """Expert e's float64 (w13, w2) through the oracle's own per-expert adapter."""
    from oracle import moe as O
    from synth import inputs
    w13, w2 = inputs.expert_w13(cfg, e), inputs.expert_w2(cfg, e)
    d = {"cfg": cfg}
    if cfg.wt in ("fp8", "int8", "int4"):
        d.update(w13={e: w13[0]}, w13_scale={e: w13[1]}, w2={e: w2[0]}, w2_scale={e: w2[1]})
    else:
        d.update(w13={e: w13}, w2={e: w2})
    return O.expert_weights_f64(d)(e)


def _ffn_sample(cfg, offsets, a_rows_of, target_s):
    """Time the oracle's grouped FFN on the whole row sets of m active experts spread
    evenly over the expert ids (the realized rows per expert of the full routing), m
    grown until the timed part takes about target_s or the experts' float64 weights reach
    ~12 GB; each expert's float64 weights are made beforehand (resident weights, as on
    the GPU).  Returns (seconds, rows timed, experts timed)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import moe as O
    n = np.diff(offsets)
    active = [int(e) for e in np.nonzero(n)[0]]
    # at most ~12 GB of float64 weights at a time
    m_max = max(1, min(len(active), int(12e9 // (3 * cfg.I * cfg.H * 8))))
    m = min(4, m_max)
    while True:
        # experts spread evenly over the active ones (hot and cold alike in skewed loads)
        chosen = [active[int(i * len(active) / m)] for i in range(m)]
        with ThreadPoolExecutor(16) as ex:
            wts = dict(zip(chosen, ex.map(lambda e: _expert_f64(cfg, e), chosen)))
        rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in chosen])
        a = a_rows_of(rows)
        sub_offs = np.concatenate([[0], np.cumsum([n[e] for e in chosen])])
        t0 = time.perf_counter()
        O.grouped_ffn(a, sub_offs, lambda j: wts[chosen[j]],
                      quant_h="int8" if cfg.wt in ("int8", "int4") else cfg.wt == "fp8")
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or m == m_max:
            return dt, int(rows.size), m
        m = min(m_max, max(m + 1, int(m * min(4.0, target_s / max(dt, 1e-3)))))
        del wts, a


def cpu_baseline(cfg, target_s=15.0):
    """Time the oracle (as it stands) stage by stage on a bounded sample of the workload
    and scale each stage to the full layer: the gate projection, the router, the
    routing sort and the row expansion over all T tokens; the grouped SwiGLU experts on
    the whole row sets of m experts (scaled by rows); the shared expert and the combine
    on a sample of tokens (scaled by tokens).  Weights are converted to float64 before
    the timers start, as the GPU's are resident in HBM."""
    from oracle import moe as O
    from synth import inputs

    if cfg.pretagged:
        return cpu_baseline_ep(cfg, target_s)
    T, k = cfg.T, cfg.k
    x_all = inputs.tokens(cfg)
    wg64 = O.to_f64(inputs.gate_weight(cfg), cfg.act)
    bias = inputs.expert_bias(cfg)
    fp8 = cfg.wt == "fp8"
    q8 = cfg.wt in ("int8", "int4")
    stages = {}
    t0 = time.perf_counter()
    x64 = O.to_f64(x_all, cfg.act)
    l32 = O.gate_logits(x64, wg64).astype(np.float32)
    stages["gate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx, w = O.route_topk(l32, bias, k)
    rt = O.init_routing(idx, cfg.E)
    stages["router+sort"] = time.perf_counter() - t0
    # the expert inputs of every row: the tokens themselves, or their fp8 / int8 codes
    t0 = time.perf_counter()
    if fp8:
        q, sc = O.quant_1x128(x64.astype(np.float32))
        a_rows_of = lambda r: O.dequant_1x128(O.expand_rows(q, rt["sorted_src"][r], k),   # noqa: E731
                                              O.expand_rows(sc, rt["sorted_src"][r], k))
    elif q8:
        q, sc = O.quant_per_token_int8(x64.astype(np.float32))
        a_rows_of = lambda r: O.dequant_rows(O.expand_rows(q, rt["sorted_src"][r], k),    # noqa: E731
                                             O.expand_rows(sc[:, None], rt["sorted_src"][r], k)[:, 0])
    else:
        a_rows_of = lambda r: O.expand_rows(x64, rt["sorted_src"][r], k)                 # noqa: E731
    stages["quant"] = time.perf_counter() - t0
    R = int(rt["expert_offsets"][-1])
    t_ffn, rows_s, m = _ffn_sample(cfg, rt["expert_offsets"], a_rows_of, target_s * 0.6)
    stages["experts (scaled)"] = t_ffn * R / rows_s
    # expansion of every row (a gather of R rows), timed on the sampled experts' rows
    t0 = time.perf_counter()
    a_rows_of(np.arange(min(R, rows_s)))
    stages["expand (scaled)"] = (time.perf_counter() - t0) * R / min(R, rows_s)
    # shared expert and combine on a token sample
    inp = {"cfg": cfg, **inputs.shared_weights(cfg)}
    shw = O.shared_weights_f64(inp)
    ts = min(T, max(64, rows_s // k))
    t0 = time.perf_counter()
    sh = O.shared_expert(x64[:ts], inp, shw)
    stages["shared (scaled)"] = (time.perf_counter() - t0) * T / ts
    y = np.zeros((ts * k, cfg.H))
    eri = np.arange(ts * k, dtype=np.int32)
    t0 = time.perf_counter()
    O.finalize(y, eri, k, w[:ts], sh)
    stages["combine (scaled)"] = (time.perf_counter() - t0) * T / ts
    total = sum(stages.values())
    return {"value": T / total, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "seconds_per_layer": total,
            "stages_s": {kk: round(v, 3) for kk, v in stages.items()},
            "sample": f"float64 oracle on {cfg.name}: gate, router, routing sort and activation "
                      f"quantization over all {T} tokens; the grouped experts on the whole row sets of "
                      f"{m} experts ({rows_s} of {R} rows, scaled by rows); shared expert and combine on "
                      f"{ts} tokens (scaled by tokens); weights in float64 before timing"}


def cpu_baseline_ep(cfg, target_s):
    """The oracle on a rank share, stage by stage: the re-routing sort over all received
    rows; the grouped experts on the whole row sets of m local experts (scaled by rows);
    the un-sort and the shared expert on samples (scaled); local tokens per second."""
    from oracle import moe as O
    from synth import inputs

    ids = inputs.pretagged_ids(cfg)
    x_all = inputs.tokens(cfg)
    xl_all = inputs.local_tokens(cfg)
    stages = {}
    t0 = time.perf_counter()
    rt = O.init_routing(ids, cfg.E, cfg.e_base)
    stages["re-route"] = time.perf_counter() - t0
    R = int(rt["expert_offsets"][-1])

    def a_rows_of(r):
        src = rt["sorted_src"][r]
        return O.to_f64(x_all[src], cfg.act)
    t_ffn, rows_s, m = _ffn_sample(cfg, rt["expert_offsets"], a_rows_of, target_s * 0.6)
    stages["experts (scaled)"] = t_ffn * R / rows_s
    y = np.zeros((rows_s, cfg.H))
    t0 = time.perf_counter()
    O.unsort(y, np.random.default_rng(0).permutation(rows_s))
    stages["un-sort (scaled)"] = (time.perf_counter() - t0) * R / rows_s
    inp = {"cfg": cfg, **inputs.shared_weights(cfg)}
    shw = O.shared_weights_f64(inp)
    tl = min(cfg.T_local, max(64, rows_s // 8))
    t0 = time.perf_counter()
    O.shared_expert(O.to_f64(xl_all[:tl], cfg.act), inp, shw)
    stages["shared (scaled)"] = (time.perf_counter() - t0) * cfg.T_local / tl
    total = sum(stages.values())
    return {"value": cfg.T_local / total, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "seconds_per_layer": total,
            "stages_s": {kk: round(v, 3) for kk, v in stages.items()},
            "sample": f"float64 oracle on {cfg.name}: re-routing sort over all {cfg.T} received rows; the "
                      f"grouped experts on the whole row sets of {m} of the {cfg.E} local experts "
                      f"({rows_s} of {R} rows, scaled by rows); un-sort and shared expert on samples "
                      f"(scaled); weights in float64 before timing"}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of `nbytes`: reads and writes exactly nbytes per
    launch, so the FETCH_SIZE / WRITE_SIZE counters of this launch give the factor
    between counter units and bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)


def rows_histogram(tpe) -> dict:
    """Realized routed rows per expert, as the number of experts in each row-count bucket."""
    edges = [(0, 0), (1, 2), (3, 8), (9, 32), (33, 128), (129, 512), (513, 2048), (2049, 1 << 40)]
    out = {}
    for lo, hi in edges:
        key = str(lo) if lo == hi else (f"{lo}-{hi}" if hi < 1 << 40 else f">={lo}")
        out[key] = int(np.count_nonzero((tpe >= lo) & (tpe <= hi)))
    return out


def copy_ceiling(nbytes=1 << 30, reps=5) -> dict:
    """The achievable HBM rate beside the nominal 8 TB/s: a device-to-device copy of
    `nbytes` (it reads nbytes and writes nbytes) timed with HIP events on the current
    stream, after the bench's timed region; GB/s = 2 * nbytes / mean time per copy."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": 2 * nbytes / (ms / 1e3) / 1e9, "bytes_per_copy": 2 * nbytes, "ms_per_copy": ms,
            "note": "device-to-device copy of 1 GiB (read + write bytes), after the timed region"}


# ----------------------------------------------------------------------------- main

DEFAULT_ALSO = "c5_skewed_fp8,c3_ep_rank_bf16,c4_decode_bf16"


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2_prefill_bf16")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed after the main one in the same run and "
                         f"reported under 'other_workloads' (default with the c2 layer: {DEFAULT_ALSO}; "
                         "'none' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--flush", action="store_true",
                    help="also time layers one by one after a 512 MB cache-evicting write (cold_ms_per_step)")
    ap.add_argument("--one-stream", action="store_true",
                    help="run the shared expert's own launches on the layer's stream")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (scales the HBM byte counters)")
    return ap.parse_args(argv)


def main():
    args = parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this layer is one GPU's share of tokens and "
              f"experts, with no cross-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    from synth import configs
    cfg = configs.get(args.config)
    line = ep_line(cfg, args.steps, args.warmup) if cfg.pretagged else layer_line(cfg, args)
    also = args.also if args.also is not None else (DEFAULT_ALSO if args.config == "c2_prefill_bf16" else "none")
    others = [n for n in also.split(",") if n and n != "none" and n != cfg.name]
    if others:
        import torch
        line["other_workloads"] = {}
        for name in others:
            torch.cuda.empty_cache()
            ocfg = configs.get(name)
            steps, warm = min(args.steps, 10), min(args.warmup, 2)
            o = ep_line(ocfg, steps, warm) if ocfg.pretagged else layer_line(ocfg, args, steps, warm)
            line["other_workloads"][name] = summary_of(o)
    line["hbm_copy"] = copy_ceiling()
    if line["roofline"]["unit"] == "GB/s":
        line["roofline"]["frac_of_copy"] = line["roofline"]["achieved"] / line["hbm_copy"]["GB/s"]
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def summary_of(line: dict) -> dict:
    """The figures of a bench line that another workload's entry carries."""
    roof = line["roofline"]
    out = {"ms_per_step": line["ms_per_step"], "tokens_per_s": line["value"], "steps": line["steps"],
           "dtype": line["dtype"], "config": line["config"],
           "roofline": {k: roof[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic",
                                              "mfma_frac", "traffic_ratio", "rereads_flag") if k in roof},
           "ffn_mfma_frac": line["ffn_mfma_frac"], "permute_combine_hbm_frac": line["permute_combine_hbm_frac"],
           "kernels_ms": {k: round(v["ms"], 4) for k, v in line["kernels"].items()}}
    for k in ("rows_per_s", "ffn_mfma_frac_bf16_peak", "rows_per_expert_histogram"):
        if k in line:
            out[k] = line[k]
    return out


def layer_line(cfg, args, steps=None, warmup=None) -> dict:
    """Bench line (without the CPU baseline) of a gated layer workload."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    r = run_gpu(cfg, steps, warmup, two_streams=not args.one_stream, flush=args.flush)
    ms = r["total_ms"] / steps
    tokens = cfg.shared_rows
    acc = launch_accounting(cfg, account(cfg, r["tpe"]))
    kern = {name: roofline_entry(acc[name], r["stage_ms"][name]) for name in acc}
    if shared_is_merged(cfg):
        kern["shared"] = {"ms": r["stage_ms"]["shared"], "merged_into": ["ffn1", "ffn2"]}
        shared_mode = "merged into the routed launches"
    elif not args.one_stream:
        # the shared stage is only the wait for the side stream: no rates for it
        kern["shared"] = {"ms": r["stage_ms"]["shared"], "side_stream": True,
                          "note": "ms = time the layer's stream waited for the shared expert"}
        shared_mode = "side stream"
    else:
        shared_mode = "in line"
    dom = max(("ffn1", "ffn2"), key=lambda n: r["stage_ms"][n])
    dk = kern[dom]
    if dk["bound"] == "mfma":
        achieved = acc[dom]["flops"] / (r["stage_ms"][dom] / 1e3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved,
                "peak": PEAK_TFLOPS[acc[dom]["dt"]], "unit": "TOP/s" if acc[dom]["dt"] == "int8" else "TFLOP/s"}
    else:
        achieved = acc[dom]["bytes"] / (r["stage_ms"][dom] / 1e3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name, dom)
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["algorithmic_bytes"] = acc[dom]["bytes"]
    roof["mfma_frac"] = dk.get("mfma_frac")
    if roof["traffic"] is not None:
        # measured over algorithmic bytes; above 1.2 means panels or rows are read again
        roof["traffic_ratio"] = roof["traffic"] / roof["algorithmic_bytes"]
        roof["rereads_flag"] = roof["traffic_ratio"] > 1.2
    # expand is an empty stage when the rows are gathered inside ffn1
    permute_ms = r["stage_ms"]["expand"] + r["stage_ms"]["finalize"]
    permute_bytes = acc["expand"]["bytes"] + acc["finalize"]["bytes"]
    ffn_ms = r["stage_ms"]["ffn1"] + r["stage_ms"]["ffn2"]
    ffn_flops = acc["ffn1"]["flops"] + acc["ffn2"]["flops"]
    line = {
        "metric": METRIC,
        "value": tokens * 1e3 / ms,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if cfg.wt == "int4" else cfg.wt if cfg.wt in ("fp8", "int8") else cfg.act,
        "data": "synthetic (seeded generators of synth/inputs.py)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_shared, "act": cfg.act, "wt": cfg.wt},
        "roofline": roof,
        "ffn_mfma_frac": ffn_flops / (ffn_ms / 1e3) / 1e12 / PEAK_TFLOPS[acc["ffn1"]["dt"]],
        # fp8 experts: the same FFN rate against the bf16 peak as well
        "ffn_mfma_frac_bf16_peak": ffn_flops / (ffn_ms / 1e3) / 1e12 / PEAK_TFLOPS["bf16"],
        "permute_combine_hbm_frac": permute_bytes / (permute_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "kernels": kern,
        "shared_expert": shared_mode,
        "active_experts": int(np.count_nonzero(r["tpe"])),
        "max_rows_per_expert": int(r["tpe"].max()),
        "rows_per_expert_histogram": rows_histogram(r["tpe"]),
        "wall_ms_per_step": r["wall_s"] * 1e3 / steps,
        "cold_ms_per_step": r["cold_ms"],
        "setup_s": r["setup_s"],
    }
    return line



def ep_line(cfg, steps, warmup) -> dict:
    """Bench line (without the CPU baseline) of an expert-parallel rank share: value =
    local tokens/s; the received rows/s beside it."""
    r = run_gpu_ep(cfg, steps, warmup)
    ms = r["total_ms"] / steps
    acc = account_ep(cfg, r["tpe"])
    kern = {name: roofline_entry(acc[name], r["stage_ms"][name]) for name in acc if name not in EP_SIDE}
    kern["shared"] = {"ms": r["stage_ms"]["shared"], "side_stream": True,
                      "note": "ms = time the main stream waited for the shared expert"}
    dk = kern["ffn"]
    if dk["bound"] == "mfma":
        roof = {"kernel": "ffn (plan + GEMM1 + GEMM2 of moe_grouped_ffn_gathered)", "bound": "mfma",
                "achieved": acc["ffn"]["flops"] / (r["stage_ms"]["ffn"] / 1e3) / 1e12,
                "peak": PEAK_TFLOPS[acc["ffn"]["dt"]], "unit": "TFLOP/s"}
    else:
        roof = {"kernel": "ffn (plan + GEMM1 + GEMM2 of moe_grouped_ffn_gathered)", "bound": "hbm",
                "achieved": acc["ffn"]["bytes"] / (r["stage_ms"]["ffn"] / 1e3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name, "ffn")
    roof["traffic_unit"] = "HBM bytes per ffn stage (both expert GEMMs; rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["algorithmic_bytes"] = acc["ffn"]["bytes"]
    roof["mfma_frac"] = dk.get("mfma_frac")
    if roof["traffic"] is not None:
        roof["traffic_ratio"] = roof["traffic"] / roof["algorithmic_bytes"]
        roof["rereads_flag"] = roof["traffic_ratio"] > 1.2
    perm_ms = r["stage_ms"]["route"] + r["stage_ms"]["unsort"]
    perm_bytes = acc["route"]["bytes"] + acc["unsort"]["bytes"]
    line = {
        "metric": METRIC,
        "value": cfg.T_local * 1e3 / ms,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic (seeded generators of synth/inputs.py)",
        "config": {"workload": cfg.name, "rows": cfg.T, "T_local": cfg.T_local, "H": cfg.H, "E": cfg.E,
                   "e_base": cfg.e_base, "I": cfg.I, "I_shared": cfg.I_shared, "act": cfg.act, "wt": cfg.wt},
        "rows_per_s": cfg.T * 1e3 / ms,
        "roofline": roof,
        "ffn_mfma_frac": dk.get("mfma_frac"),
        "permute_combine_hbm_frac": perm_bytes / (perm_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "kernels": kern,
        "wall_ms_per_step": r["wall_s"] * 1e3 / steps,
        "setup_s": r["setup_s"],
    }
    return line



if __name__ == "__main__":
    main()
