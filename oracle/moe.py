"""CPU oracle of the DeepSeek-V3/R1-style MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``.  The GPU library never calls it, and this module shares no code
with the GPU path: it reads the same input bytes and nothing else.

Every step is written as its plain definition, in float64 unless the step's
definition fixes another precision (the router's float32 scores, the fp8
quantizer's float32 arithmetic).  Library primitives (matmul, stable argsort,
bincount) serve as single steps; there is no blocking, fusion or reordering.

Sources (cited by short name throughout):

* [MND] page "Lower latency and higher throughput with multi-node DeepSeek
  deployment" (Perplexity, 2025-04-18).
* [R1P] page "CANN/cann-recipes-infer: DeepSeek-R1 prefill optimization"
  (DeepSeek-R1 prefill on Atlas A3).
* [V32] page "NPU DeepSeek-V3.2-Exp inference optimization practice" (W8A8: static
  per-channel int8 weights, dynamic per-token int8 activations).
* The workload statement that accompanies them fixes what the pages leave
  open: sigmoid gate scores, top-k renormalized to sum to 1, SwiGLU experts
  with gate/up/down projections.

Readings where the pages are silent (each one is also listed in the design
notes): ties in the top-k go to the lower expert id; slots are flattened
token-major (s = t*k + j); rows of one expert keep ascending s; no routed
scaling factor; the expert bias is added to the logits and used for both
selection and weights; invalid expert ids are dropped from the routing and
reported; fp8 is OCP e4m3fn (max 448, round-to-nearest-even, saturating).  The
router's variants (route_grouped: group-limited selection, softmax weights, no
renormalization, a routed scaling factor) state their readings where they are defined.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0
QBLOCK = 128

# --------------------------------------------------------------------------- formats


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> exact float64 value (bf16 is the upper half of a float32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(v32: np.ndarray) -> np.ndarray:
    """float32 -> the nearest bf16 value (ties to even), returned as float32.

    bf16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of a float32,
    so rounding works on the float32 bit pattern: the low 16 bits are dropped after
    adding half a bf16 step (0x7FFF) plus the kept half's last bit (ties to even).
    Finite inputs only (the GPU path never rounds a NaN or an infinity here).
    """
    x = np.asarray(v32, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("the oracle rounds finite values only")
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def fp8_e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN code -> float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); the all-ones pattern S.1111.111 is NaN and there are
    no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    return _fp8_decode_table()[np.asarray(codes, dtype=np.uint8)]


_FP8_DECODE = []


def _fp8_decode_table() -> np.ndarray:
    """The decode of every one of the 256 codes (the formula above, evaluated once); a
    tensor of codes is decoded by indexing it."""
    if not _FP8_DECODE:
        c = np.arange(256, dtype=np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        exp = (c >> 3) & 0xF
        man = (c & 0x7).astype(np.float64)
        val = np.where(exp == 0, man / 8.0 * 2.0 ** -6,
                       (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0))
        val = np.where((c & 0x7F) == 0x7F, np.nan, val)
        _FP8_DECODE.append(sign * val)
    return _FP8_DECODE[0]


def fp8_e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3FN code, round to nearest (ties to even), saturating.

    Works from the value, not from bit tricks: for |v| the representable grid
    spacing is 2^(e-3) inside binade [2^e, 2^(e+1)) for e >= -6, and 2^-9 for the
    subnormal range below 2^-6.  |v| is divided by that spacing (exact: a power of
    two), rounded half-to-even with np.rint, and scaled back.  Results above 448
    saturate to 448.  NaN inputs are rejected.
    """
    x = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN cannot be encoded by the oracle")
    a = np.abs(x)
    _, ex = np.frexp(a)                         # a = m * 2^ex, m in [0.5, 1): binade 2^(ex-1)
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)
    spacing = np.exp2(e - 3.0)
    q = np.rint(a / spacing) * spacing          # round half to even on the grid
    q = np.minimum(q, FP8_MAX)                   # saturate
    # back to a code
    _, qex = np.frexp(q)
    qe = qex.astype(np.float64) - 1.0
    sub = q < 2.0 ** -6
    exp_field = np.where(sub, 0, qe + 7).astype(np.int64)
    man_field = np.where(sub, np.rint(q / 2.0 ** -9),
                         np.rint((q / np.exp2(qe) - 1.0) * 8.0)).astype(np.int64)
    code = (exp_field << 3) | man_field
    code = np.where(np.signbit(x), code | 0x80, code)   # -0 and tiny negatives keep the sign
    return code.astype(np.uint8)


def quant_1x128(x32: np.ndarray):
    """Dynamic activation quantization to fp8 with one fp32 scale per 1x128 vector.

    [MND §Quantization]: activations are scaled per 128-element vector along the
    reduction dimension, computed on the fly; the scale tensor of an [M, K]
    activation has shape M x ceil(K/128).  Arithmetic (all float32):
    amax = max|x| over the block, scale = amax / 448, q = e4m3(x * (448 / amax));
    a block of zeros gets scale 1 and codes 0.
    """
    x = np.asarray(x32, dtype=np.float32)
    M, K = x.shape
    assert K % QBLOCK == 0
    xb = x.reshape(M, K // QBLOCK, QBLOCK)
    amax = np.abs(xb).max(axis=2)                                   # float32, exact
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(FP8_MAX)).astype(np.float32)
    inv = (np.float32(FP8_MAX) / safe).astype(np.float32)
    v = (xb * inv[:, :, None]).astype(np.float32)
    q = fp8_e4m3fn_encode(v)
    q = np.where(zero[:, :, None], np.uint8(0), q).astype(np.uint8)
    return q.reshape(M, K), scale


def dequant_1x128(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    M, K = q.shape
    v = fp8_e4m3fn_decode(q).reshape(M, K // QBLOCK, QBLOCK)
    return (v * scale.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_block128(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Static weight dequantization: one fp32 scale per 128x128 tile of an [N, K] weight
    ([MND §Quantization]: weight scale shape ceil(K/128) x ceil(N/128))."""
    N, K = q.shape
    v = fp8_e4m3fn_decode(q).reshape(N // QBLOCK, QBLOCK, K // QBLOCK, QBLOCK)
    return (v * scale.astype(np.float64)[:, None, :, None]).reshape(N, K)


INT8_MAX = 127.0


def quant_per_token_int8(x32: np.ndarray):
    """Dynamic per-token int8 quantization, the A8 of W8A8 ([V32 §quantization
    strategy]: activations are quantized per token on the fly, weights per channel
    offline).  Arithmetic, all float32: amax = max|x| over the row, scale = amax / 127,
    q = round-half-even(x * (127 / amax)) clipped to [-127, 127]; a row of zeros gets
    scale 1 and codes 0.  Returns (codes int8 [M, K], scale float32 [M]).
    """
    x = np.asarray(x32, dtype=np.float32)
    amax = np.abs(x).max(axis=1)                                     # float32, exact
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(INT8_MAX)).astype(np.float32)
    inv = (np.float32(INT8_MAX) / safe).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(v), -INT8_MAX, INT8_MAX).astype(np.int8)
    q[zero] = 0
    return q, scale


def dequant_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """int8 codes with one fp32 scale per row -> float64 (per-token activations, and
    per-output-channel weights [N, K] with one scale per row N)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def int4_unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """Packed int4 weights [N, K/2] bytes -> int8 codes [N, K] in [-8, 7].

    Layout (a storage convention of the W4A8 weights): K is cut into groups of 16;
    byte i (0..7) of a group's 8 bytes holds element i in its low nibble and element
    8 + i in its high nibble, each a 4-bit two's-complement code.
    """
    b = np.asarray(packed, dtype=np.uint8)
    N = b.shape[0]
    g = b.reshape(N, K // 16, 8)
    lo = (g & 0x0F).astype(np.int16)
    hi = (g >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.concatenate([lo, hi], axis=2).reshape(N, K).astype(np.int8)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- the layer


def gate_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """Gate projection l[t, e] = sum_h x[t, h] * W_g[e, h] (float64).

    [MND §Overlapping computation and communication]: "Gate" is the last op of the
    attention stage feeding the MoE layer; the gate matrix maps H to E scores.
    """
    return x @ w_gate.T


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def route_topk(logits32: np.ndarray, bias32, k: int):
    """Top-k router on float32 scores.

    [MND §Expert Parallelism]: each token goes to k *different* routed experts and
    the routed results are weighted-summed.  [MND §MoE Router]: the router is a
    sort that tracks element indices, taking the top-k per token.  Scores are
    z = logit + bias in float32; the selection is the k largest z with ties to
    the lower expert id, listed in that order; the weights are the selected
    sigmoid scores renormalized to sum to 1, returned as float32.
    """
    z = np.asarray(logits32, dtype=np.float32)
    if bias32 is not None:
        z = (z + np.asarray(bias32, dtype=np.float32)[None, :]).astype(np.float32)
    if not np.isfinite(z).all():
        raise ValueError("non-finite router score")
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    order = np.argsort(-z, axis=1, kind="stable")    # z descending, equal z: lower id first
    idx = order[:, :k].astype(np.int32)
    s = sigmoid(np.take_along_axis(z, idx, axis=1))
    w = s / s.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


# The router's variants.  [MND §MoE Router]: one router serves every MoE model, since
# Mixtral's routing is DeepSeek's with the top-K group equal to the group of all experts.
# The pages name the top-K group but not its scoring; the readings taken here: experts
# form n_group groups of E / n_group consecutive ids; a group's score is the sum of its
# group_topn largest scores (1: its best expert; 2: its best two), added in float32; the
# topk_group best groups are kept (ties to the lower group id); the k experts are the
# best of the kept groups' experts.  Scores z = logit + bias decide both steps.  Weights:
# sigmoid(z) of the selected (the workload's scoring) or softmax(z) over all E experts
# taken at the selected (Mixtral's), optionally renormalized over the k selected, then
# multiplied by a routed scaling factor.
DEFAULT_ROUTER = dict(scoring="sigmoid", renormalize=True, n_group=1, topk_group=1, group_topn=1,
                      scale=1.0)


def route_grouped(logits32: np.ndarray, bias32, k: int, router=None):
    """General top-k router (group-limited selection, sigmoid or softmax weights).

    With the default router this is route_topk.  Returns (idx int32 [T, k], w float32
    [T, k]); idx lists each token's experts by z descending, ties to the lower id.
    """
    r = dict(DEFAULT_ROUTER, **(router or {}))
    z = np.asarray(logits32, dtype=np.float32)
    if bias32 is not None:
        z = (z + np.asarray(bias32, dtype=np.float32)[None, :]).astype(np.float32)
    if not np.isfinite(z).all():
        raise ValueError("non-finite router score")
    T, E = z.shape
    G, TG, GN = int(r["n_group"]), int(r["topk_group"]), int(r["group_topn"])
    if G < 1 or E % G or not 1 <= TG <= G or GN not in (1, 2) or GN > E // G:
        raise ValueError("bad expert grouping")
    gsz = E // G
    if not 1 <= k <= TG * gsz:
        raise ValueError("k must be in [1, topk_group * E / n_group]")
    if r["scoring"] not in ("sigmoid", "softmax"):
        raise ValueError("scoring is sigmoid or softmax")
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # group scores, in float32: the largest score plus (group_topn = 2) the second
        gscore = np.empty(G, dtype=np.float32)
        for g in range(G):
            vals = sorted(z[t, g * gsz:(g + 1) * gsz].tolist(), reverse=True)
            acc = np.float32(vals[0])
            if GN == 2:
                acc = np.float32(acc + np.float32(vals[1]))
            gscore[g] = acc
        kept = np.argsort(-gscore, kind="stable")[:TG]          # ties: lower group id first
        cand = np.sort(np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in kept]))
        order = cand[np.argsort(-z[t, cand], kind="stable")]    # ties: lower expert id first
        idx[t] = order[:k]
    zsel = np.take_along_axis(z, idx, axis=1).astype(np.float64)
    if r["scoring"] == "sigmoid":
        s = sigmoid(zsel)
    else:
        z64 = z.astype(np.float64)
        e = np.exp(z64 - z64.max(axis=1, keepdims=True))
        p_all = e / e.sum(axis=1, keepdims=True)
        s = np.take_along_axis(p_all, idx, axis=1)
    if r["renormalize"]:
        s = s / s.sum(axis=1, keepdims=True)
    w = s * float(r["scale"])
    return idx, w.astype(np.float32)


def init_routing(ids: np.ndarray, E: int, e_base: int = 0) -> dict:
    """Expand-and-sort routing (the first routing of double routing, and re-routing).

    [R1P §MoE deployment strategy optimization]: init-routing expands each token
    once per selected expert and sorts the copies by expert, returning
    tokens_per_expert and expanded_row_idx (used later to restore the original
    order); re-routing does the same for received rows with k = 1 and returns
    the ids that undo it.  [MND §MoE Router]: dense dispatch needs the routing
    aggregated per expert rather than per token.

    ids: [T, k] global expert ids.  Slot s = t*k + j; local id = id - e_base.
    Slots whose local id falls outside [0, E) are invalid: they are left out of
    every count, get expanded_row_idx = -1, and are reported in ``n_invalid``.
    Returns
      tokens_per_expert [E]   number of valid slots per local expert
      expert_offsets   [E+1]  exclusive prefix sum, offsets[E] = valid slots
      sorted_src       [Rv]   destination row r -> source slot s (rows grouped by
                              expert, ascending s inside an expert)
      expanded_row_idx [R]    source slot s -> destination row (-1 if invalid)
    """
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1) - e_base
    R = flat.size
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    counts = np.bincount(key[valid], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_src = np.argsort(key, kind="stable")[: int(valid.sum())].astype(np.int32)
    eri = np.full(R, -1, dtype=np.int32)
    eri[sorted_src] = np.arange(sorted_src.size, dtype=np.int32)
    return {"tokens_per_expert": counts, "expert_offsets": offsets,
            "sorted_src": sorted_src, "expanded_row_idx": eri,
            "n_invalid": int(R - valid.sum())}


def expand_rows(x: np.ndarray, sorted_src: np.ndarray, k: int) -> np.ndarray:
    """expanded_x[r] = x[sorted_src[r] // k]  ([R1P §MoE deployment strategy
    optimization]: init-routing yields expanded_x, the expanded and sorted tokens)."""
    return x[np.asarray(sorted_src) // k]


def swiglu_ffn(a: np.ndarray, w13: np.ndarray, w2: np.ndarray, quant_h=False) -> np.ndarray:
    """One SwiGLU expert: y = (silu(a W1^T) * (a W3^T)) W2^T, float64.

    w13 stacks W1 (gate, rows 0..I-1) over W3 (up, rows I..2I-1); w2 is [H, I].
    [MND §Quantization]: the SiLU output is quantized per 1x128 block for the
    fp8 down projection; ``quant_h`` True (or "fp8") applies that quantization
    (float32 values, then :func:`quant_1x128`) before the down projection, and
    "int8" the per-token int8 quantization of W8A8 (:func:`quant_per_token_int8`) of
    h rounded to bf16 (:func:`round_to_bf16`).
    """
    I = w13.shape[0] // 2
    g = a @ w13[:I].T
    u = a @ w13[I:].T
    h = g * sigmoid(g) * u
    if quant_h == "int8":
        # The row's int8 codes are decided from h held in bf16 (float32 h rounded to the
        # nearest bf16): the page fixes no precision for h before its A8 quantization, so
        # the decision is taken in the precision the kernels hold h in (they store h in
        # bf16 and quantize each row from those values; a row's amax spans all I columns,
        # which no single kernel tile holds).
        q, s = quant_per_token_int8(round_to_bf16(h.astype(np.float32)))
        h = dequant_rows(q, s)
    elif quant_h:
        q, s = quant_1x128(h.astype(np.float32))
        h = dequant_1x128(q, s)
    return h @ w2.T


def grouped_ffn(a_sorted: np.ndarray, offsets: np.ndarray, expert_weights, quant_h=False) -> np.ndarray:
    """GroupGEMM over ragged groups ([MND §Roofline / GroupGEMM]: group i has m_i rows
    and computes [m_i, k] x [k, n]).  Rows offsets[e]..offsets[e+1]-1 belong to
    expert e; expert_weights(e) -> (w13, w2) in float64."""
    R = int(offsets[-1])
    H = a_sorted.shape[1]
    y = np.zeros((R, H), dtype=np.float64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            w13, w2 = expert_weights(e)
            y[r0:r1] = swiglu_ffn(a_sorted[r0:r1], w13, w2, quant_h)
    return y


def finalize(y: np.ndarray, expanded_row_idx: np.ndarray, k: int, topk_w=None, skip=None) -> np.ndarray:
    """Un-permute and combine: out[t] = skip[t] + sum_j w[t, j] * y[expanded_row_idx[t*k + j]].

    [R1P §MoE deployment strategy optimization]: finalize-routing restores token
    order through expanded_src_to_dst_row = expanded_row_idx and forms the
    routed-expert weighted sum plus the shared-expert output (skip1) in one op.
    [MND §Expert Parallelism]: the shared-expert result is added to the weighted
    sum.  With k = 1, no weights and no skip this is the plain un-sort.
    Slots with expanded_row_idx = -1 contribute nothing.
    """
    eri = np.asarray(expanded_row_idx).reshape(-1, k)
    T = eri.shape[0]
    H = y.shape[1]
    out = np.zeros((T, H), dtype=np.float64) if skip is None else np.array(skip, dtype=np.float64)
    w = np.ones((T, k)) if topk_w is None else np.asarray(topk_w, dtype=np.float64)
    for j in range(k):
        r = eri[:, j]
        ok = r >= 0
        out[ok] += w[ok, j][:, None] * y[r[ok]]
    return out


def unsort(y_sorted: np.ndarray, sorted_src: np.ndarray) -> np.ndarray:
    """Arrival-order un-sort of re-routed rows, as the page writes it:
    index_select(y_sorted, 0, argsort(gathered_ids_unsort)) where
    gathered_ids_unsort = sorted_src ([R1P §MoE deployment strategy optimization])."""
    return y_sorted[np.argsort(np.asarray(sorted_src), kind="stable")]


# --------------------------------------------------------------------------- whole layer


def expert_weights_f64(inp: dict):
    """Adapter: per-expert float64 (w13, w2) from the generated arrays."""
    cfg = inp["cfg"]

    def get(e):
        if cfg.wt == "fp8":
            return (dequant_block128(inp["w13"][e], inp["w13_scale"][e]),
                    dequant_block128(inp["w2"][e], inp["w2_scale"][e]))
        if cfg.wt == "int8":
            return (dequant_rows(inp["w13"][e], inp["w13_scale"][e]),
                    dequant_rows(inp["w2"][e], inp["w2_scale"][e]))
        if cfg.wt == "int4":
            return (dequant_rows(int4_unpack(inp["w13"][e], cfg.H), inp["w13_scale"][e]),
                    dequant_rows(int4_unpack(inp["w2"][e], cfg.I), inp["w2_scale"][e]))
        return to_f64(inp["w13"][e], cfg.wt), to_f64(inp["w2"][e], cfg.wt)
    return get


def shared_weights_f64(inp: dict):
    """The shared expert's float64 (w13, w2): dequantized int8 codes beside W8A8 / W4A8
    experts, else the activation-dtype weights."""
    cfg = inp["cfg"]
    if cfg.sh_wt == "int8":
        return (dequant_rows(inp["sh_w13"], inp["sh_w13_scale"]),
                dequant_rows(inp["sh_w2"], inp["sh_w2_scale"]))
    return to_f64(inp["sh_w13"], cfg.sh_wt), to_f64(inp["sh_w2"], cfg.sh_wt)


def shared_expert(x: np.ndarray, inp: dict, weights=None) -> np.ndarray:
    """The shared expert on float64 tokens x: the same SwiGLU FFN with the shared
    weights ([MND §Expert Parallelism]).  Beside W8A8 or W4A8 routed experts it is
    W8A8 ([V32 §quantization strategy] quantizes the shared expert W8A8 in both): per-
    token int8 tokens, int8 weights with per-channel scales, h requantized per row.
    ``weights``: the float64 (w13, w2) of :func:`shared_weights_f64`, if already made."""
    cfg = inp["cfg"]
    w13, w2 = shared_weights_f64(inp) if weights is None else weights
    if cfg.sh_wt == "int8":
        xq, xs = quant_per_token_int8(x.astype(np.float32))
        return swiglu_ffn(dequant_rows(xq, xs), w13, w2, quant_h="int8")
    return swiglu_ffn(x, w13, w2)


def moe_layer(inp: dict, logits32_override=None, router=None, expert_weights=None,
              shared_weights=None) -> dict:
    """The whole layer on one GPU's share, step by step.

    Token path ([MND §Expert Parallelism], [R1P §MoE deployment strategy
    optimization]): gate -> top-k -> init-routing (expand + sort) -> grouped
    SwiGLU experts -> finalize-routing (un-permute, weighted sum, + shared
    expert).  Pretagged rows (an expert-parallel rank's received buffer): the
    re-routing sort with k = 1, the grouped experts, the un-sort back to arrival
    order, and the shared expert on the rank's local tokens.

    ``logits32_override`` lets a test route on another float32 logit matrix
    (the routing policy is exact only given identical float32 logits); ``router``
    selects a variant of the router (route_grouped), default the workload's.
    ``expert_weights`` (e -> float64 (w13, w2), default :func:`expert_weights_f64`) and
    ``shared_weights`` (float64 (w13, w2), default :func:`shared_weights_f64`) let a
    caller hand in weights it has already converted, e.g. one expert at a time.
    """
    cfg = inp["cfg"]
    fp8 = cfg.wt == "fp8"
    int8 = cfg.wt in ("int8", "int4")       # W8A8 and W4A8 share the A8 activations
    x = to_f64(inp["x"], cfg.act)
    res = {}
    if cfg.pretagged:
        ids = np.asarray(inp["ids"], dtype=np.int32)
        k = 1
    else:
        k = cfg.k
        logits = gate_logits(x, to_f64(inp["w_gate"], cfg.act))
        res["logits"] = logits
        l32 = logits.astype(np.float32) if logits32_override is None else logits32_override
        if router is None:
            idx, w = route_topk(l32, inp.get("bias"), k)
        else:
            idx, w = route_grouped(l32, inp.get("bias"), k, router)
        res["topk_idx"], res["topk_w"] = idx, w
        ids = idx
    rt = init_routing(ids, cfg.E, cfg.e_base)
    res.update(rt)
    if fp8:
        xq, xs = quant_1x128(x.astype(np.float32))
        res["x_q"], res["x_scale"] = xq, xs
        res["expanded_x"] = expand_rows(xq, rt["sorted_src"], k)
        res["expanded_scale"] = expand_rows(xs, rt["sorted_src"], k)
        a = dequant_1x128(res["expanded_x"], res["expanded_scale"])
    elif int8:
        # W8A8 ([V32 §quantization strategy]): each token quantized once, then copied
        xq, xs = quant_per_token_int8(x.astype(np.float32))
        res["x_q"], res["x_scale"] = xq, xs
        res["expanded_x"] = expand_rows(xq, rt["sorted_src"], k)
        res["expanded_scale"] = expand_rows(xs[:, None], rt["sorted_src"], k)[:, 0]
        a = dequant_rows(res["expanded_x"], res["expanded_scale"])
    else:
        res["expanded_x"] = expand_rows(inp["x"], rt["sorted_src"], k)
        a = expand_rows(x, rt["sorted_src"], k)
    y = grouped_ffn(a, rt["expert_offsets"], expert_weights or expert_weights_f64(inp),
                    quant_h="int8" if int8 else fp8)
    res["y_sorted"] = y
    sx = to_f64(inp["x_local"], cfg.act) if cfg.pretagged else x
    s = shared_expert(sx, inp, shared_weights)
    res["shared"] = s
    if cfg.pretagged:
        res["y_arrival"] = finalize(y, rt["expanded_row_idx"], 1)
    else:
        res["out"] = finalize(y, rt["expanded_row_idx"], k, res["topk_w"], s)
    return res
