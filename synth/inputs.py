"""Seeded synthetic inputs for the MoE expert layer.

This module only draws inputs.  It holds none of the layer's arithmetic: no
gate, routing, FFN or combine step, and no activation quantization.  Both the
CPU oracle and the GPU path consume exactly the bytes produced here.

Recipe
------
* Every tensor comes from its own counter-based stream,
  ``Philox(SeedSequence([seed, cfg.cid, tensor_id, expert]))``, so one expert's
  weights can be regenerated alone and experts can be drawn in parallel.
* Normal values are drawn by inverse-CDF lookup: 16 random bits ``u`` select the
  quantile ``std * Phi^-1((u + 0.5) / 65536)`` (a normal truncated at about
  +-4.17 sigma on a 16-bit quantile grid), rounded once to the storage dtype
  (bf16 with round-to-nearest-even).  fp32 tensors use 32 random bits instead.
* fp8 expert weights (static block quantization, as DeepSeek-V3/R1 ships them):
  e4m3fn codes of the quantile grid scaled so the +-4.2 sigma extreme maps
  below 448, times one fp32 scale per 128x128 block drawn as
  ``std * 4.2 / 448 * 2**U(-0.5, 0.5)``.
* int8 expert weights (static per-output-channel quantization, the W8 of W8A8):
  codes round(Phi^-1(u) * 127 / 4.2) of the same 16-bit quantile grid (|code| <= 127),
  times one fp32 scale per output channel drawn as ``std * 4.2 / 127 * 2**U(-0.5, 0.5)``.
* int4 expert weights (the W4 of W4A8): codes round(Phi^-1(u) * 7 / 4.2) in [-7, 7] of
  the same grid, packed two per byte (per 16 elements of K: byte i holds element i in
  its low nibble and element 8 + i in its high nibble), with per-output-channel fp32
  scales drawn as ``std * 4.2 / 7 * 2**U(-0.5, 0.5)``.
* Expert-popularity bias (decode / skewed workloads): a seeded permutation ranks
  the experts, p_e is proportional to rank_e**-s, and b_e = alpha * ln p_e.
* The shared expert beside int8 or int4 experts is int8 (W8A8), drawn like the int8
  expert weights from its own streams; otherwise it is in the activation dtype.
* Pretagged rows (expert-parallel rank share): ids i.i.d. uniform over the
  rank's experts [e_base, e_base + E).

bf16 tensors are returned as ``uint16`` bit patterns, fp8 tensors as ``uint8``
codes, int8 tensors as ``int8`` codes, fp32 tensors as ``float32``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np
from scipy.special import ndtri

from .configs import MoEConfig

# tensor ids folded into the seed
X, WG, W13, W2, SW13, SW2, BIAS, IDS, XLOCAL, W13S, W2S, PERM, SW13S, SW2S = range(1, 15)
SHARED = 0xFFFF  # "expert" slot used for non-expert tensors

_FP8_RANGE_SIGMA = 4.2


def stream(cfg: MoEConfig, tensor_id: int, expert: int = SHARED) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, cfg.cid, tensor_id, expert])
    return np.random.Generator(np.random.Philox(ss))


def _u16(gen: np.random.Generator, n: int) -> np.ndarray:
    words = (n + 3) // 4
    return gen.bit_generator.random_raw(words).view(np.uint16)[:n]


def _u32(gen: np.random.Generator, n: int) -> np.ndarray:
    words = (n + 1) // 2
    return gen.bit_generator.random_raw(words).view(np.uint32)[:n]


@lru_cache(maxsize=None)
def _quantiles16() -> np.ndarray:
    i = np.arange(65536, dtype=np.float64)
    return ndtri((i + 0.5) / 65536.0)


def _round_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@lru_cache(maxsize=None)
def _bf16_table(std: float) -> np.ndarray:
    return _round_bf16_bits((_quantiles16() * std).astype(np.float32))


@lru_cache(maxsize=None)
def _fp8_table() -> np.ndarray:
    import torch  # the library cast encodes the static weight grid
    v = torch.from_numpy((_quantiles16() * (448.0 / _FP8_RANGE_SIGMA)).astype(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def normal_bf16(gen: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    return _bf16_table(float(std))[_u16(gen, n)].reshape(shape)


def normal_f32(gen: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    u = _u32(gen, n).astype(np.float64)
    return (ndtri((u + 0.5) / 4294967296.0) * std).astype(np.float32).reshape(shape)


def normal_fp8_blocks(gen_codes: np.random.Generator, gen_scales: np.random.Generator,
                      shape, std: float):
    """fp8 e4m3fn codes [..., N, K] and fp32 scales [..., N/128, K/128]."""
    *lead, N, K = shape
    assert N % 128 == 0 and K % 128 == 0
    n = int(np.prod(shape))
    codes = _fp8_table()[_u16(gen_codes, n)].reshape(shape)
    sshape = tuple(lead) + (N // 128, K // 128)
    u = gen_scales.random(int(np.prod(sshape)))
    scales = (std * _FP8_RANGE_SIGMA / 448.0) * np.exp2(u - 0.5)
    return codes, scales.astype(np.float32).reshape(sshape)


@lru_cache(maxsize=None)
def _int8_table() -> np.ndarray:
    return np.clip(np.rint(_quantiles16() * (127.0 / _FP8_RANGE_SIGMA)), -127, 127).astype(np.int8)


def normal_int8_channels(gen_codes: np.random.Generator, gen_scales: np.random.Generator,
                         shape, std: float):
    """int8 codes [..., N, K] and fp32 scales [..., N] (one per output channel)."""
    *lead, N, K = shape
    n = int(np.prod(shape))
    codes = _int8_table()[_u16(gen_codes, n)].reshape(shape)
    sshape = tuple(lead) + (N,)
    u = gen_scales.random(int(np.prod(sshape)))
    scales = (std * _FP8_RANGE_SIGMA / 127.0) * np.exp2(u - 0.5)
    return codes, scales.astype(np.float32).reshape(sshape)


@lru_cache(maxsize=None)
def _int4_table() -> np.ndarray:
    return np.clip(np.rint(_quantiles16() * (7.0 / _FP8_RANGE_SIGMA)), -7, 7).astype(np.int8)


def normal_int4_channels(gen_codes: np.random.Generator, gen_scales: np.random.Generator,
                         shape, std: float):
    """Packed int4 codes [..., N, K/2] (uint8) and fp32 scales [..., N]."""
    *lead, N, K = shape
    assert K % 16 == 0
    n = int(np.prod(shape))
    codes = _int4_table()[_u16(gen_codes, n)].reshape(-1, K // 16, 2, 8).astype(np.int16) & 0xF
    packed = (codes[:, :, 0, :] | (codes[:, :, 1, :] << 4)).astype(np.uint8)
    u = gen_scales.random(int(np.prod(tuple(lead) + (N,))))
    scales = (std * _FP8_RANGE_SIGMA / 7.0) * np.exp2(u - 0.5)
    return packed.reshape(tuple(lead) + (N, K // 2)), scales.astype(np.float32).reshape(tuple(lead) + (N,))


def _normal(cfg: MoEConfig, dtype: str, gen, shape, std):
    if dtype == "f32":
        return normal_f32(gen, shape, std)
    if dtype == "bf16":
        return normal_bf16(gen, shape, std)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------- tensors

def tokens(cfg: MoEConfig) -> np.ndarray:
    """x [T, H] (pretagged: the received rows)."""
    return _normal(cfg, cfg.act, stream(cfg, X), (cfg.T, cfg.H), cfg.x_std)


def local_tokens(cfg: MoEConfig) -> np.ndarray:
    """Local tokens [T_local, H] fed to the shared expert (pretagged only)."""
    return _normal(cfg, cfg.act, stream(cfg, XLOCAL), (cfg.T_local, cfg.H), cfg.x_std)


def gate_weight(cfg: MoEConfig) -> np.ndarray:
    """W_g [E, H] (activation dtype)."""
    return _normal(cfg, cfg.act, stream(cfg, WG), (cfg.E, cfg.H), cfg.gate_std)


def expert_bias(cfg: MoEConfig):
    """b [E] fp32 or None."""
    if not cfg.has_bias:
        return None
    perm = stream(cfg, PERM).permutation(cfg.E)
    rank = np.empty(cfg.E, dtype=np.float64)
    rank[perm] = np.arange(1, cfg.E + 1, dtype=np.float64)
    logp = -cfg.zipf_s * np.log(rank)
    logp -= np.log(np.exp(logp).sum())
    return (cfg.bias_alpha * logp).astype(np.float32)


def pretagged_ids(cfg: MoEConfig) -> np.ndarray:
    """Global expert ids [T, 1] int32 of the received rows."""
    g = stream(cfg, IDS)
    return (cfg.e_base + g.integers(0, cfg.E, size=(cfg.T, 1))).astype(np.int32)


def expert_w13(cfg: MoEConfig, e: int):
    """Stacked gate (rows 0..I-1) and up (rows I..2I-1) projections [2I, H].

    fp8: returns (codes, scales [2I/128, H/128]); int8: (codes, scales [2I])."""
    shape = (2 * cfg.I, cfg.H)
    if cfg.wt == "fp8":
        return normal_fp8_blocks(stream(cfg, W13, e), stream(cfg, W13S, e), shape, cfg.w_std)
    if cfg.wt == "int8":
        return normal_int8_channels(stream(cfg, W13, e), stream(cfg, W13S, e), shape, cfg.w_std)
    if cfg.wt == "int4":
        return normal_int4_channels(stream(cfg, W13, e), stream(cfg, W13S, e), shape, cfg.w_std)
    return _normal(cfg, cfg.wt, stream(cfg, W13, e), shape, cfg.w_std)


def expert_w2(cfg: MoEConfig, e: int):
    """Down projection [H, I]. fp8: returns (codes, scales [H/128, I/128]); int8:
    (codes, scales [H])."""
    shape = (cfg.H, cfg.I)
    if cfg.wt == "fp8":
        return normal_fp8_blocks(stream(cfg, W2, e), stream(cfg, W2S, e), shape, cfg.w_std)
    if cfg.wt == "int8":
        return normal_int8_channels(stream(cfg, W2, e), stream(cfg, W2S, e), shape, cfg.w_std)
    if cfg.wt == "int4":
        return normal_int4_channels(stream(cfg, W2, e), stream(cfg, W2S, e), shape, cfg.w_std)
    return _normal(cfg, cfg.wt, stream(cfg, W2, e), shape, cfg.w_std)


def shared_w13(cfg: MoEConfig):
    """Shared expert [2*I_shared, H] in cfg.sh_wt: the activation dtype, or for int8
    (codes, scales [2*I_shared]) drawn like the int8 expert weights."""
    shape = (2 * cfg.I_shared, cfg.H)
    if cfg.sh_wt == "int8":
        return normal_int8_channels(stream(cfg, SW13), stream(cfg, SW13S), shape, cfg.w_std)
    return _normal(cfg, cfg.sh_wt, stream(cfg, SW13), shape, cfg.w_std)


def shared_w2(cfg: MoEConfig):
    """Shared expert down projection [H, I_shared]; int8: (codes, scales [H])."""
    shape = (cfg.H, cfg.I_shared)
    if cfg.sh_wt == "int8":
        return normal_int8_channels(stream(cfg, SW2), stream(cfg, SW2S), shape, cfg.w_std)
    return _normal(cfg, cfg.sh_wt, stream(cfg, SW2), shape, cfg.w_std)


def shared_weights(cfg: MoEConfig) -> dict:
    """sh_w13, sh_w2 and, for int8, sh_w13_scale and sh_w2_scale."""
    d = {}
    for name, fn in (("sh_w13", shared_w13), ("sh_w2", shared_w2)):
        v = fn(cfg)
        if cfg.sh_wt == "int8":
            d[name], d[name + "_scale"] = v
        else:
            d[name] = v
    return d


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def for_each_expert(cfg: MoEConfig, fn, experts=None, workers=None):
    """Yield (e, fn(cfg, e)) for the given experts, drawn on a thread pool."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    with ThreadPoolExecutor(workers or _workers()) as ex:
        for e, v in zip(experts, ex.map(lambda e: fn(cfg, e), experts)):
            yield e, v


def layer_inputs(cfg: MoEConfig, with_experts: bool = True) -> dict:
    """All inputs of one layer call as host arrays (small configurations)."""
    d = {"cfg": cfg, "x": tokens(cfg), "bias": expert_bias(cfg)}
    if cfg.pretagged:
        d["ids"] = pretagged_ids(cfg)
        d["x_local"] = local_tokens(cfg)
    else:
        d["w_gate"] = gate_weight(cfg)
    d.update(shared_weights(cfg))
    if with_experts:
        w13 = [None] * cfg.E
        w2 = [None] * cfg.E
        for e, v in for_each_expert(cfg, expert_w13):
            w13[e] = v
        for e, v in for_each_expert(cfg, expert_w2):
            w2[e] = v
        if cfg.wt in ("fp8", "int8", "int4"):
            d["w13"] = np.stack([c for c, _ in w13])
            d["w13_scale"] = np.stack([s for _, s in w13])
            d["w2"] = np.stack([c for c, _ in w2])
            d["w2_scale"] = np.stack([s for _, s in w2])
        else:
            d["w13"] = np.stack(w13)
            d["w2"] = np.stack(w2)
    return d
