"""Upload seeded synthetic inputs to device memory (torch tensors).

Marshalling only: the bytes are exactly those drawn by :mod:`synth.inputs`.
bf16 tensors travel as int16 bit patterns, fp8 as uint8 codes.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import inputs
from .configs import MoEConfig


def to_dev(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload_small(d: dict, device="cuda") -> dict:
    """All arrays of :func:`synth.inputs.layer_inputs` as device tensors."""
    return {k: (to_dev(v, device) if isinstance(v, np.ndarray) else v) for k, v in d.items()}


def _dtype_of(kind: str):
    return {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8, "int8": torch.int8,
            "int4": torch.uint8}[kind]


def upload_experts(cfg: MoEConfig, device="cuda", workers=None) -> dict:
    """Routed expert weights drawn expert by expert on a thread pool and copied into
    [E, 2I, H] / [E, H, I] device tensors (plus fp8 block scales or int8 channel scales)."""
    E, I, H = cfg.E, cfg.I, cfg.H
    dt = _dtype_of(cfg.wt)
    pk = 2 if cfg.wt == "int4" else 1                # int4: two codes per byte
    out = {"w13": torch.empty((E, 2 * I, H // pk), dtype=dt, device=device),
           "w2": torch.empty((E, H, I // pk), dtype=dt, device=device)}
    fp8 = cfg.wt == "fp8"
    scaled = cfg.wt in ("fp8", "int8", "int4")
    if fp8:
        out["w13_scale"] = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        out["w2_scale"] = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=device)
    elif scaled:
        out["w13_scale"] = torch.empty((E, 2 * I), dtype=torch.float32, device=device)
        out["w2_scale"] = torch.empty((E, H), dtype=torch.float32, device=device)
    for name, fn in (("w13", inputs.expert_w13), ("w2", inputs.expert_w2)):
        for e, v in inputs.for_each_expert(cfg, fn, workers=workers):
            if scaled:
                codes, scales = v
                out[name][e].copy_(torch.from_numpy(codes))
                out[name + "_scale"][e].copy_(torch.from_numpy(scales))
            else:
                if v.dtype == np.uint16:
                    v = v.view(np.int16)
                out[name][e].copy_(torch.from_numpy(v))
    return out


def upload_layer(cfg: MoEConfig, device="cuda") -> dict:
    """Every input of one full-size layer call, in device memory."""
    d = {"cfg": cfg}
    d["x"] = to_dev(inputs.tokens(cfg), device)
    b = inputs.expert_bias(cfg)
    d["bias"] = to_dev(b, device)
    if cfg.pretagged:
        d["ids"] = to_dev(inputs.pretagged_ids(cfg), device)
        d["x_local"] = to_dev(inputs.local_tokens(cfg), device)
    else:
        d["w_gate"] = to_dev(inputs.gate_weight(cfg), device)
    for name, v in inputs.shared_weights(cfg).items():
        d[name] = to_dev(v, device)
    d.update(upload_experts(cfg, device))
    return d
