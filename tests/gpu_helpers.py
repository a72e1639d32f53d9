"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

# max relative error bounds: bf16 2e-2, fp8 6e-2, fp32 1e-5 (the workload statement).
# W8A8 / W4A8: 2e-2, the bf16 bound.  Their integer work is exact on both sides (int8
# codes of the tokens bit for bit, int32 accumulation); the oracle decides h's int8 codes
# from h rounded to bf16, the precision the kernels hold h in, so a code differs only
# where the two float32 h values straddle a bf16 rounding boundary (about one element in
# 4000, by one code step, i.e. at most 1/127 of the row's amax times one weight); what
# remains is the bf16 rounding of h and y, as in the bf16 layer.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "int8": 2e-2, "int4": 2e-2}

# (test, workload, observed max row relative error, bound) of every checked float output
ERRS = []


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def tol_of(cfg) -> float:
    return TOL[cfg.wt] if cfg.wt in ("fp8", "int8", "int4") else TOL[cfg.act]


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def act_to_f64(t: torch.Tensor, act: str) -> np.ndarray:
    a = host(t)
    if act == "bf16":
        return (a.astype(np.int16).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float -> bf16 bits (round to nearest even), for feeding oracle values to a GPU call."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def max_row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_h |got - ref| / max_h |ref| (rows of zeros compare absolutely)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - ref).max(axis=1) / den).max())


def act_dtype(act: str):
    return torch.float32 if act == "f32" else torch.int16


def empty_act(shape, act, device="cuda"):
    return torch.empty(shape, dtype=act_dtype(act), device=device)


def poison_(t: torch.Tensor):
    """Fill with a recognisable pattern so unwritten outputs show up."""
    if t.dtype == torch.float32:
        t.fill_(float("nan"))
    elif t.dtype == torch.int32:
        t.fill_(-7777)
    elif t.dtype == torch.int16:
        t.fill_(0x7FC1)  # a bf16 NaN
    else:
        t.fill_(0x7F)  # fp8 NaN code
    return t


def check_close(label: str, got: np.ndarray, ref: np.ndarray, tol: float) -> float:
    """max_row_rel_err(got, ref) <= tol; the observed error is printed and recorded so
    the run's summary lists every workload's margin."""
    err = max_row_rel_err(got, ref)
    ERRS.append((label, err, tol))
    say(f"  {label}: max row rel err {err:.3e} (bound {tol:.0e})")
    assert err <= tol, f"{label}: {err:.3e} > {tol:.0e}"
    return err
