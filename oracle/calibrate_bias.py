"""Choose the expert-bias strength alpha of the skewed fp8 workload.

The skewed long-prefill workload (T=16384, 256 experts, top-8) adds a Zipf(1.2)
expert bias b_e = alpha * ln p_e to the gate logits so that the most-loaded
expert receives about 8x the mean number of rows.  This script bisects alpha on
the seeded inputs until max(tokens_per_expert) / mean lies in [7.5, 8.5] and
prints it; the value is stored as ``C5_BIAS_ALPHA`` in ``synth/configs.py``.
It uses only the oracle's router and init-routing.

    python -m oracle.calibrate_bias
"""
from __future__ import annotations

import dataclasses

import numpy as np

from synth import configs, inputs
from oracle import moe


def load_ratio(cfg, logits32) -> float:
    idx, _ = moe.route_topk(logits32, inputs.expert_bias(cfg), cfg.k)
    tpe = moe.init_routing(idx, cfg.E)["tokens_per_expert"]
    return float(tpe.max() / tpe.mean())


def main():
    cfg = configs.get("c5_skewed_fp8")
    x = moe.to_f64(inputs.tokens(cfg), cfg.act)
    wg = moe.to_f64(inputs.gate_weight(cfg), cfg.act)
    logits32 = moe.gate_logits(x, wg).astype(np.float32)
    lo, hi = 0.0, 1.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        r = load_ratio(dataclasses.replace(cfg, bias_alpha=mid), logits32)
        print(f"alpha={mid:.10f} max/mean={r:.3f}", flush=True)
        if 7.5 <= r <= 8.5:
            print(f"C5_BIAS_ALPHA = {mid!r}")
            return mid
        if r < 8.0:
            lo = mid
        else:
            hi = mid
    raise SystemExit("no alpha found")


if __name__ == "__main__":
    main()
