"""Workload configurations for the MoE expert layer.

Each configuration fixes the sizes, dtypes and input distributions of one
seeded synthetic workload.  The five full-size workloads mirror the shapes the
pages discuss:

* [MND] = page "Lower latency and higher throughput with multi-node DeepSeek
  deployment" (Perplexity blog, 2025-04-18): 256 routed experts + 1 shared
  expert, 8 routed experts per token (section "Expert Parallelism");
  decode batches of 128 per GPU (section "Latency breakdown").
* [R1P] = page "CANN/cann-recipes-infer: DeepSeek-R1 prefill optimization"
  (Atlas A3): prefill of 4K-token requests with expert-parallel double routing
  (section "MoE deployment strategy optimization"), two 4K requests per card
  (section "micro-batch optimization").

The ``p*`` configurations are reduced copies that keep every structural
feature (ragged expert loads, empty experts, an expert base offset, the fp8
scale layout, partial N tiles) at sizes a plain CPU reference finishes in
seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cid: int                 # stable integer folded into every seed
    T: int                   # tokens (for pretagged: received expanded rows)
    H: int                   # hidden size
    E: int                   # routed experts held on this GPU
    k: int                   # routed experts per token (1 for pretagged rows)
    I: int                   # routed SwiGLU intermediate size
    I_shared: int            # shared-expert intermediate size
    act: str                 # activation dtype: "f32" | "bf16"
    wt: str                  # expert-weight dtype: "f32" | "bf16" | "fp8" | "int8" | "int4"
    x_std: float = 1.0
    wg_std: Optional[float] = None   # None -> 1/sqrt(H) (logits ~ N(0,1))
    w_std: float = 0.02
    zipf_s: Optional[float] = None   # expert-popularity bias exponent
    bias_alpha: float = 0.0          # bias b_e = alpha * ln p_e
    pretagged: bool = False          # rows arrive with expert ids (no gate)
    e_base: int = 0                  # first global expert id held here
    E_total: Optional[int] = None    # experts in the whole model (pretagged)
    T_local: int = 0                 # local tokens for the shared expert (pretagged)
    seed: int = 0
    description: str = ""

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def gate_std(self) -> float:
        return self.wg_std if self.wg_std is not None else self.H ** -0.5

    @property
    def has_bias(self) -> bool:
        return self.zipf_s is not None and self.bias_alpha != 0.0

    @property
    def shared_rows(self) -> int:
        return self.T_local if self.pretagged else self.T

    @property
    def sh_wt(self) -> str:
        """Shared-expert weight dtype: int8 (W8A8) beside W8A8 or W4A8 routed experts,
        else the activation dtype (bf16 also beside fp8 routed experts)."""
        return "int8" if self.wt in ("int8", "int4") else self.act


# Calibrated by oracle/calibrate_bias.py so that the most-loaded expert receives
# about 8x the mean rows (max/mean in [7.5, 8.5]) at the full T=16384 workload.
C5_BIAS_ALPHA = 0.234375

CONFIGS = {
    "c1_tiny_fp32": MoEConfig(
        name="c1_tiny_fp32", cid=1, T=64, H=256, E=16, k=2, I=128, I_shared=128,
        act="f32", wt="f32", x_std=0.02, wg_std=0.02, w_std=0.02,
        description="tiny MoE layer, fp32, N(0,1)*0.02 tokens and weights"),
    "c2_prefill_bf16": MoEConfig(
        name="c2_prefill_bf16", cid=2, T=8192, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="bf16",
        description="DeepSeek-V3-shaped prefill layer (two 4K requests), bf16"),
    "c3_ep_rank_bf16": MoEConfig(
        name="c3_ep_rank_bf16", cid=3, T=8192, H=7168, E=32, k=1, I=2048, I_shared=2048,
        act="bf16", wt="bf16", pretagged=True, e_base=96, E_total=256, T_local=1024,
        description="one expert-parallel rank's share at ep=8: 8192 received rows "
                    "tagged with local experts 96..127, 1024 local tokens"),
    "c4_decode_bf16": MoEConfig(
        name="c4_decode_bf16", cid=4, T=128, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="bf16", zipf_s=1.1, bias_alpha=0.5,
        description="decode batch of 128 tokens, Zipf(1.1) expert popularity"),
    "c5_skewed_fp8": MoEConfig(
        name="c5_skewed_fp8", cid=5, T=16384, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="fp8", zipf_s=1.2, bias_alpha=C5_BIAS_ALPHA,
        description="skewed long prefill, fp8 e4m3 experts with 128x128 scales, "
                    "bf16 activations quantized 1x128 per token"),
    # ---- W8A8 experts (int8 weights per output channel, int8 activations per token) --
    "c6_prefill_w8a8": MoEConfig(
        name="c6_prefill_w8a8", cid=6, T=8192, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="int8",
        description="the c2 prefill layer with W8A8 experts and shared expert (static "
                    "per-channel int8 weights, dynamic per-token int8 activations)"),
    "c7_decode_w8a8": MoEConfig(
        name="c7_decode_w8a8", cid=7, T=128, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="int8", zipf_s=1.1, bias_alpha=0.5,
        description="the c4 decode batch with W8A8 experts"),
    "c9_decode1_bf16": MoEConfig(
        name="c9_decode1_bf16", cid=9, T=1, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="bf16", zipf_s=1.1, bias_alpha=0.5,
        description="one-token decode step of the c4 layer: 8 routed experts of one row each, "
                    "the expert GEMMs split along K"),
    "c10_decode_fp8": MoEConfig(
        name="c10_decode_fp8", cid=10, T=128, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="fp8", zipf_s=1.1, bias_alpha=0.5,
        description="the c4 decode batch with fp8 e4m3 experts (128x128 scales); bf16 shared "
                    "expert"),
    "c8_decode_w4a8": MoEConfig(
        name="c8_decode_w4a8", cid=8, T=128, H=7168, E=256, k=8, I=2048, I_shared=2048,
        act="bf16", wt="int4", zipf_s=1.1, bias_alpha=0.5,
        description="the c4 decode batch with W4A8 experts (packed int4 weights per channel, "
                    "int8 activations per token)"),
    # ---- reduced parity workloads -------------------------------------------------
    "p2_prefill_bf16": MoEConfig(
        name="p2_prefill_bf16", cid=12, T=1000, H=512, E=16, k=6, I=256, I_shared=256,
        act="bf16", wt="bf16",
        description="reduced prefill: ~375 rows/expert, so experts split into units"),
    "p2b_prefill_bf16": MoEConfig(
        name="p2b_prefill_bf16", cid=22, T=613, H=640, E=32, k=8, I=384, I_shared=384,
        act="bf16", wt="bf16",
        description="reduced prefill with H=640 (partial 256-wide N tile) and I=384"),
    "p2c_prefill_bf16": MoEConfig(
        name="p2c_prefill_bf16", cid=32, T=400, H=384, E=8, k=2, I=256, I_shared=384,
        act="bf16", wt="bf16",
        description="reduced bf16 prefill with I != I_shared (shared expert in its own launches)"),
    "p3_ep_rank_bf16": MoEConfig(
        name="p3_ep_rank_bf16", cid=13, T=1500, H=512, E=8, k=1, I=256, I_shared=256,
        act="bf16", wt="bf16", pretagged=True, e_base=24, E_total=64, T_local=200,
        description="reduced expert-parallel rank share (experts 24..31 of 64)"),
    "p4_decode_bf16": MoEConfig(
        name="p4_decode_bf16", cid=14, T=24, H=512, E=64, k=8, I=256, I_shared=256,
        act="bf16", wt="bf16", zipf_s=1.1, bias_alpha=0.5,
        description="reduced decode: many experts with 0-2 rows"),
    "p5_skewed_fp8": MoEConfig(
        name="p5_skewed_fp8", cid=15, T=700, H=512, E=16, k=4, I=256, I_shared=256,
        act="bf16", wt="fp8", zipf_s=1.2, bias_alpha=1.0,
        description="reduced skewed fp8 layer"),
    "p5b_decode_fp8": MoEConfig(
        name="p5b_decode_fp8", cid=25, T=24, H=512, E=64, k=8, I=256, I_shared=256,
        act="bf16", wt="fp8", zipf_s=1.1, bias_alpha=0.5,
        description="reduced fp8 decode: many experts with 0-2 rows (the 32-row fp8 tiles)"),
    "p6_prefill_w8a8": MoEConfig(
        name="p6_prefill_w8a8", cid=16, T=700, H=512, E=16, k=4, I=256, I_shared=256,
        act="bf16", wt="int8", zipf_s=1.2, bias_alpha=1.0,
        description="reduced skewed W8A8 layer (experts split into several units)"),
    "p7_decode_w8a8": MoEConfig(
        name="p7_decode_w8a8", cid=17, T=24, H=512, E=64, k=8, I=256, I_shared=256,
        act="bf16", wt="int8", zipf_s=1.1, bias_alpha=0.5,
        description="reduced W8A8 decode: many experts with 0-2 rows"),
    "p8_prefill_w4a8": MoEConfig(
        name="p8_prefill_w4a8", cid=18, T=700, H=512, E=16, k=4, I=256, I_shared=256,
        act="bf16", wt="int4", zipf_s=1.2, bias_alpha=1.0,
        description="reduced skewed W4A8 layer"),
    "p9_decode_w4a8": MoEConfig(
        name="p9_decode_w4a8", cid=19, T=24, H=512, E=64, k=8, I=256, I_shared=256,
        act="bf16", wt="int4", zipf_s=1.1, bias_alpha=0.5,
        description="reduced W4A8 decode"),
    "p9b_decode_w4a8": MoEConfig(
        name="p9b_decode_w4a8", cid=29, T=24, H=384, E=64, k=8, I=384, I_shared=384,
        act="bf16", wt="int4", zipf_s=1.1, bias_alpha=0.5,
        description="reduced W4A8 decode with H and I multiples of 128 but not of 256 "
                    "(the 128-element weight stages)"),
    # ---- split-K decode: a few tokens over long K, so the expert GEMMs store fp32
    # partials of K slices (T=3, k=2: at most 6 units; slices of at least 16 stages) ----
    "p10_split_bf16": MoEConfig(
        name="p10_split_bf16", cid=40, T=3, H=2048, E=8, k=2, I=2048, I_shared=2048,
        act="bf16", wt="bf16", description="three-token decode, both expert GEMMs split along K, bf16"),
    "p11_split_fp8": MoEConfig(
        name="p11_split_fp8", cid=41, T=3, H=4096, E=8, k=2, I=1024, I_shared=1024,
        act="bf16", wt="fp8", description="three-token decode, split-K first expert GEMM, fp8"),
    "p12_split_w8a8": MoEConfig(
        name="p12_split_w8a8", cid=42, T=3, H=4096, E=8, k=2, I=1024, I_shared=1024,
        act="bf16", wt="int8", description="three-token decode, split-K first expert GEMM, W8A8"),
    "p13_split_w4a8": MoEConfig(
        name="p13_split_w4a8", cid=43, T=3, H=8192, E=8, k=2, I=1024, I_shared=1024,
        act="bf16", wt="int4", description="three-token decode, split-K first expert GEMM, W4A8"),
    # ---- prefill with enough experts (128) for the down projection to compute several
    # output tiles per workgroup: H = 1280 is five 256-column tiles, so the workgroups
    # take four tiles and then one; I = 384 gives the int8 / int4 down projection an odd
    # number of K stages (each tile starts its own load ring) ----
    "p14_multi_bf16": MoEConfig(
        name="p14_multi_bf16", cid=44, T=1125, H=1280, E=128, k=8, I=256, I_shared=256,
        act="bf16", wt="bf16", description="prefill, 128 experts, H = 1280 (bf16 twin of p15 and p16)"),
    "p15_multi_w8a8": MoEConfig(
        name="p15_multi_w8a8", cid=45, T=1125, H=1280, E=128, k=8, I=384, I_shared=384,
        act="bf16", wt="int8", description="W8A8 prefill, 128 experts, several tiles per workgroup, odd K stages"),
    "p16_multi_w4a8": MoEConfig(
        name="p16_multi_w4a8", cid=46, T=1125, H=1280, E=128, k=8, I=384, I_shared=384,
        act="bf16", wt="int4", description="W4A8 prefill, 128 experts, several tiles per workgroup, odd K stages"),
    "p1_small_fp32": MoEConfig(
        name="p1_small_fp32", cid=11, T=150, H=384, E=12, k=3, I=256, I_shared=128,
        act="f32", wt="f32", x_std=0.02, wg_std=0.02, w_std=0.02,
        description="fp32 layer with a ragged tail and I != I_shared"),
}

FULL_CONFIGS = ["c1_tiny_fp32", "c2_prefill_bf16", "c3_ep_rank_bf16",
                "c4_decode_bf16", "c5_skewed_fp8", "c6_prefill_w8a8", "c7_decode_w8a8",
                "c8_decode_w4a8", "c9_decode1_bf16", "c10_decode_fp8"]
SMALL_CONFIGS = ["c1_tiny_fp32", "p1_small_fp32", "p2_prefill_bf16", "p2b_prefill_bf16",
                 "p2c_prefill_bf16", "p3_ep_rank_bf16", "p4_decode_bf16", "p5_skewed_fp8", "p5b_decode_fp8",
                 "p6_prefill_w8a8", "p7_decode_w8a8", "p8_prefill_w4a8", "p9_decode_w4a8",
                 "p9b_decode_w4a8", "p10_split_bf16", "p11_split_fp8", "p12_split_w8a8",
                 "p13_split_w4a8", "p14_multi_bf16", "p15_multi_w8a8", "p16_multi_w4a8"]


def get(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg
