"""The bench's roofline accounting against the formulas and worked numbers the pages print.

Fixture: tests/golden/page_accounting.json (each value cites its passage)."""
import json
import os

import numpy as np

import bench
from synth import configs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_accounting.json")))


def test_rows_per_expert_worked_example():
    ex = GOLD["rows_per_expert"]
    assert bench.rows_per_expert(ex["batch"], ex["qlen"], ex["topk"], ex["ep"], ex["experts"]) == ex["m"]


def test_group_gemm_formulas():
    g = GOLD["group_gemm"]
    assert bench.group_gemm_flops(g["g"], g["m"], g["k"], g["n"]) == g["flops"]
    assert bench.group_gemm_elems(g["g"], g["m"], g["k"], g["n"]) == g["elems"]
    d = GOLD["gemm"]
    assert bench.gemm_flops(d["m"], d["k"], d["n"]) == d["flops"]
    assert bench.gemm_elems(d["m"], d["k"], d["n"]) == d["elems"]


def test_fp8_scale_shapes():
    s = GOLD["fp8_scale_shapes"]
    M, K, N = s["M"], s["K"], s["N"]
    assert (M, -(-K // 128)) == tuple(s["activation"])
    assert (-(-K // 128), -(-N // 128)) == tuple(s["weight"])


def test_layer_accounting_matches_group_gemm_formula():
    """With every expert holding m rows, GEMM1's FLOPs are the grouped-GEMM formula with
    n = 2I, and its weight bytes are E panels of 2I x H."""
    cfg = configs.get("c2_prefill_bf16")
    tpe = np.full(cfg.E, cfg.T * cfg.k // cfg.E)
    acc = bench.account(cfg, tpe)
    m = cfg.T * cfg.k // cfg.E
    assert acc["ffn1"]["flops"] == bench.group_gemm_flops(cfg.E, m, cfg.H, 2 * cfg.I)
    assert acc["ffn2"]["flops"] == bench.group_gemm_flops(cfg.E, m, cfg.I, cfg.H)
    w = cfg.E * 2 * cfg.I * cfg.H * 2
    assert acc["ffn1"]["bytes"] == w + cfg.R * cfg.H * 2 + cfg.R * cfg.I * 2
    # empty experts cost no weight bytes
    tpe2 = tpe.copy()
    tpe2[:10] = 0
    assert bench.account(cfg, tpe2)["ffn1"]["bytes"] < acc["ffn1"]["bytes"]


def test_activated_experts_per_gpu_example():
    """[MND §Single node vs multi-node]: batch 1, query length 2, top-8 over 8 GPUs ->
    on average 2*8/8 = 2 activated experts per GPU."""
    ex = GOLD["activated_experts"]
    assert ex["tokens"] * ex["topk"] / ex["gpus"] == ex["per_gpu"]


def test_launch_accounting_merged_and_gathered():
    """The c2 launches fold the shared expert into ffn1/ffn2 and gather the routed rows
    from x: ffn1 then reads x (T rows) instead of R expanded rows, plus the shared GEMM1."""
    cfg = configs.get("c2_prefill_bf16")
    tpe = np.full(cfg.E, cfg.T * cfg.k // cfg.E)
    acc = bench.account(cfg, tpe)
    la = bench.launch_accounting(cfg, acc)
    assert bench.shared_is_merged(cfg) and bench.gathers_rows(cfg)
    assert "shared" not in la and la["expand"]["bytes"] == 0
    T, H, I = cfg.T, cfg.H, cfg.I
    assert la["ffn1"]["flops"] == acc["ffn1"]["flops"] + 2 * T * H * 2 * I
    w_routed = cfg.E * 2 * I * H * 2
    shared1 = 2 * I * H * 2 + T * H * 2 + T * I * 2
    assert la["ffn1"]["bytes"] == w_routed + T * H * 2 + cfg.R * I * 2 + shared1
    assert la["ffn2"]["flops"] == acc["ffn2"]["flops"] + 2 * T * I * H
    # fp8 layers keep the separate shared stage; their expand stage quantizes each token once
    # (x read, T x H codes and T x H/128 scales written) and ffn1 gathers T token rows
    c5 = configs.get("c5_skewed_fp8")
    a5 = bench.account(c5, np.full(c5.E, c5.T * c5.k // c5.E))
    l5 = bench.launch_accounting(c5, a5)
    T5, H5 = c5.T, c5.H
    assert "shared" in l5
    assert l5["expand"]["bytes"] == T5 * H5 * 2 + T5 * H5 + T5 * (H5 // 128) * 4
    assert l5["ffn1"]["bytes"] == a5["ffn1"]["bytes"] - (c5.R - T5) * (H5 + (H5 // 128) * 4)


def test_measured_traffic_requires_matching_sources(tmp_path, monkeypatch):
    import hashlib
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "ffn1_wl_hbm_traffic.txt").write_text(
        f"# record\nsources: k.hip\nsource_sha256: {sha}\ntraffic_bytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", "ffn1") == 1234
    assert bench.measured_traffic("other", "ffn1") is None
    src.write_text("kernel v2\n")   # the kernel changed since the counters were taken
    assert bench.measured_traffic("wl", "ffn1") is None
