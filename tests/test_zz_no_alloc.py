"""moe_layer_static (the layer on the library's fixed per-GPU scratch array, no workspace
argument, no allocation) against moe_layer on the same inputs: every output bit for bit,
on two calls in a row, the second with fewer tokens (the array keeps the first call's
contents)."""
import ctypes

import numpy as np
import pytest
import torch

from synth import configs
from synth.device import upload_layer
from tests.gpu_helpers import empty_act, host, poison_, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


def outputs(cfg, T):
    out = poison_(empty_act((T, cfg.H), cfg.act))
    idx = poison_(torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"))
    w = poison_(torch.empty((T, cfg.k), dtype=torch.float32, device="cuda"))
    logits = poison_(torch.empty((T, cfg.E), dtype=torch.float32, device="cuda"))
    return out, idx, w, logits


@pytest.mark.parametrize("name", ["c4_decode_bf16", "c10_decode_fp8"])
def test_static_scratch_layer_matches_moe_layer(M, name):
    cfg = configs.get(name)
    say("static scratch layer", name, "upload")
    g = upload_layer(cfg)
    W = M.weights_of(g)
    for T in (cfg.T, 17):               # second call: fewer tokens than the first
        s = M.shape(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
        assert 0 < M.moe_workspace_bytes(s) <= M.MOE_STATIC_SCRATCH_BYTES
        x = g["x"][:T].contiguous()
        say("static scratch layer", name, f"T={T}")
        ref = outputs(cfg, T)
        ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
        M.moe_layer(s, W, x, *ref, ws)
        got = outputs(cfg, T)
        M.moe_layer_static(s, W, x, *got)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert np.array_equal(host(a), host(b)), (name, T)
        # without the optional outputs (they stay in the array) the layer output is the same
        out2 = poison_(empty_act((T, cfg.H), cfg.act))
        M.moe_layer_static(s, W, x, out2, None, None, None)
        torch.cuda.synchronize()
        assert np.array_equal(host(out2), host(ref[0]))
    # a shape whose workspace exceeds the array is refused before anything is enqueued
    big = M.shape(4096, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    assert M.moe_workspace_bytes(big) > M.MOE_STATIC_SCRATCH_BYTES
    st = M.lib().moe_layer_static(ctypes.byref(big), ctypes.byref(W), None, None, None, None, None, None)
    assert st == M.MOE_EWORKSPACE
    del g
    torch.cuda.empty_cache()
