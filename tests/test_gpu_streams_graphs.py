"""The layer with its shared expert on a second stream, and the layer captured in a HIP
graph, against the plain single-stream call.

All three run the same kernels on the same inputs, so every output (out, top-k ids and
weights, logits) must match the single-stream call bit for bit.  The layer itself is
checked against the oracle in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

from synth import configs
from tests.gpu_helpers import empty_act, host, poison_, say
from tests.test_gpu_parity import case

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

# fp32 and fp8 layers and I_shared != I run the shared expert in launches of its own (the
# side stream is used); p2 has it inside the routed launches (the side stream is not).
# p6: the int8 shared expert is a group of the routed launches (side unused); p9: the int8
# shared expert of a W4A8 layer quantizes x itself on the side stream; p10, p11: split-K
# expert GEMMs with the shared expert (also split) on the side stream
OVERLAP = ["p1_small_fp32", "p2_prefill_bf16", "p2c_prefill_bf16", "p5_skewed_fp8",
           "p6_prefill_w8a8", "p9_decode_w4a8", "p10_split_bf16", "p11_split_fp8"]


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_layer_top_amd as m
    m.lib()
    return m


def layer_bufs(M, cfg, T=None):
    T = cfg.T if T is None else T
    s = M.shape(T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)
    b = {
        "out": poison_(empty_act((T, cfg.H), cfg.act)),
        "idx": poison_(torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")),
        "w": poison_(torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")),
        "logits": poison_(torch.empty((T, cfg.E), dtype=torch.float32, device="cuda")),
        # poisoned workspace: a missing join would let finalize read an unwritten
        # shared-expert output
        "ws": poison_(torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")),
    }
    return s, b


def weights_of(M, g):
    return M.weights_of(g)


def outputs(b):
    return [host(b[k]).copy() for k in ("out", "idx", "w", "logits")]


def assert_same(a, b):
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("name", OVERLAP)
def test_overlap_matches_single_stream(M, name):
    cfg, d, g = case(name)
    say("overlap", name)
    W = weights_of(M, g)
    s, ref = layer_bufs(M, cfg)
    M.moe_layer(s, W, g["x"], ref["out"], ref["idx"], ref["w"], ref["logits"], ref["ws"])
    torch.cuda.synchronize()
    want = outputs(ref)
    side = torch.cuda.Stream()
    for rep in range(2):
        s, b = layer_bufs(M, cfg)
        torch.cuda.synchronize()
        M.moe_layer_overlap(s, W, g["x"], b["out"], b["idx"], b["w"], b["logits"], b["ws"], side)
        # read the output through the calling stream only: it must already wait for the
        # side stream's shared expert
        got_out = b["out"].clone()
        torch.cuda.synchronize()
        got = outputs(b)
        got[0] = host(got_out)
        assert_same(got, want)
    # side == NULL behaves as moe_layer
    s, b = layer_bufs(M, cfg)
    M.moe_layer_overlap(s, W, g["x"], b["out"], b["idx"], b["w"], b["logits"], b["ws"], None)
    torch.cuda.synchronize()
    assert_same(outputs(b), want)


def new_x(cfg, g, seed):
    """Another input of the same shape and distribution: the workload's rows, permuted."""
    p = torch.randperm(cfg.T, generator=torch.Generator().manual_seed(seed))
    return g["x"][p.to(g["x"].device)].contiguous()


@pytest.mark.parametrize("name,overlap", [("p2_prefill_bf16", False), ("p5_skewed_fp8", False),
                                          ("p5_skewed_fp8", True), ("p4_decode_bf16", False),
                                          ("p6_prefill_w8a8", False), ("p9_decode_w4a8", True),
                                          ("p12_split_w8a8", True)])
def test_layer_graph_replay(M, name, overlap):
    """Capture the layer once, then replay it on new inputs written into the captured
    input buffer, with eager calls and synchronizations between replays; every replay
    equals the eager call on the same input."""
    cfg, d, g = case(name)
    say("graph", name, "overlap" if overlap else "one stream")
    W = weights_of(M, g)
    x_static = g["x"].clone()
    s, b = layer_bufs(M, cfg)
    side = torch.cuda.Stream() if overlap else None

    def call(x, bufs, stream_side):
        if stream_side is None:
            M.moe_layer(s, W, x, bufs["out"], bufs["idx"], bufs["w"], bufs["logits"], bufs["ws"])
        else:
            M.moe_layer_overlap(s, W, x, bufs["out"], bufs["idx"], bufs["w"], bufs["logits"],
                                bufs["ws"], stream_side)

    # warm up outside the capture, on a side stream as torch's capture expects
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        call(x_static, b, side)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x_static, b, side)
    torch.cuda.synchronize()
    for rep in range(3):
        x = g["x"] if rep == 0 else new_x(cfg, g, rep)
        x_static.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs(b)
        # eager reference on the same input, with buffers and workspace of its own
        _, e = layer_bufs(M, cfg)
        call(x, e, None)
        torch.cuda.synchronize()
        assert_same(got, outputs(e))
        say(f"  replay {rep} matches the eager call")
    del graph
    torch.cuda.synchronize()


def test_overlap_full_c5(M):
    """c5 at full size (the bench's launch configuration): the two-stream call equals the
    single-stream call bit for bit."""
    from synth.device import upload_layer
    cfg = configs.get("c5_skewed_fp8")
    say("overlap c5 full: upload")
    g = upload_layer(cfg)
    W = weights_of(M, g)
    say("overlap c5 full: run")
    s, ref = layer_bufs(M, cfg)
    M.moe_layer(s, W, g["x"], ref["out"], ref["idx"], ref["w"], ref["logits"], ref["ws"])
    torch.cuda.synchronize()
    want = outputs(ref)
    del ref
    side = torch.cuda.Stream()
    s, b = layer_bufs(M, cfg)
    M.moe_layer_overlap(s, W, g["x"], b["out"], b["idx"], b["w"], b["logits"], b["ws"], side)
    torch.cuda.synchronize()
    assert_same(outputs(b), want)
    del g, b
    torch.cuda.empty_cache()
