"""The C-ABI library loads and exports every entry point of include/moe.h, and its
host-side validation answers without touching a GPU (nothing here launches work)."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_expert_layer_top_amd as M
from moe_expert_layer_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(moe_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_status_strings(L):
    for st in (M.MOE_OK, M.MOE_EINVAL, M.MOE_EUNSUPPORTED, M.MOE_EWORKSPACE, M.MOE_EHIP, M.MOE_EDEVICE):
        assert M.moe_status_str(st) and M.moe_status_str(st) != "unknown status"
    assert M.moe_status_str(99) == "unknown status"


def test_workspace_query(L):
    c2 = M.shape(8192, 7168, 256, 8, 2048, 2048, "bf16", "bf16")
    n = M.moe_workspace_bytes(c2)
    # the routed outputs (R x H bf16); a bf16 layer gathers its routed rows from x and
    # keeps no expanded copy of them
    assert 65536 * 7168 * 2 <= n < 2 * 65536 * 7168 * 2
    # an fp8 layer quantizes each token once (T x H codes) and gathers its routed rows from
    # them: no expanded copy either
    c5 = M.shape(8192, 7168, 256, 8, 2048, 2048, "bf16", "fp8")
    assert 65536 * 7168 * 2 + 8192 * 7168 <= M.moe_workspace_bytes(c5) < 65536 * 7168 * (2 + 1)
    small = M.shape(100, 7168, 256, 8, 2048, 2048, "bf16", "bf16")
    assert 0 < M.moe_workspace_bytes(small) < n
    assert M.moe_workspace_bytes(M.shape(8, 128, 4, 5, 128, 128)) == 0          # k > E
    assert M.moe_workspace_bytes(M.shape(8, 100, 4, 2, 128, 128)) == 0          # H % 128
    assert M.moe_workspace_bytes(M.shape(8, 128, 4, 2, 100, 128)) == 0          # I % 128
    assert M.moe_workspace_bytes(M.shape(8, 128, 4, 2, 128, 128, "f32", "bf16")) == 0
    assert M.moe_workspace_bytes(M.shape(8, 128, 4, 2, 128, 128, "bf16", "fp8")) > 0
    assert M.moe_grouped_ffn_workspace_bytes(c2, 256, 65536) > 65536 * 2048 * 2
    # W8A8: per-token int8 codes (T x H) and row scales, gathered like fp8; h staged in bf16
    # and quantized per row
    c6 = M.shape(8192, 7168, 256, 8, 2048, 2048, "bf16", "int8")
    assert M.moe_workspace_bytes(c6) >= 65536 * 7168 * 2 + 8192 * 7168 + 65536 * 2048 * (2 + 1)
    assert M.moe_layer_plan_of(c6)["rows_gathered"] == 1
    assert M.moe_grouped_ffn_workspace_bytes(c6, 256, 65536) >= 65536 * 2048 * (2 + 1)
    assert M.moe_workspace_bytes(M.shape(8, 128, 4, 2, 128, 128, "f32", "int8")) == 0
    c8 = M.shape(128, 7168, 256, 8, 2048, 2048, "bf16", "int4")
    assert M.moe_workspace_bytes(c8) > 1024 * 7168


DUMMY = ctypes.c_void_p(4096)   # never dereferenced: validation fails first


def test_validation_errors_enqueue_nothing(L):
    s = M.shape(16, 256, 8, 2, 128, 128)
    bad_k = M.shape(16, 256, 8, 9, 128, 128)
    bad_dt = M.shape(16, 256, 8, 2, 128, 128, "f32", "fp8")
    P = [DUMMY] * 6
    assert L.moe_init_routing(None, *[None] * 2, 0, *[None] * 7, 0, None) == M.MOE_EINVAL
    assert L.moe_init_routing(ctypes.byref(bad_k), DUMMY, DUMMY, 0, DUMMY, None, DUMMY, DUMMY, DUMMY,
                              DUMMY, DUMMY, 1 << 30, None) == M.MOE_EINVAL
    assert L.moe_init_routing(ctypes.byref(bad_dt), DUMMY, DUMMY, 0, DUMMY, None, DUMMY, DUMMY, DUMMY,
                              DUMMY, DUMMY, 1 << 30, None) == M.MOE_EUNSUPPORTED
    assert L.moe_init_routing(ctypes.byref(s), DUMMY, DUMMY, 0, DUMMY, None, DUMMY, DUMMY, DUMMY,
                              DUMMY, DUMMY, 16, None) == M.MOE_EWORKSPACE
    assert L.moe_gate_topk(ctypes.byref(s), DUMMY, None, None, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 30,
                           None) == M.MOE_EINVAL
    assert L.moe_grouped_ffn(ctypes.byref(s), 0, 10, *P[:3], DUMMY, None, DUMMY, None, DUMMY, DUMMY,
                             1 << 30, None) == M.MOE_EINVAL
    # more groups than the planner's one thread per group (too small a workspace, so a
    # regression would report EWORKSPACE rather than launch)
    assert L.moe_grouped_ffn(ctypes.byref(s), 1025, 10, *P[:3], DUMMY, None, DUMMY, None, DUMMY, DUMMY,
                             16, None) == M.MOE_EUNSUPPORTED
    assert L.moe_grouped_ffn_gathered(ctypes.byref(s), 1025, 10, DUMMY, 64, None, DUMMY, 1, DUMMY, DUMMY,
                                      None, DUMMY, None, DUMMY, DUMMY, 16, None) == M.MOE_EUNSUPPORTED
    assert M.moe_grouped_ffn_workspace_bytes(s, 1025, 10) == 0
    assert M.moe_grouped_ffn_workspace_bytes(s, 1024, 10) > 0
    fp8 = M.shape(16, 256, 8, 2, 128, 128, "bf16", "fp8")
    assert L.moe_grouped_ffn(ctypes.byref(fp8), 8, 32, DUMMY, None, DUMMY, DUMMY, None, DUMMY, None,
                             DUMMY, DUMMY, 1 << 30, None) == M.MOE_EINVAL   # fp8 needs scales
    assert L.moe_finalize_routing(ctypes.byref(s), None, None, None, DUMMY, DUMMY, None) == M.MOE_EINVAL
    # gathered FFN: row_div >= 1, a row map, no fp32, row offsets of `a` within 32 bits
    gat = [8, 32, DUMMY, 64, None, DUMMY]
    rest = [DUMMY, DUMMY, None, DUMMY, None, DUMMY, DUMMY, 1 << 30, None]
    assert L.moe_grouped_ffn_gathered(ctypes.byref(s), *gat, 0, *rest) == M.MOE_EINVAL
    assert L.moe_grouped_ffn_gathered(ctypes.byref(s), 8, 32, DUMMY, 64, None, None, 1, *rest) == M.MOE_EINVAL
    f32 = M.shape(16, 256, 8, 2, 128, 128, "f32", "f32")
    assert L.moe_grouped_ffn_gathered(ctypes.byref(f32), *gat, 1, *rest) == M.MOE_EUNSUPPORTED
    # the 32-bit lane offsets of `a`: these calls pass a 16-byte workspace, so a call that
    # got past the bound check would stop at the workspace check (MOE_EWORKSPACE) and
    # never launch on the dummy pointers
    tiny = [DUMMY, DUMMY, None, DUMMY, None, DUMMY, DUMMY, 16, None]
    wide = M.shape(16, 8192, 8, 2, 128, 128)
    assert L.moe_grouped_ffn_gathered(ctypes.byref(wide), 8, 32, DUMMY, 1 << 18, None, DUMMY, 1,
                                      *tiny) == M.MOE_EUNSUPPORTED   # 2^18 rows x 16 KB = 4 GiB
    # int8 codes are one byte: the same limit falls at twice the rows
    wide8 = M.shape(16, 8192, 8, 2, 128, 128, "bf16", "int8")
    sc = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 16, None]
    assert L.moe_grouped_ffn_gathered(ctypes.byref(wide8), 8, 32, DUMMY, 1 << 19, DUMMY, DUMMY, 1,
                                      *sc) == M.MOE_EUNSUPPORTED
    # exactly at the limit (H = 128): 2^32 bytes of `a` is refused, 128 bytes fewer is not
    narrow8 = M.shape(16, 128, 8, 2, 128, 128, "bf16", "int8")
    assert L.moe_grouped_ffn_gathered(ctypes.byref(narrow8), 8, 32, DUMMY, 1 << 25, DUMMY, DUMMY, 1,
                                      *sc) == M.MOE_EUNSUPPORTED
    assert L.moe_grouped_ffn_gathered(ctypes.byref(narrow8), 8, 32, DUMMY, (1 << 25) - 1, DUMMY, DUMMY, 1,
                                      *sc) == M.MOE_EWORKSPACE
    narrow = M.shape(16, 128, 8, 2, 128, 128)
    assert L.moe_grouped_ffn_gathered(ctypes.byref(narrow), 8, 32, DUMMY, 1 << 24, None, DUMMY, 1,
                                      *tiny) == M.MOE_EUNSUPPORTED
    assert L.moe_grouped_ffn_gathered(ctypes.byref(narrow), 8, 32, DUMMY, (1 << 24) - 1, None, DUMMY, 1,
                                      *tiny) == M.MOE_EWORKSPACE
    assert L.moe_grouped_ffn_gathered(ctypes.byref(fp8), 8, 32, DUMMY, 64, None, DUMMY, 1, DUMMY, DUMMY,
                                      None, DUMMY, None, DUMMY, DUMMY, 1 << 30, None) == M.MOE_EINVAL
    w = M.moe_weights()
    assert L.moe_layer(ctypes.byref(s), ctypes.byref(w), DUMMY, DUMMY, None, None, None, DUMMY, 1 << 30,
                       None) == M.MOE_EINVAL
    assert L.moe_get_error(None, None) == M.MOE_EINVAL


def test_misaligned_pointers_are_rejected(L):
    """Tensor pointers must be 16-byte aligned: one that is not is MOE_EINVAL before
    anything is enqueued.  Every call passes a 16-byte workspace, so a call that got past
    the alignment check would stop at the workspace check (MOE_EWORKSPACE) and never
    launch on the dummy pointers."""
    s = M.shape(16, 256, 8, 2, 128, 128)
    off = ctypes.c_void_p(DUMMY.value + 8)

    def each_misaligned(args, call):
        for i, a in enumerate(args):
            if a is None:
                continue
            bad = list(args)
            bad[i] = off
            assert call(bad) == M.MOE_EINVAL, i
        assert call(args) == M.MOE_EWORKSPACE

    # x, w_gate, bias, logits, topk_idx, topk_w, ws
    each_misaligned([DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY],
                    lambda a: L.moe_gate_topk(ctypes.byref(s), *a, 16, None))
    # x, ids | expanded_x, expanded_scale, expanded_row_idx, sorted_src, counts, offsets, ws
    each_misaligned([DUMMY, DUMMY, DUMMY, None, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY],
                    lambda a: L.moe_init_routing(ctypes.byref(s), a[0], a[1], 0, *a[2:], 16, None))
    # a, a_scale, offsets, w13, w13_scale, w2, w2_scale, y, ws
    each_misaligned([DUMMY, None, DUMMY, DUMMY, None, DUMMY, None, DUMMY, DUMMY],
                    lambda a: L.moe_grouped_ffn(ctypes.byref(s), 8, 32, *a, 16, None))
    fp8 = M.shape(16, 256, 8, 2, 128, 128, "bf16", "fp8")
    each_misaligned([DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY],
                    lambda a: L.moe_grouped_ffn(ctypes.byref(fp8), 8, 32, *a, 16, None))
    # a | a_scale, row_of | offsets, w13, w13_scale, w2, w2_scale, y, ws
    each_misaligned([DUMMY, None, DUMMY, DUMMY, DUMMY, None, DUMMY, None, DUMMY, DUMMY],
                    lambda a: L.moe_grouped_ffn_gathered(ctypes.byref(s), 8, 32, a[0], 64, a[1], a[2], 1,
                                                         *a[3:], 16, None))

    # the layer: its own pointers, then each weight pointer
    def layer(a):
        w = M.moe_weights(*a[4:])
        return L.moe_layer(ctypes.byref(s), ctypes.byref(w), a[0], a[1], a[2], a[3], None, DUMMY, 16, None)
    each_misaligned([DUMMY, DUMMY, DUMMY, DUMMY] + [DUMMY] * 5 + [None, None, DUMMY, None, None], layer)


def test_router_validation_enqueues_nothing(L):
    """Invalid router variants are rejected on the host (MOE_EINVAL) before any launch."""
    s = M.shape(16, 256, 16, 4, 128, 128)
    ws_big = 1 << 30
    bad = [M.router(n_group=3),                       # does not divide E
           M.router(n_group=4, topk_group=5),         # more groups kept than exist
           M.router(n_group=16, group_topn=2),        # groups of one expert have no second best
           M.router(n_group=8, topk_group=1),         # k = 4 > 1 group of 2 experts
           M.router(n_group=128),                     # above 64 groups
           M.router(scale=0.0), M.router(scale=float("inf")),
           M.moe_router(7, 1, 1, 1, 1, 1.0),          # unknown scoring
           M.moe_router(0, 2, 1, 1, 1, 1.0)]          # renormalize not 0/1
    for r in bad:
        assert L.moe_gate_topk_ex(ctypes.byref(s), ctypes.byref(r), DUMMY, DUMMY, None, DUMMY, DUMMY, DUMMY,
                                  DUMMY, ws_big, None) == M.MOE_EINVAL
        w = M.moe_weights(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, None, None)
        assert L.moe_layer_ex(ctypes.byref(s), ctypes.byref(r), ctypes.byref(w), DUMMY, DUMMY, None, None,
                              None, DUMMY, ws_big, None, None) == M.MOE_EINVAL
    good = M.router(scoring="softmax", n_group=4, topk_group=2, group_topn=2, scale=2.5)
    # a valid router reaches the workspace check (still nothing launched)
    assert L.moe_gate_topk_ex(ctypes.byref(s), ctypes.byref(good), DUMMY, DUMMY, None, DUMMY, DUMMY, DUMMY,
                              DUMMY, 16, None) == M.MOE_EWORKSPACE


def test_layer_plan_query(L):
    """moe_layer_plan_of describes the launch plan from the shape alone (host logic)."""
    from synth import configs

    def plan(name, **kw):
        return M.moe_layer_plan_of(M.shape_of(configs.get(name, **kw)))

    p = plan("c2_prefill_bf16")       # prefill: tall tiles, shared expert merged, rows gathered
    assert p == {"shared_merged": 1, "rows_gathered": 1, "ffn1_splits": 1, "ffn2_splits": 1, "block_m": 320,
                 "ffn2_tiles_per_wg": 1}
    # the int8 down projection chains four N tiles per workgroup at the same shape
    assert plan("c6_prefill_w8a8")["ffn2_tiles_per_wg"] == 4
    # 32 experts of 256 rows (int8) and a shared expert of its own shape (not merged): 32
    # units, where two down-projection tiles per workgroup keep a round of workgroups
    # (32 x 14 >= 256 CUs) and four would not
    p = M.moe_layer_plan_of(M.shape(8192, 7168, 32, 1, 2048, 1024, "bf16", "int8"))
    assert p["shared_merged"] == 0 and p["ffn2_tiles_per_wg"] == 2
    assert plan("c5_skewed_fp8")["ffn2_tiles_per_wg"] == 1      # fp8: one tile per workgroup
    assert plan("c4_decode_bf16")["ffn2_tiles_per_wg"] == 1     # decode tiles
    p = plan("c5_skewed_fp8")         # fp8 experts beside a bf16 shared expert; rows gathered
    assert p["shared_merged"] == 0 and p["rows_gathered"] == 1 and p["block_m"] == 256
    assert plan("c6_prefill_w8a8")["shared_merged"] == 1      # int8 shared expert in the int8 launches
    assert plan("c8_decode_w4a8")["shared_merged"] == 0       # int4 experts, int8 shared expert
    p = plan("c4_decode_bf16")        # decode: short tiles, grid large enough not to split
    assert p["block_m"] == 32 and p["ffn1_splits"] == 1 and p["shared_merged"] == 1
    # one token of the DeepSeek shape keeps 128 workgroups per GEMM: no split
    assert plan("c9_decode1_bf16")["ffn1_splits"] == 1
    # a few tokens over long K split the expert GEMMs (the merged shared expert's rows
    # take their own partials)
    p = plan("p10_split_bf16")
    assert p["ffn1_splits"] > 1 and p["ffn2_splits"] > 1 and p["shared_merged"] == 1
    for name in ("p11_split_fp8", "p12_split_w8a8", "p13_split_w4a8"):
        assert plan(name)["ffn1_splits"] > 1, name
    assert plan("p4_decode_bf16")["ffn1_splits"] == 1        # short K: slices would be too thin
    bad = M.shape(8, 100, 16, 2, 128, 128, "bf16", "bf16")   # H not a multiple of 128
    with pytest.raises(M.MoEError):
        M.moe_layer_plan_of(bad)


def test_plan_helpers_on_the_cpu(tmp_path):
    """The work-plan index arithmetic of the planner kernel and the grouped GEMM
    (unit slices, the shared expert's slices spread through the table, per-XCD chunk
    bounds by cost, slot -> (unit, N tile)), compiled from the kernels' own header by the
    host compiler: on 405 unit tables (one dense group, empty and hot groups, more rows
    than the sized bound, random uniform / Zipf-like / clustered counts) every N tile of
    every unit is reached by exactly one workgroup of the launch grid, no XCD's chunk
    exceeds the grid's slots for it, and a run of units is walked N tile major."""
    exe = tmp_path / "plan_check"
    src = os.path.join(ROOT, "tests", "csrc", "plan_check.cpp")
    inc = os.path.join(ROOT, "moe_expert_layer_top_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", inc, src, "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all plan checks passed" in r.stdout


def test_address_helpers_on_the_cpu(tmp_path):
    """The 64-bit base rebuilt from two 32-bit halves (the fp8 scale loads of the grouped
    GEMM) and the 32-bit lane-offset bound, compiled from the kernels' own header by the
    host compiler and checked on the CPU: a low half with bit 31 set must not spill into
    the high half, and the bound must fall exactly at 2^32 bytes."""
    exe = tmp_path / "addr_check"
    src = os.path.join(ROOT, "tests", "csrc", "addr_check.cpp")
    inc = os.path.join(ROOT, "moe_expert_layer_top_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", inc, src, "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all address checks passed" in r.stdout
