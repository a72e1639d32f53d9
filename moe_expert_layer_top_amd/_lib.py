"""ctypes binding of ``libmoe.so`` -- argument marshalling only.

Every step of the layer runs in the HIP kernels behind the C ABI declared in
``include/moe.h``; this module converts torch tensors to device pointers and the
current torch stream to a ``hipStream_t``, and raises on a non-OK status.  It
never computes anything itself, and it fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so libmoe.so binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_EDEVICE = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_INT8, MOE_INT4 = 3, 4
DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "int8": MOE_INT8, "int4": MOE_INT4}

EXPORTS = [
    "moe_workspace_bytes", "moe_grouped_ffn_workspace_bytes", "moe_gate_topk", "moe_gate_topk_ex",
    "moe_init_routing", "moe_grouped_ffn", "moe_finalize_routing", "moe_layer", "moe_layer_ex",
    "moe_layer_overlap", "moe_layer_profiled", "moe_get_error", "moe_status_str",
    "moe_layer_plan_of", "moe_grouped_ffn_gathered", "moe_layer_static",
]
MOE_STATIC_SCRATCH_BYTES = 64 << 20
SCORING = {"sigmoid": 0, "softmax": 1}
EV_NAMES = ["start", "gate", "topk", "route", "expand", "plan", "ffn1", "ffn2", "shared", "finalize"]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("act", ctypes.c_int32), ("wt", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("sh_w13", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("sh_w13_scale", ctypes.c_void_p),
                ("sh_w2_scale", ctypes.c_void_p)]


class moe_layer_plan(ctypes.Structure):
    _fields_ = [("shared_merged", ctypes.c_int32), ("rows_gathered", ctypes.c_int32),
                ("ffn1_splits", ctypes.c_int32), ("ffn2_splits", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("ffn2_tiles_per_wg", ctypes.c_int32)]


def moe_layer_plan_of(s) -> dict:
    """The layer's launch plan for shape s (host-side; see include/moe.h)."""
    p = moe_layer_plan()
    _check(lib().moe_layer_plan_of(ctypes.byref(s), ctypes.byref(p)), "moe_layer_plan_of")
    return {f: int(getattr(p, f)) for f, _ in moe_layer_plan._fields_}


class moe_router(ctypes.Structure):
    _fields_ = [("scoring", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("group_topn", ctypes.c_int32), ("scale", ctypes.c_float)]


def router(scoring="sigmoid", renormalize=True, n_group=1, topk_group=1, group_topn=1, scale=1.0) -> moe_router:
    """A router variant (include/moe.h); the defaults are the plain router."""
    return moe_router(SCORING[scoring], int(bool(renormalize)), n_group, topk_group, group_topn, scale)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m moe_expert_layer_top_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_size_t
        sig = {
            "moe_workspace_bytes": (SZ, [S]),
            "moe_grouped_ffn_workspace_bytes": (SZ, [S, I32, I32]),
            "moe_gate_topk": (I32, [S, P, P, P, P, P, P, P, SZ, P]),
            "moe_gate_topk_ex": (I32, [S, ctypes.POINTER(moe_router), P, P, P, P, P, P, P, SZ, P]),
            "moe_init_routing": (I32, [S, P, P, I32, P, P, P, P, P, P, P, SZ, P]),
            "moe_grouped_ffn": (I32, [S, I32, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_finalize_routing": (I32, [S, P, P, P, P, P, P]),
            "moe_layer": (I32, [S, ctypes.POINTER(moe_weights), P, P, P, P, P, P, SZ, P]),
            "moe_layer_overlap": (I32, [S, ctypes.POINTER(moe_weights), P, P, P, P, P, P, SZ, P, P]),
            "moe_layer_ex": (I32, [S, ctypes.POINTER(moe_router), ctypes.POINTER(moe_weights), P, P, P, P, P,
                                   P, SZ, P, P]),
            "moe_layer_profiled": (I32, [S, ctypes.POINTER(moe_weights), P, P, P, P, P, P, SZ, P, P,
                                         ctypes.POINTER(ctypes.c_void_p), I32]),
            "moe_get_error": (I32, [P, P]),
            "moe_status_str": (ctypes.c_char_p, [I32]),
            "moe_layer_plan_of": (I32, [S, ctypes.POINTER(moe_layer_plan)]),
            "moe_grouped_ffn_gathered": (I32, [S, I32, I32, P, I32, P, P, I32, P, P, P, P, P, P, P, SZ, P]),
            "moe_layer_static": (I32, [S, ctypes.POINTER(moe_weights), P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def shape(T, H, E, k, I, I_shared, act="bf16", wt="bf16") -> moe_shape:
    return moe_shape(int(T), int(H), int(E), int(k), int(I), int(I_shared),
                     DTYPE_CODES[act] if isinstance(act, str) else int(act),
                     DTYPE_CODES[wt] if isinstance(wt, str) else int(wt))


def shape_of(cfg) -> moe_shape:
    """moe_shape of a workload configuration (synth.configs.MoEConfig)."""
    return shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.wt)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoEError(st, where)


def moe_workspace_bytes(s: moe_shape) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(s))


def moe_grouped_ffn_workspace_bytes(s: moe_shape, G: int, R_max: int) -> int:
    return lib().moe_grouped_ffn_workspace_bytes(ctypes.byref(s), int(G), int(R_max))


def moe_gate_topk(s, x, w_gate, bias, logits, topk_idx, topk_w, ws, stream=None):
    _check(lib().moe_gate_topk(ctypes.byref(s), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(logits),
                               _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "moe_gate_topk")


def moe_gate_topk_ex(s, rt, x, w_gate, bias, logits, topk_idx, topk_w, ws, stream=None):
    """moe_gate_topk with a router variant `rt` (moe_router or None)."""
    _check(lib().moe_gate_topk_ex(ctypes.byref(s), None if rt is None else ctypes.byref(rt), _ptr(x),
                                  _ptr(w_gate), _ptr(bias), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_gate_topk_ex")


def moe_init_routing(s, x, ids, e_base, expanded_x, expanded_scale, expanded_row_idx, sorted_src,
                     tokens_per_expert, expert_offsets, ws, stream=None):
    _check(lib().moe_init_routing(ctypes.byref(s), _ptr(x), _ptr(ids), int(e_base), _ptr(expanded_x),
                                  _ptr(expanded_scale), _ptr(expanded_row_idx), _ptr(sorted_src),
                                  _ptr(tokens_per_expert), _ptr(expert_offsets), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "moe_init_routing")


def moe_grouped_ffn(s, G, R_max, a, a_scale, group_offsets, w13, w13_scale, w2, w2_scale, y, ws,
                    stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(s), int(G), int(R_max), _ptr(a), _ptr(a_scale),
                                 _ptr(group_offsets), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                 _ptr(w2_scale), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_grouped_ffn")


def moe_grouped_ffn_gathered(s, G, R_max, a, a_rows, a_scale, row_of, row_div, group_offsets, w13,
                             w13_scale, w2, w2_scale, y, ws, stream=None):
    _check(lib().moe_grouped_ffn_gathered(ctypes.byref(s), int(G), int(R_max), _ptr(a), int(a_rows),
                                          _ptr(a_scale), _ptr(row_of), int(row_div), _ptr(group_offsets),
                                          _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(y),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_grouped_ffn_gathered")


def moe_finalize_routing(s, y, skip, topk_w, expanded_row_idx, out, stream=None):
    _check(lib().moe_finalize_routing(ctypes.byref(s), _ptr(y), _ptr(skip), _ptr(topk_w),
                                      _ptr(expanded_row_idx), _ptr(out), _stream(stream)),
           "moe_finalize_routing")


def weights(w_gate, w13, w2, sh_w13, sh_w2, w13_scale=None, w2_scale=None, bias=None,
            sh_w13_scale=None, sh_w2_scale=None) -> moe_weights:
    return moe_weights(_ptr(w_gate), _ptr(w13), _ptr(w2), _ptr(sh_w13), _ptr(sh_w2),
                       _ptr(w13_scale), _ptr(w2_scale), _ptr(bias), _ptr(sh_w13_scale),
                       _ptr(sh_w2_scale))


def weights_of(g: dict) -> moe_weights:
    """moe_weights from a dict of device tensors named as the layer's inputs (w_gate, w13,
    w2, sh_w13, sh_w2 and, where present, w13_scale, w2_scale, bias, sh_w13_scale,
    sh_w2_scale)."""
    return weights(g.get("w_gate"), g["w13"], g["w2"], g["sh_w13"], g["sh_w2"],
                   g.get("w13_scale"), g.get("w2_scale"), g.get("bias"), g.get("sh_w13_scale"),
                   g.get("sh_w2_scale"))


def moe_layer(s, w: moe_weights, x, out, topk_idx, topk_w, logits, ws, stream=None):
    _check(lib().moe_layer(ctypes.byref(s), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)), "moe_layer")


def moe_layer_static(s, w: moe_weights, x, out, topk_idx, topk_w, logits, stream=None):
    """moe_layer on the library's fixed per-GPU scratch array (no workspace argument)."""
    _check(lib().moe_layer_static(ctypes.byref(s), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(logits), _stream(stream)), "moe_layer_static")


def moe_layer_ex(s, rt, w: moe_weights, x, out, topk_idx, topk_w, logits, ws, side=None, stream=None):
    """The general layer call: router variant `rt` (or None) and an optional side stream."""
    _check(lib().moe_layer_ex(ctypes.byref(s), None if rt is None else ctypes.byref(rt), ctypes.byref(w),
                              _ptr(x), _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream),
                              None if side is None else _stream(side)), "moe_layer_ex")


def moe_layer_overlap(s, w: moe_weights, x, out, topk_idx, topk_w, logits, ws, side, stream=None):
    """moe_layer with the shared expert's own launches on `side` (a torch.cuda.Stream)."""
    _check(lib().moe_layer_overlap(ctypes.byref(s), ctypes.byref(w), _ptr(x), _ptr(out),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream),
                                   None if side is None else _stream(side)), "moe_layer_overlap")


def moe_layer_profiled(s, w: moe_weights, x, out, topk_idx, topk_w, logits, ws, events,
                       side=None, stream=None):
    """moe_layer_overlap (side=None: moe_layer) recording `events` (torch.cuda.Event,
    already created) at its launch boundaries, in the order of EV_NAMES."""
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(lib().moe_layer_profiled(ctypes.byref(s), ctypes.byref(w), _ptr(x), _ptr(out),
                                    _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream),
                                    None if side is None else _stream(side), arr,
                                    len(events)), "moe_layer_profiled")


def moe_get_error(ws, stream=None) -> int:
    """MOE_OK or MOE_EDEVICE for the last routing call on this workspace (synchronizes)."""
    st = lib().moe_get_error(_ptr(ws), _stream(stream))
    if st not in (MOE_OK, MOE_EDEVICE):
        raise MoEError(st, "moe_get_error")
    return st


def moe_status_str(st: int) -> str:
    return status_str(st)
