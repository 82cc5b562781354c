"""Thin ctypes binding of libmoe_mi355x.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors (device memory) or None.  Every step of the layer runs in the HIP
library; torch is used only to own device memory and to name the stream.
A missing library raises immediately: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB names another build of the same library (the host-only
# sanitizer build that the host tests load); by default the in-tree one.
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(PKG, "libmoe_mi355x.so")
# the debug build with device-side index-range checks (same entry points)
LIB_CHECKS_PATH = os.path.join(PKG, "libmoe_mi355x_checks.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EHIP",
          -4: "MOE_ENONFINITE", -5: "MOE_EALIGN"}

# every entry point declared in include/moe.h
ENTRY_POINTS = ("moe_workspace_bytes", "moe_strerror", "moe_device_cu_count", "moe_route",
                "moe_dispatch", "moe_expert_ffn", "moe_ffn_gate_up", "moe_ffn_down",
                "moe_combine", "moe_pid_update", "moe_balance_update", "moe_dispatch_noalloc",
                "moe_eplb_plan", "moe_debug_checks")

# bits of moe_debug_checks
CHECK_BITS = {1 << 0: "MOE_CHECK_ROUTE_ID", 1 << 1: "MOE_CHECK_DISPATCH_ID",
              1 << 2: "MOE_CHECK_DISPATCH_POS", 1 << 3: "MOE_CHECK_GEMM_ROW",
              1 << 4: "MOE_CHECK_GEMM_ITEMS", 1 << 5: "MOE_CHECK_GEMM_TILE",
              1 << 6: "MOE_CHECK_COMBINE_ROW"}


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_ffn", ctypes.c_int32),
                ("n_zero", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("routed_scaling", ctypes.c_float)]


class MoePidParams(ctypes.Structure):
    _fields_ = [("setpoint", ctypes.c_float), ("kp", ctypes.c_float), ("ki", ctypes.c_float),
                ("kd", ctypes.c_float)]


class MoeError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}: {text}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_moe_layer_03_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sp = ctypes.POINTER(MoeShape)
        L.moe_workspace_bytes.argtypes, L.moe_workspace_bytes.restype = [sp], sz
        L.moe_strerror.argtypes, L.moe_strerror.restype = [ctypes.c_int], ctypes.c_char_p
        L.moe_device_cu_count.argtypes, L.moe_device_cu_count.restype = [], ctypes.c_int
        L.moe_route.argtypes = [sp] + [vp] * 9
        L.moe_dispatch.argtypes = [sp] + [vp] * 9
        L.moe_expert_ffn.argtypes = [sp] + [vp] * 10
        L.moe_ffn_gate_up.argtypes = [sp] + [vp] * 8
        L.moe_ffn_down.argtypes = [sp] + [vp] * 5
        L.moe_combine.argtypes = [sp] + [vp] * 7
        L.moe_pid_update.argtypes = [sp, ctypes.POINTER(MoePidParams), vp, vp, vp, vp, i32, vp]
        L.moe_balance_update.argtypes = [sp, ctypes.c_float, vp, vp, vp]
        L.moe_dispatch_noalloc.argtypes = [sp] + [vp] * 8
        L.moe_eplb_plan.argtypes = [sp, i32, i32] + [vp] * 8
        L.moe_debug_checks.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        for n in ENTRY_POINTS[3:]:
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def make_shape(T, d_model, n_ffn, n_zero, d_ff, top_k, dtype, routed_scaling=1.0) -> MoeShape:
    if isinstance(dtype, torch.dtype):
        dtype = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    elif isinstance(dtype, str):
        dtype = MOE_BF16 if dtype == "bf16" else MOE_F32
    return MoeShape(T, d_model, n_ffn, n_zero, d_ff, top_k, dtype, routed_scaling)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc, lib().moe_strerror(rc).decode())


def moe_workspace_bytes(shape: MoeShape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def moe_device_cu_count() -> int:
    return int(lib().moe_device_cu_count())


def moe_route(shape, x, w_router, logit_bias, bias, topk_idx, topk_gate, logits_out, ws,
              stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(shape), _p(x), _p(w_router), _p(logit_bias),
                                        _p(bias), _p(topk_idx), _p(topk_gate), _p(logits_out),
                                        _p(ws), _stream(stream)))


def moe_dispatch(shape, topk_idx, x, counts, offsets, perm, inv_perm, x_perm, ws, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(shape), _p(topk_idx), _p(x),
                                              _p(counts), _p(offsets), _p(perm), _p(inv_perm),
                                              _p(x_perm), _p(ws), _stream(stream)))


def moe_dispatch_noalloc(shape, topk_idx, x, counts, offsets, perm, inv_perm, x_perm,
                         stream=None):
    _check("moe_dispatch_noalloc",
           lib().moe_dispatch_noalloc(ctypes.byref(shape), _p(topk_idx), _p(x), _p(counts),
                                      _p(offsets), _p(perm), _p(inv_perm), _p(x_perm),
                                      _stream(stream)))


def moe_expert_ffn(shape, x, x_perm, perm, offsets, w_gate, w_up, w_down, y_perm, ws,
                   stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(shape), _p(x), _p(x_perm),
                                                  _p(perm), _p(offsets), _p(w_gate), _p(w_up),
                                                  _p(w_down), _p(y_perm), _p(ws),
                                                  _stream(stream)))


def moe_ffn_gate_up(shape, x, x_perm, perm, offsets, w_gate, w_up, ws, stream=None):
    _check("moe_ffn_gate_up", lib().moe_ffn_gate_up(ctypes.byref(shape), _p(x), _p(x_perm),
                                                    _p(perm), _p(offsets), _p(w_gate), _p(w_up),
                                                    _p(ws), _stream(stream)))


def moe_ffn_down(shape, offsets, w_down, y_perm, ws, stream=None):
    _check("moe_ffn_down", lib().moe_ffn_down(ctypes.byref(shape), _p(offsets), _p(w_down),
                                              _p(y_perm), _p(ws), _stream(stream)))


def moe_combine(shape, x, y_perm, topk_idx, topk_gate, inv_perm, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(shape), _p(x), _p(y_perm), _p(topk_idx),
                                            _p(topk_gate), _p(inv_perm), _p(y), _stream(stream)))


def moe_pid_update(shape, params: MoePidParams, counts, state, bias, r_log=None, r_log_len=0,
                   stream=None):
    _check("moe_pid_update", lib().moe_pid_update(ctypes.byref(shape), ctypes.byref(params),
                                                  _p(counts), _p(state), _p(bias), _p(r_log),
                                                  int(r_log_len), _stream(stream)))


def moe_balance_update(shape, gamma, counts, bias, stream=None):
    _check("moe_balance_update", lib().moe_balance_update(ctypes.byref(shape), float(gamma),
                                                          _p(counts), _p(bias), _stream(stream)))


def moe_eplb_plan(shape, n_slots, n_devices, counts, offsets, replicas, slot_expert, slot_rows,
                  slot_device, device_load, stream=None):
    _check("moe_eplb_plan",
           lib().moe_eplb_plan(ctypes.byref(shape), int(n_slots), int(n_devices), _p(counts),
                               _p(offsets), _p(replicas), _p(slot_expert), _p(slot_rows),
                               _p(slot_device), _p(device_load), _stream(stream)))


def moe_debug_checks(clear=True) -> int:
    """The failed device-check bits since the last clearing call (debug
    build); raises MoeError with MOE_EUNSUPPORTED on a release build."""
    v = ctypes.c_uint32(0)
    _check("moe_debug_checks", lib().moe_debug_checks(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


class LayerBuffers:
    """Device buffers for one layer shape (routing arrays, workspace, outputs).

    ``pid_state`` is a 16-byte moe_pid_state viewed as int32[4] (fields 0 and
    1 hold float bit patterns)."""

    def __init__(self, shape: MoeShape, device="cuda", x_perm=False):
        E = shape.n_ffn + shape.n_zero
        Tk = shape.T * shape.top_k
        dt = torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32
        i32 = dict(dtype=torch.int32, device=device)
        self.shape = shape
        self.topk_idx = torch.empty((shape.T, shape.top_k), **i32)
        self.topk_gate = torch.empty((shape.T, shape.top_k), dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(Tk, **i32)
        self.inv_perm = torch.empty(Tk, **i32)
        self.x_perm = torch.empty((Tk, shape.d_model), dtype=dt, device=device) if x_perm else None
        self.y_perm = torch.empty((Tk, shape.d_model), dtype=dt, device=device)
        self.y = torch.empty((shape.T, shape.d_model), dtype=dt, device=device)
        self.ws = torch.empty(max(moe_workspace_bytes(shape), 256), dtype=torch.uint8,
                              device=device)
        self.pid_state = torch.zeros(4, **i32)


def layer_forward(buf: LayerBuffers, x, w_router, bias, w_gate, w_up, w_down, logit_bias=None,
                  logits_out=None, stream=None):
    """route -> dispatch -> expert FFN -> combine; outputs land in ``buf``."""
    s = buf.shape
    moe_route(s, x, w_router, logit_bias, bias, buf.topk_idx, buf.topk_gate, logits_out, buf.ws,
              stream)
    moe_dispatch(s, buf.topk_idx, x, buf.counts, buf.offsets, buf.perm, buf.inv_perm,
                 buf.x_perm, buf.ws, stream)
    moe_expert_ffn(s, x, buf.x_perm, buf.perm, buf.offsets, w_gate, w_up, w_down, buf.y_perm,
                   buf.ws, stream)
    moe_combine(s, x, buf.y_perm, buf.topk_idx, buf.topk_gate, buf.inv_perm, buf.y, stream)
    return buf.y
