"""Dense SwiGLU branch of a shortcut-connected MoE block, run beside the MoE
layer on its own stream.

LongCat-2.0's backbone is built from shortcut-connected blocks (LongCat-2.0
Danish article, section "ScMoE og throughput"; model-summary page, Shape and
Feed-forward: each block holds dense-FFN sublayers of intermediate width
12,288 alongside one MoE).  The Ascend deployment article (section
"计算流并行调度优化") runs MoE and dense work on separate streams in decode,
each stream with its own share of the cores.

The dense FFN is the one-expert case of the grouped expert FFN, so it runs
through the same library entry points: moe_ffn_gate_up / moe_ffn_down with
one FFN expert, no identity experts, top_k = 1, offsets [0, T], and x itself
as the gathered rows.  This module only sets up those arguments, and the
CU-partitioned streams (HIP streams created with a CU mask, at the default
priority) that give each branch its own share of the chip; the library
sizes its persistent grids by the CU mask of the stream it is given.
"""

from __future__ import annotations

import ctypes

import torch

from . import binding as B

_hip = None


def _hiplib():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.c_uint32,
                                                      ctypes.POINTER(ctypes.c_uint32)]
        _hip.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
        _hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipStreamDestroy.restype = ctypes.c_int
    return _hip


def cu_mask(n_cus: int, first: int, count: int, pattern: str = "spread"):
    """Bit mask (list of uint32 words) selecting `count` of `n_cus` CUs, in
    whole pairs of adjacent CUs (2j, 2j+1).  "contiguous": CUs first ..
    first + count - 1 (first rounded down to an even CU); "spread": count / 2
    pairs evenly spaced over the chip, starting at the pair of `first`.  The
    HIP runtime on MI355X has accepted contiguous masks (a range of CUs, or
    16 contiguous CUs of every 32) and refused spread ones (every other CU,
    single CUs or pairs at a stride: hipErrorOutOfMemory at stream creation),
    so the measurements use contiguous masks."""
    if count % 2 or count < 2 or count > n_cus:
        raise ValueError("count must be an even number of CUs, at most n_cus")
    words = [0] * ((n_cus + 31) // 32)
    pairs = n_cus // 2
    p0 = (first // 2) % pairs
    if pattern == "contiguous":
        sel = [(p0 + j) % pairs for j in range(count // 2)]
    else:
        step = pairs / (count // 2)
        sel = sorted({(p0 + int(j * step)) % pairs for j in range(count // 2)})
    for p in sel:
        for c in (2 * p, 2 * p + 1):
            words[c // 32] |= 1 << (c % 32)
    return words


class MaskedStream:
    """A HIP stream restricted to the CUs of `words` (default priority),
    usable as a torch stream; destroyed with close()."""

    def __init__(self, words, device="cuda"):
        arr = (ctypes.c_uint32 * len(words))(*words)
        h = ctypes.c_void_p()
        torch.cuda.current_stream(device)  # the device's context exists first
        rc = _hiplib().hipExtStreamCreateWithCUMask(ctypes.byref(h), len(words), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
        self.handle = h.value
        self.stream = torch.cuda.ExternalStream(self.handle, device=device)
        self.cus = sum(bin(w).count("1") for w in words)

    def close(self):
        if self.handle is not None:
            torch.cuda.synchronize()
            _hiplib().hipStreamDestroy(ctypes.c_void_p(self.handle))
            self.handle = None


class DenseBranch:
    """y = (silu(x W1^T) * (x W3^T)) W2^T for T rows of width d_model."""

    def __init__(self, T: int, d_model: int, d_ff: int, dtype, device="cuda"):
        self.shape = B.make_shape(T, d_model, 1, 0, d_ff, 1, dtype)
        dt = torch.bfloat16 if self.shape.dtype == B.MOE_BF16 else torch.float32
        self.offsets = torch.tensor([0, T], dtype=torch.int32, device=device)
        self.ws = torch.empty(max(B.moe_workspace_bytes(self.shape), 256), dtype=torch.uint8,
                              device=device)
        self.y = torch.empty((T, d_model), dtype=dt, device=device)

    def run(self, x, w1, w3, w2, stream=None):
        """Enqueue the branch on ``stream`` (default: torch's current stream);
        w1, w3 [d_ff, d_model], w2 [d_model, d_ff].  Returns self.y."""
        B.moe_ffn_gate_up(self.shape, None, x, None, self.offsets, w1, w3, self.ws, stream)
        B.moe_ffn_down(self.shape, self.offsets, w2, self.y, self.ws, stream)
        return self.y
