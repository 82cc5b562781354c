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
as the gathered rows.  This module only sets up those arguments.
"""

from __future__ import annotations

import torch

from . import binding as B


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
