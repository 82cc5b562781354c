"""Chained layers as one captured graph (the multi-layer decode measurement
of the weight-prefetch study): three resident layers with distinct weights,
each taking the previous one's output, captured once with the next layer's
router matrix read on a second stream during each layer's expert GEMMs.
Every replay equals the eager chain bit for bit, and the last layer's output
matches the oracle on that layer's input."""

import dataclasses

import numpy as np
import pytest
import torch

from sparse_moe_layer_03_amd import binding as B
from sparse_moe_layer_03_amd import synth as S
from tests.parity_util import (Model, full_oracle, row_rel_l2, say, tolerances)

pytestmark = pytest.mark.gpu


def test_three_chained_layers_graph_with_prefetch_matches_eager_and_oracle():
    base = S.Workload("chain", T=256, d_model=512, n_ffn=32, n_zero=16, d_ff=384, top_k=6,
                      dtype="bf16", bias_var=0.01, seed=21)
    ws = [dataclasses.replace(base, seed=base.seed + 7 * i) for i in range(3)]
    ms = [Model(w) for w in ws]
    bufs = [B.LayerBuffers(m.shape, "cuda") for m in ms]
    x0 = S.make_x(base, 0, "cuda")
    side = torch.cuda.Stream()
    sink = torch.empty_like(ms[0].wr)
    evs = [torch.cuda.Event() for _ in ms]

    def chain(prefetch):
        x = x0
        for i, (m, buf) in enumerate(zip(ms, bufs)):
            s = m.shape
            B.moe_route(s, x, m.wr, None, m.bias, buf.topk_idx, buf.topk_gate, None, buf.ws)
            B.moe_dispatch(s, buf.topk_idx, x, buf.counts, buf.offsets, buf.perm, buf.inv_perm,
                           None, buf.ws)
            cur = torch.cuda.current_stream()
            if prefetch and i + 1 < len(ms):
                evs[i].record(cur)
                side.wait_event(evs[i])
                with torch.cuda.stream(side):
                    sink.copy_(ms[i + 1].wr)
            B.moe_ffn_gate_up(s, x, None, buf.perm, buf.offsets, m.wg, m.wu, buf.ws)
            B.moe_ffn_down(s, buf.offsets, m.wd, buf.y_perm, buf.ws)
            B.moe_combine(s, x, buf.y_perm, buf.topk_idx, buf.topk_gate, buf.inv_perm, buf.y)
            if prefetch and i + 1 < len(ms):
                cur.wait_stream(side)
            x = buf.y
        return x

    y_eager = chain(False).clone()
    x_last = bufs[1].y.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    chain(True)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        chain(True)
    for rep in range(3):
        for buf in bufs:
            buf.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[-1].y, y_eager), rep
    o = full_oracle(ms[-1], x_last, gpu_idx=bufs[-1].topk_idx.cpu().numpy())
    err = row_rel_l2(S.to_numpy64(bufs[-1].y), o["y"])
    say(f"  chained graph: replays bitwise equal to eager; last layer row rel L2 {err.max():.2e}")
    assert err.max() <= tolerances("bf16")["y"]
