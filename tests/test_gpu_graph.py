"""The layer step (route, dispatch, expert FFN, combine, PID update) captured
as HIP graphs, one per batch, and replayed.  The library makes no
allocation, memset or synchronisation inside a call, so a step can be
captured whole; every replay must reproduce the eager run bit for bit
(outputs, selection, counts and the controller's bias), with eager work and
synchronisations between the replays."""

import numpy as np
import pytest
import torch

from sparse_moe_layer_03_amd import binding as B
from sparse_moe_layer_03_amd import synth as S
from tests.parity_util import Model, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,N,Z,dff,k", [
    (512, 256, 16, 8, 128, 4),      # router in the general kernel, 16-row expert tiles
    (2048, 1024, 32, 16, 256, 8),   # router fused with the top-k, 256x256 expert tiles
])
def test_graph_replays_match_eager(T, d, N, Z, dff, k):
    w = S.Workload("graph", T=T, d_model=d, n_ffn=N, n_zero=Z, d_ff=dff, top_k=k, dtype="bf16",
                   bias_var=0.1, pid=(k * 0.75, 0.01, 0.001, 0.0), batches=3, seed=31)
    say(f"[graph] {w}")
    m = Model(w, "cuda")
    xs = [S.make_x(w, b, "cuda") for b in range(w.batches)]
    buf = B.LayerBuffers(m.shape, "cuda")
    params = B.MoePidParams(*w.pid)
    bias0 = m.bias.clone()

    def step(b):
        B.layer_forward(buf, xs[b], m.wr, m.bias, m.wg, m.wu, m.wd)
        B.moe_pid_update(m.shape, params, buf.counts, buf.pid_state, m.bias)

    def reset():
        m.bias.copy_(bias0)
        buf.pid_state.zero_()
        torch.cuda.synchronize()

    names = ("y", "topk_idx", "topk_gate", "counts", "perm")
    want = []
    for b in range(w.batches):
        step(b)
        torch.cuda.synchronize()
        want.append({n: getattr(buf, n).clone() for n in names} | {"bias": m.bias.clone()})
    assert not torch.equal(want[0]["bias"], want[-1]["bias"]), "PID did not move the bias"

    reset()
    graphs = []
    cap = torch.cuda.Stream()  # default priority
    for b in range(w.batches):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(b)
        graphs.append(g)

    for rep in range(3):
        reset()
        for b, g in enumerate(graphs):
            buf.y.zero_()  # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            got = {n: getattr(buf, n) for n in names} | {"bias": m.bias}
            for n, v in want[b].items():
                assert torch.equal(got[n], v), f"replay {rep}, batch {b}: {n} differs"
    say("  3 x 3 replays bitwise equal to eager")
