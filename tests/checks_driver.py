"""Runs layer cases through the library that MOE_MI355X_LIB names (the debug
build with device-side index-range checks, in a process of its own) and
prints one JSON line: the check bits after the valid cases, the bits after a
dispatch given an out-of-range expert id, and a digest of each valid case's
output, so the caller can compare it with the release build's.

    MOE_MI355X_LIB=.../libmoe_mi355x_checks.so python -m tests.checks_driver
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from sparse_moe_layer_03_amd import binding as B  # noqa: E402
from sparse_moe_layer_03_amd import synth as S  # noqa: E402
from tests.parity_util import Model, run_gpu  # noqa: E402

# whole-layer cases, one per kernel path: fused router + top-k, three-kernel
# dispatch and 256x256 expert tiles (small); a decode-shaped batch (top-k
# kernel, one-workgroup dispatch, 16-row tiles); the router's 256x256 split-K
# path; a half-empty last round cut into row slices; fp32
LAYER_CASES = [
    S.WORKLOADS["small_bf16"],
    S.Workload("decode_like", T=128, d_model=1024, n_ffn=512, n_zero=256, d_ff=512, top_k=12,
               dtype="bf16", seed=41),
    S.Workload("router_big", T=4000, d_model=1536, n_ffn=200, n_zero=100, d_ff=64, top_k=6,
               dtype="bf16", bias_var=0.01, seed=23),
    S.Workload("tail_slices", T=4096, d_model=512, n_ffn=8, n_zero=4, d_ff=256, top_k=2,
               dtype="bf16", bias_var=0.01, seed=24),
    S.WORKLOADS["tiny_f32"],
]

# expert GEMMs on hand-written top-1 routings with 35 experts of 257..320
# rows: the 320x192 launches of gate/up and of down
R320_COUNTS = [256, 257, 320, 321, 0, 1, 255] + [257 + (7 * i) % 64 for i in range(33)]
R320_CASES = [(512, 4096), (6144, 256)]


def digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]


def layer_case(w):
    m = Model(w, "cuda")
    _, buf = run_gpu(m, S.make_x(w, 0, "cuda"), with_logits=False)
    return digest(buf.y)


def r320_case(d, dff):
    counts = R320_COUNTS
    N = len(counts)
    idx = np.repeat(np.arange(N), counts).astype(np.int32)
    np.random.default_rng(31).shuffle(idx)
    T = idx.size
    w = S.Workload("rows320_exact", T=T, d_model=d, n_ffn=N, n_zero=0, d_ff=dff, top_k=1,
                   dtype="bf16", seed=28)
    m = Model(w, "cuda")
    x = S.make_x(w, 0, "cuda")
    buf = B.LayerBuffers(m.shape, "cuda")
    tidx = torch.as_tensor(idx.reshape(T, 1), device="cuda")
    B.moe_dispatch(m.shape, tidx, x, buf.counts, buf.offsets, buf.perm, buf.inv_perm, None, buf.ws)
    B.moe_expert_ffn(m.shape, x, None, buf.perm, buf.offsets, m.wg, m.wu, m.wd, buf.y_perm, buf.ws)
    torch.cuda.synchronize()
    return digest(buf.y_perm[:T])


def invalid_dispatch(T, N, k):
    # one expert id equal to E (out of range); both dispatch paths skip it
    w = S.Workload("bad_ids", T=T, d_model=64, n_ffn=N, n_zero=0, d_ff=64, top_k=k, dtype="f32",
                   seed=5)
    s = B.make_shape(w.T, w.d_model, w.n_ffn, w.n_zero, w.d_ff, w.top_k, w.dtype)
    buf = B.LayerBuffers(s, "cuda")
    idx = torch.arange(T * k, dtype=torch.int32, device="cuda").remainder(N).reshape(T, k)
    idx[T // 2, 0] = N
    x = torch.zeros((T, w.d_model), dtype=torch.float32, device="cuda")
    B.moe_dispatch(s, idx, x, buf.counts, buf.offsets, buf.perm, buf.inv_perm, None, buf.ws)
    torch.cuda.synchronize()


def main():
    assert torch.cuda.is_available()
    B.moe_debug_checks(clear=True)
    out = {"lib": os.path.basename(B.LIB_PATH), "digests": {}}
    for w in LAYER_CASES:
        out["digests"][w.name] = layer_case(w)
        print(f"[checks] {w.name}", file=sys.stderr, flush=True)
    for d, dff in R320_CASES:
        out["digests"][f"rows320_{d}_{dff}"] = r320_case(d, dff)
        print(f"[checks] rows320 {d} {dff}", file=sys.stderr, flush=True)
    out["valid_bits"] = B.moe_debug_checks(clear=True)
    out["invalid_bits"] = []
    for T, N, k in ((100, 8, 2), (3000, 8, 2)):   # one-workgroup and three-kernel dispatch
        invalid_dispatch(T, N, k)
        out["invalid_bits"].append(B.moe_debug_checks(clear=True))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
