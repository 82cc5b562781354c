"""GPU parity of the whole layer (route, dispatch, expert FFN, combine)
against the oracle, through the C ABI, on the workload shapes and on
ragged multi-tile shapes."""

import numpy as np
import pytest
import torch

from sparse_moe_layer_03_amd import synth as S
from tests.parity_util import (Model, check_dispatch, check_gates, check_routing,
                               covering_tokens, full_oracle, full_parity,
                               oracle_outputs_for_tokens, oracle_route, row_rel_l2, run_gpu, say,
                               tolerances, zipf_alpha)

pytestmark = pytest.mark.gpu


def test_tiny_f32_workload():
    full_parity(S.WORKLOADS["tiny_f32"])


def test_tiny_f32_with_materialised_x_perm():
    full_parity(S.WORKLOADS["tiny_f32"], x_perm=True)


def test_small_bf16_workload_batch0():
    full_parity(S.WORKLOADS["small_bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    # T, d, N, Z, d_ff, k   -- several tiles with ragged tails in M and N
    (1600, 192, 32, 8, 320, 4),    # 128x128 tiles (>= 32 rows per expert, >= 64 tiles)
    (77, 256, 40, 24, 192, 6),     # 16-row tiles
    (1, 64, 3, 1, 64, 2),          # single token
    (2048, 512, 16, 8, 384, 4),    # bf16: 256x256 direct-to-LDS tiles, 2 m-tiles/expert,
                                   # K-steps 8 (gate/up) and 6 (down)
    (777, 1024, 24, 16, 256, 5),   # bf16: router + top-k in one kernel (40 experts: a
                                   # partial 16-expert block; a partial 16-token block)
])
def test_ragged_shapes(dtype, shape):
    T, d, N, Z, dff, k = shape
    w = S.Workload(f"ragged_{dtype}", T=T, d_model=d, n_ffn=N, n_zero=Z, d_ff=dff, top_k=k,
                   dtype=dtype, bias_var=0.01, seed=3)
    full_parity(w)
    full_parity(w, x_perm=True)


def test_routed_scaling_applies_to_every_gate():
    w = S.Workload("scaled", T=96, d_model=128, n_ffn=6, n_zero=6, d_ff=128, top_k=3,
                   dtype="f32", routed_scaling=9.0, seed=5)
    full_parity(w)


def check_sampled_outputs(m, x, gpu, toks, tol, label):
    """Oracle outputs of the sampled tokens (their experts streamed to the
    host one at a time) against the GPU's rows."""
    y_ref = oracle_outputs_for_tokens(m, x, toks, gpu["topk_idx"])
    err = row_rel_l2(gpu["y"][toks], y_ref)
    say(f"  {label}: {toks.size} tokens checked, y_row_relL2_max={err.max():.3e} "
        f"mean={err.mean():.3e}")
    assert err.max() <= tol["y"]


@pytest.mark.parametrize("n_min", [1024])
def test_skewed_bf16_workload_batch0_sampled(n_min):
    w = S.WORKLOADS["skewed_bf16"]
    say(f"[parity] {w}")
    m = Model(w, "cuda", zipf_alpha())
    x = S.make_x(w, 0, "cuda")
    gpu, _ = run_gpu(m, x)
    tol = tolerances(w.dtype)
    ref = oracle_route(m, x)
    check_routing(gpu, ref, w.top_k, tol["logits"])
    check_gates(gpu, ref, w.routed_scaling, tol["gate_rtol"])
    check_dispatch(gpu, w.E)
    r = (gpu["topk_idx"] < w.n_ffn).sum() / w.T
    assert abs(r - 7.5) < 0.1
    toks, tiles, _ = covering_tokens(gpu, w.n_ffn, w.top_k, n_min, seed=7)
    say(f"  {len(tiles)} m-tiles, every one hit by a sampled token")
    check_sampled_outputs(m, x, gpu, toks, tol, "skewed batch 0")


@pytest.fixture(scope="module")
def big_model():
    w = S.WORKLOADS["decode_bf16"]
    say("[fixture] generating 512-expert d_model=6144 weights on the GPU")
    m = Model(w, "cuda")
    yield m
    del m
    torch.cuda.empty_cache()


def _run_big(m, w):
    from sparse_moe_layer_03_amd import binding as B
    m.w = w
    m.shape = B.make_shape(w.T, w.d_model, w.n_ffn, w.n_zero, w.d_ff, w.top_k, w.dtype,
                           w.routed_scaling)
    x = S.make_x(w, 0, "cuda")
    gpu, buf = run_gpu(m, x)
    del buf
    tol = tolerances(w.dtype)
    ref = oracle_route(m, x)
    rep = {}
    check_routing(gpu, ref, w.top_k, tol["logits"], rep)
    check_gates(gpu, ref, w.routed_scaling, tol["gate_rtol"])
    check_dispatch(gpu, w.E)
    say(f"  routing of all {w.T} tokens: uncertified={rep['uncertified']}, dispatch bit-exact")
    return x, gpu, tol


@pytest.mark.parametrize("n_min", [128])
def test_decode_full_size_every_token(big_model, n_min):
    w = S.WORKLOADS["decode_bf16"]
    say(f"[parity] {w}")
    x, gpu, tol = _run_big(big_model, w)
    check_sampled_outputs(big_model, x, gpu, np.arange(w.T), tol, "decode, all tokens")


@pytest.mark.parametrize("n_min", [1024])
def test_prefill_full_size_every_mtile(big_model, n_min):
    w = S.WORKLOADS["prefill_bf16"]
    say(f"[parity] {w}")
    x, gpu, tol = _run_big(big_model, w)
    toks, tiles, _ = covering_tokens(gpu, w.n_ffn, w.top_k, n_min, seed=11)
    say(f"  {len(tiles)} m-tiles, every one hit by a sampled token")
    check_sampled_outputs(big_model, x, gpu, toks, tol, "prefill")


@pytest.mark.parametrize("n_min", [1024])
def test_prefill_model_twice_the_batch(big_model, n_min):
    # 32768 tokens: 393,216 assignments; x_perm-sized offsets pass 2^32 bytes
    # and a workgroup runs more than 128 tiles -- still the many-row kernel
    w = S.Workload("prefill32k_bf16", T=32768, d_model=6144, n_ffn=512, n_zero=256, d_ff=2048,
                   top_k=12, dtype="bf16")
    say(f"[parity] {w}")
    x, gpu, tol = _run_big(big_model, w)
    toks, tiles, _ = covering_tokens(gpu, w.n_ffn, w.top_k, n_min, seed=13)
    say(f"  {len(tiles)} m-tiles, every one hit by a sampled token")
    check_sampled_outputs(big_model, x, gpu, toks, tol, "prefill model, T=32768")


@pytest.mark.parametrize("n_min", [1024])
def test_prefill_model_four_times_the_batch(big_model, n_min):
    # 65536 tokens: 786,432 assignments, about 1024 rows per expert.  For the
    # worst spread of rows the descriptor registers of a one-per-CU grid
    # would not hold every workgroup's tiles, so the many-row kernel runs on
    # twice the CU count of workgroups, in two waves (plan::big_grid_mult)
    w = S.Workload("prefill64k_bf16", T=65536, d_model=6144, n_ffn=512, n_zero=256, d_ff=2048,
                   top_k=12, dtype="bf16")
    say(f"[parity] {w}")
    x, gpu, tol = _run_big(big_model, w)
    toks, tiles, _ = covering_tokens(gpu, w.n_ffn, w.top_k, n_min, seed=17)
    say(f"  {len(tiles)} m-tiles, every one hit by a sampled token")
    check_sampled_outputs(big_model, x, gpu, toks, tol, "prefill model, T=65536")
