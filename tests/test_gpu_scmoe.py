"""Dense SwiGLU branch of a shortcut-connected block, through the library's
one-expert FFN call, and its overlap with the MoE layer on two streams.

Oracle: the textbook dense SwiGLU FFN (oracle swiglu_ffn over all tokens).
Overlap: running the MoE layer and the dense branch concurrently on two
streams must give bitwise the outputs of running them one after the other
(the kernels are deterministic and share no buffers)."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_moe_layer_03_amd import binding as B
from sparse_moe_layer_03_amd import scmoe
from sparse_moe_layer_03_amd import synth as S
from tests.parity_util import Model, row_rel_l2, run_gpu, say, tolerances

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,dff,dtype", [
    (64, 128, 256, "f32"),
    (300, 512, 768, "bf16"),     # 16-row tiles, ragged last tile
    (8192, 512, 1024, "bf16"),   # 256x256 direct-to-LDS tiles (many rows, one expert)
])
def test_dense_branch_matches_oracle(T, d, dff, dtype):
    w = S.Workload("dense", T=T, d_model=d, n_ffn=1, n_zero=0, d_ff=dff, top_k=1, dtype=dtype,
                   seed=5)
    say(f"dense branch T={T} d={d} d_ff={dff} {dtype}")
    x = S.make_x(w, 0, "cuda")
    w1, w3, w2 = S.make_dense(w, dff, "cuda")
    br = scmoe.DenseBranch(T, d, dff, dtype)
    y = br.run(x, w1, w3, w2)
    torch.cuda.synchronize()
    ref = O.swiglu_ffn(S.to_numpy64(x), S.to_numpy64(w1), S.to_numpy64(w3), S.to_numpy64(w2))
    err = row_rel_l2(S.to_numpy64(y), ref)
    say(f"  max row rel L2 {err.max():.3e}")
    assert err.max() <= tolerances(dtype)["y"]


def test_dense_branch_decode_shape_sampled_rows():
    # T = 128 tokens of width 6144 through a 12,288-wide dense FFN
    w = S.Workload("dense_decode", T=128, d_model=6144, n_ffn=1, n_zero=0, d_ff=12288, top_k=1,
                   dtype="bf16", seed=5)
    say("dense branch decode shape")
    x = S.make_x(w, 0, "cuda")
    w1, w3, w2 = S.make_dense(w, w.d_ff, "cuda")
    br = scmoe.DenseBranch(w.T, w.d_model, w.d_ff, "bf16")
    y = br.run(x, w1, w3, w2)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(w.T, 16, replace=False)
    ref = O.swiglu_ffn(S.to_numpy64(x[rows]), S.to_numpy64(w1), S.to_numpy64(w3),
                       S.to_numpy64(w2))
    err = row_rel_l2(S.to_numpy64(y[rows]), ref)
    say(f"  max row rel L2 {err.max():.3e}")
    assert err.max() <= tolerances("bf16")["y"]


def test_moe_and_dense_on_two_streams_match_serial():
    w = S.Workload("scmoe", T=512, d_model=512, n_ffn=16, n_zero=8, d_ff=256, top_k=4,
                   dtype="bf16", bias_var=0.01, seed=7)
    say("MoE layer || dense branch on two streams")
    m = Model(w)
    x = S.make_x(w, 0, "cuda")
    w1, w3, w2 = S.make_dense(w, 1536, "cuda")
    br = scmoe.DenseBranch(w.T, w.d_model, 1536, "bf16")

    buf = B.LayerBuffers(m.shape, "cuda")
    run_gpu(m, x, buf, with_logits=False)
    y_dense = br.run(x, w1, w3, w2).clone()
    torch.cuda.synchronize()
    y_moe = buf.y.clone()

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    for rep in range(3):
        buf.y.zero_()
        br.y.zero_()
        side.wait_stream(main)
        B.layer_forward(buf, x, m.wr, m.bias, m.wg, m.wu, m.wd)  # main stream, no sync
        with torch.cuda.stream(side):
            br.run(x, w1, w3, w2, stream=side)
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(buf.y, y_moe), rep
        assert torch.equal(br.y, y_dense), rep


@pytest.mark.parametrize("dense_cus,pattern", [(32, "contiguous"), (64, "contiguous")])
def test_moe_and_dense_on_cu_partitioned_streams_match_serial(dense_cus, pattern):
    # the MoE layer and the dense branch each on its own CU-masked stream
    # (disjoint CU sets, default priority): outputs equal the serial run bit
    # for bit, with persistent grids sized to each stream's share
    w = S.Workload("scmoe_cu", T=2048, d_model=512, n_ffn=16, n_zero=8, d_ff=384, top_k=4,
                   dtype="bf16", bias_var=0.01, seed=8)
    say(f"MoE layer || dense branch on CU-partitioned streams ({dense_cus} CUs, {pattern})")
    m = Model(w)
    x = S.make_x(w, 0, "cuda")
    w1, w3, w2 = S.make_dense(w, 1536, "cuda")
    br = scmoe.DenseBranch(w.T, w.d_model, 1536, "bf16")
    buf = B.LayerBuffers(m.shape, "cuda")
    run_gpu(m, x, buf, with_logits=False)
    y_dense = br.run(x, w1, w3, w2).clone()
    torch.cuda.synchronize()
    y_moe = buf.y.clone()

    n = B.moe_device_cu_count()
    d_words = scmoe.cu_mask(n, 0, dense_cus, pattern)
    m_words = [(~v) & 0xFFFFFFFF for v in d_words]
    if n % 32:
        m_words[-1] &= (1 << (n % 32)) - 1
    ms, ds = scmoe.MaskedStream(m_words), scmoe.MaskedStream(d_words)
    try:
        assert ms.cus == n - dense_cus and ds.cus == dense_cus
        main = torch.cuda.current_stream()
        for rep in range(3):
            buf.y.zero_()
            br.y.zero_()
            ms.stream.wait_stream(main)
            ds.stream.wait_stream(main)
            with torch.cuda.stream(ms.stream):
                B.layer_forward(buf, x, m.wr, m.bias, m.wg, m.wu, m.wd, stream=ms.stream)
            with torch.cuda.stream(ds.stream):
                br.run(x, w1, w3, w2, stream=ds.stream)
            main.wait_stream(ms.stream)
            main.wait_stream(ds.stream)
            torch.cuda.synchronize()
            assert torch.equal(buf.y, y_moe), rep
            assert torch.equal(br.y, y_dense), rep
    finally:
        ms.close()
        ds.close()


@pytest.mark.parametrize("cus,T,N", [(64, 3480, 48), (32, 3480, 48), (32, 14500, 200)])
def test_many_row_gemms_on_a_cu_masked_stream_match_the_full_chip(cus, T, N):
    # The whole layer on a stream restricted to `cus` contiguous CUs: the
    # persistent expert GEMMs (256x256 and 320x192 tiles; most experts hold
    # 257..320 rows) size their grids by the stream's CU mask, so the tiles
    # land on other workgroups and the last round is cut differently, and
    # the outputs still equal the full-chip run bit for bit.  With 200
    # experts on 32 CUs the worst-case tile count needs two waves of
    # workgroups (the plan's grid multiple), the full chip one.
    w = S.Workload("rows320", T=T, d_model=512, n_ffn=N, n_zero=0, d_ff=4096, top_k=4,
                   dtype="bf16", bias_var=0.0, seed=27)
    cdiv = lambda a, b: -(-a // b)  # noqa: E731
    Tk = T * w.top_k
    tiles_max = (N + (Tk - N) // 256) * max(cdiv(w.d_ff, 128), cdiv(w.d_model, 256))
    waves = 1 if cdiv(tiles_max, cus) <= 256 else 2
    assert cdiv(tiles_max, cus * waves) <= 256
    assert waves == (2 if N == 200 else 1)
    say(f"layer on a {cus}-CU stream ({waves} wave(s) of workgroups) vs the full chip")
    m = Model(w)
    x = S.make_x(w, 0, "cuda")
    buf = B.LayerBuffers(m.shape, "cuda")
    gpu, _ = run_gpu(m, x, buf, with_logits=False)
    c = gpu["counts"][:w.n_ffn]
    assert ((c >= 257) & (c <= 320)).sum() * -(-w.d_ff // 96) >= 4 * cus
    y_full = buf.y.clone()
    n = B.moe_device_cu_count()
    ms = scmoe.MaskedStream(scmoe.cu_mask(n, 0, cus, "contiguous"))
    try:
        assert ms.cus == cus
        main = torch.cuda.current_stream()
        for rep in range(2):
            buf.y.zero_()
            ms.stream.wait_stream(main)
            with torch.cuda.stream(ms.stream):
                B.layer_forward(buf, x, m.wr, m.bias, m.wg, m.wu, m.wd, stream=ms.stream)
            main.wait_stream(ms.stream)
            torch.cuda.synchronize()
            assert torch.equal(buf.y, y_full), rep
    finally:
        ms.close()
