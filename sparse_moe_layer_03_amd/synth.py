"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the HIP path and the CPU oracle are fed from here.

Every tensor comes from its own torch generator seeded by (seed, tag, index),
so a tensor can be regenerated on its own and large expert weights can be
drawn directly in device memory, one expert at a time.  Values are drawn in
float32 and rounded to the workload dtype (bf16: round-to-nearest-even).

Recipe (value distributions follow each workload's statement):
  x         ~ N(0, 1)                    tag 1, index = batch
  W_router  ~ N(0, 1/d_model)            tag 2
  bias      ~ N(0, bias_var) or 0        tag 3 (float32, never rounded)
  W_gate    ~ N(0, 1/d_model)            tag 4, index = expert
  W_up      ~ N(0, 1/d_model)            tag 5, index = expert
  W_down    ~ N(0, 1/d_ff)               tag 6, index = expert
  Zipf rank permutation of FFN experts   tag 7
  dense branch W1, W3 ~ N(0, 1/d_model)  tags 8, 9 (shortcut-connected block)
  dense branch W2     ~ N(0, 1/d_ff)     tag 10
N(m, v) names mean and variance.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

TAG_X, TAG_WR, TAG_BIAS, TAG_WG, TAG_WU, TAG_WD, TAG_ZIPF = 1, 2, 3, 4, 5, 6, 7
TAG_D1, TAG_D3, TAG_D2 = 8, 9, 10


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    n_ffn: int
    n_zero: int
    d_ff: int
    top_k: int
    dtype: str                  # "f32" or "bf16"
    bias_var: float = 0.0       # router correction bias ~ N(0, bias_var)
    routed_scaling: float = 1.0
    pid: Optional[tuple] = None  # (setpoint, kp, ki, kd)
    batches: int = 1
    zipf_s: float = 0.0         # >0: per-FFN-expert Zipf logit offset
    seed: int = 0

    @property
    def E(self) -> int:
        return self.n_ffn + self.n_zero

    def expert_weight_bytes(self) -> int:
        el = 2 if self.dtype == "bf16" else 4
        return 3 * self.n_ffn * self.d_model * self.d_ff * el


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", T=64, d_model=128, n_ffn=8, n_zero=4, d_ff=256,
                 top_k=2, dtype="f32"),
        Workload("small_bf16", T=4096, d_model=2048, n_ffn=64, n_zero=32,
                 d_ff=1024, top_k=8, dtype="bf16", bias_var=0.1,
                 pid=(6.0, 0.01, 0.001, 0.0), batches=20),
        Workload("decode_bf16", T=128, d_model=6144, n_ffn=512, n_zero=256,
                 d_ff=2048, top_k=12, dtype="bf16"),
        Workload("prefill_bf16", T=16384, d_model=6144, n_ffn=512, n_zero=256,
                 d_ff=2048, top_k=12, dtype="bf16"),
        Workload("skewed_bf16", T=8192, d_model=4096, n_ffn=256, n_zero=128,
                 d_ff=1536, top_k=8, dtype="bf16",
                 pid=(5.0, 0.01, 0.001, 0.0), batches=100, zipf_s=1.2),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, seed: int, tag: int, index: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    # distinct 63-bit seed per (seed, tag, index)
    g.manual_seed(((seed * 1_000_003 + tag) * 1_000_033 + index) & ((1 << 63) - 1))
    return g


def normal(shape, std: float, dtype: torch.dtype, device, seed: int, tag: int,
           index: int = 0) -> torch.Tensor:
    """float32 draw of N(0, std^2), rounded once to ``dtype``."""
    g = _gen(device, seed, tag, index)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_x(w: Workload, batch: int = 0, device="cpu", T: Optional[int] = None):
    return normal((T or w.T, w.d_model), 1.0, torch_dtype(w.dtype), device,
                  w.seed, TAG_X, batch)


def make_router(w: Workload, device="cpu"):
    return normal((w.E, w.d_model), 1.0 / math.sqrt(w.d_model),
                  torch_dtype(w.dtype), device, w.seed, TAG_WR)


def make_bias(w: Workload, device="cpu"):
    if w.bias_var <= 0.0:
        return torch.zeros(w.E, dtype=torch.float32, device=device)
    return normal((w.E,), math.sqrt(w.bias_var), torch.float32, device,
                  w.seed, TAG_BIAS)


def make_experts(w: Workload, device="cpu", experts=None):
    """W_gate, W_up [N, d_ff, d] and W_down [N, d, d_ff].

    With ``experts`` (a list of expert ids) only those experts are drawn, in
    that order; each expert's values do not depend on which others are drawn.
    """
    dt = torch_dtype(w.dtype)
    ids = list(range(w.n_ffn)) if experts is None else list(experts)
    n = len(ids)
    wg = torch.empty((n, w.d_ff, w.d_model), dtype=dt, device=device)
    wu = torch.empty((n, w.d_ff, w.d_model), dtype=dt, device=device)
    wd = torch.empty((n, w.d_model, w.d_ff), dtype=dt, device=device)
    s_in = 1.0 / math.sqrt(w.d_model)
    s_ff = 1.0 / math.sqrt(w.d_ff)
    for i, e in enumerate(ids):
        wg[i] = normal((w.d_ff, w.d_model), s_in, dt, device, w.seed, TAG_WG, e)
        wu[i] = normal((w.d_ff, w.d_model), s_in, dt, device, w.seed, TAG_WU, e)
        wd[i] = normal((w.d_model, w.d_ff), s_ff, dt, device, w.seed, TAG_WD, e)
    return wg, wu, wd


def make_dense(w: Workload, d_ff: int, device="cpu"):
    """Dense SwiGLU branch weights W1, W3 [d_ff, d] and W2 [d, d_ff] of a
    shortcut-connected block (the dense FFN beside the MoE layer)."""
    dt = torch_dtype(w.dtype)
    s_in, s_ff = 1.0 / math.sqrt(w.d_model), 1.0 / math.sqrt(d_ff)
    w1 = normal((d_ff, w.d_model), s_in, dt, device, w.seed, TAG_D1, 0)
    w3 = normal((d_ff, w.d_model), s_in, dt, device, w.seed, TAG_D3, 0)
    w2 = normal((w.d_model, d_ff), s_ff, dt, device, w.seed, TAG_D2, 0)
    return w1, w3, w2


def zipf_logit_offset(w: Workload, alpha: float, device="cpu"):
    """Per-expert classifier offset that makes a few FFN experts hot.

    FFN expert e gets alpha * ln(N * q_{r(e)}) with q the Zipf(s) pmf over
    ranks 1..N and r a seeded random permutation of the ranks; zero experts
    get 0.  ``alpha`` is a stored calibration constant (see the oracle-side
    calibration script in tests/golden).
    """
    off = torch.zeros(w.E, dtype=torch.float64)
    if w.zipf_s <= 0.0:
        return off.to(torch.float32).to(device)
    g = _gen("cpu", w.seed, TAG_ZIPF)
    ranks = torch.randperm(w.n_ffn, generator=g).to(torch.float64) + 1.0
    q = ranks.pow(-w.zipf_s)
    hn = torch.arange(1, w.n_ffn + 1, dtype=torch.float64).pow(-w.zipf_s).sum()
    q = q / hn
    off[: w.n_ffn] = alpha * torch.log(w.n_ffn * q)
    return off.to(torch.float32).to(device)


def to_numpy64(t: torch.Tensor):
    """Exact float64 copy of a (possibly bf16, possibly device) tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()
