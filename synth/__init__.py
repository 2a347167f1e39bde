"""Seeded synthetic inputs for the Hymba hybrid-head layer.

This module holds shapes and random draws only: none of the layer's arithmetic.
Both the CPU oracle's tests and the GPU path's tests/bench take their inputs from
here, so that the two sides see bit-identical weights and activations.

Distributions follow the layer workloads used throughout (weights N(0, 0.02),
meta tokens and X N(0, 1), dt bias U[-4, -2], A = -exp(U[0, 2]), D N(0, 1),
beta = 1).  Streams are numpy PCG64 seeded with SeedSequence([1000 + case, role]):
role 0 = meta tokens, 1 = X, 10 + layer = that layer's weights, 100 + s = decode
step s inputs, 300 + layer = block weights, 400 + b = the prior context of decode
sequence b.

bf16 cases are drawn in fp32 and converted with torch's round-to-nearest-even
conversion; the float32 view of the bf16 values is what the oracle receives.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class LayerDims:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_inner: int
    d_state: int
    dt_rank: int
    n_meta: int
    window: int = 0          # 0 = full causal
    kv_share: int = 0        # 0 = producer (own K/V columns), 1 = consumer
    dtype: str = BF16
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0  # 0 => 1/sqrt(head_dim)
    ssm_heads: int = 0          # 0 = Mamba head (per-channel A, dt of rank dt_rank);
                                # H > 0 = Mamba-2 head: H heads, scalar A and dt per head
    norm_group: int = 0         # 0 = RMSNorm per branch; g > 0 = group norm, g channels
    scan_chunk: int = 0         # tokens per time chunk of the scan (0 = chosen per call)

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_in(self) -> int:
        kv = 0 if self.kv_share else 2 * self.kv_width
        return self.q_width + kv + 2 * self.d_inner

    @property
    def n_xproj(self) -> int:
        return (self.ssm_heads or self.dt_rank) + 2 * self.d_state

    @property
    def f_width(self) -> int:
        return self.q_width + self.d_inner

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "LayerDims":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Case:
    """A workload: layer dims, batch, token count and (for decode) steps."""
    case_id: int
    name: str
    dims: LayerDims
    batch: int
    seq_len: int
    n_layers: int = 1          # 2 => producer + KV-sharing consumer pair
    decode_steps: int = 0
    prior_tokens: int = 0      # decode: tokens already in the cache
    ring_slots: int = 0        # decode: KV ring capacity


def _dims_1(**kw) -> LayerDims:
    base = dict(d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, d_inner=4096,
                d_state=16, dt_rank=128, n_meta=128, window=0, kv_share=0, dtype=BF16)
    base.update(kw)
    return LayerDims(**base)


# The five workloads.  dt_rank = ceil(d_model / 16).
CASES: Dict[int, Case] = {
    0: Case(0, "tiny-fp32", LayerDims(d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                                      d_inner=256, d_state=16, dt_rank=8, n_meta=8,
                                      window=0, dtype=F32), batch=1, seq_len=64),
    1: Case(1, "prefill-b8-l2048-full", _dims_1(), batch=8, seq_len=2048),
    2: Case(2, "prefill-pair-b4-l8192-swa1024-kvshare", _dims_1(window=1024), batch=4,
            seq_len=8192, n_layers=2),
    3: Case(3, "prefill-b1-l32768-swa1024-n128", _dims_1(window=1024, d_state=128), batch=1,
            seq_len=32768),
    4: Case(4, "decode-b128-ring1024", _dims_1(window=1024), batch=128, seq_len=1,
            decode_steps=256, prior_tokens=4096, ring_slots=1024),
}


def rng(case_id: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + case_id, role])))


def to_storage(a: np.ndarray, dtype: str):
    """Return (torch tensor in storage dtype on CPU, float32 numpy view of its values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == BF16:
        t = t.to(torch.bfloat16)
        return t, t.float().numpy()
    return t, t.numpy().copy()


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float64) * std).astype(np.float32)


@dataclasses.dataclass
class LayerWeights:
    """Weights of one layer.  `np_*` are float32 arrays holding exactly the values
    the device sees; `t_*` are the torch CPU tensors in storage dtype (or fp32)."""
    w_in: np.ndarray      # [n_in, d]
    w_x: np.ndarray       # [R + 2N, Di]  (Mamba-2 head: [H + 2N, Di])
    w_dt: np.ndarray      # [Di, R]       (Mamba-2 head: empty, [Di, 0])
    dt_bias: np.ndarray   # [Di] fp32     (Mamba-2 head: [H])
    A: np.ndarray         # [Di, N] fp32  (Mamba-2 head: [H])
    D: np.ndarray         # [Di] fp32
    w_out: np.ndarray     # [d, Hq*dh + Di]
    beta_attn: np.ndarray  # [Hq*dh] fp32
    beta_ssm: np.ndarray   # [Di] fp32
    torch: Dict[str, object]


def gen_layer_weights(dims: LayerDims, case_id: int, layer: int = 0,
                      std: float = 0.02) -> LayerWeights:
    g = rng(case_id, 10 + layer)
    d, Di, N, R = dims.d_model, dims.d_inner, dims.d_state, dims.dt_rank
    w_in = _normal(g, (dims.n_in, d), std)
    if dims.ssm_heads:  # Mamba-2 head: one dt and one A per head, no dt projection
        H = dims.ssm_heads
        w_x = _normal(g, (H + 2 * N, Di), std)
        w_dt = np.zeros((Di, 0), np.float32)
        dt_bias = g.uniform(-4.0, -2.0, size=(H,)).astype(np.float32)
        A = (-np.exp(g.uniform(0.0, 2.0, size=(H,)))).astype(np.float32)
    else:
        w_x = _normal(g, (R + 2 * N, Di), std)
        w_dt = _normal(g, (Di, R), std)
        dt_bias = g.uniform(-4.0, -2.0, size=(Di,)).astype(np.float32)
        A = (-np.exp(g.uniform(0.0, 2.0, size=(Di, N)))).astype(np.float32)
    D = g.standard_normal(size=(Di,)).astype(np.float32)
    w_out = _normal(g, (d, dims.f_width), std)
    beta_attn = np.ones(dims.q_width, np.float32)
    beta_ssm = np.ones(Di, np.float32)
    tt = {}
    vals = {}
    for name, arr in (("w_in", w_in), ("w_x", w_x), ("w_dt", w_dt), ("w_out", w_out)):
        tt[name], vals[name] = to_storage(arr, dims.dtype)
    for name, arr in (("dt_bias", dt_bias), ("A", A), ("D", D), ("beta_attn", beta_attn),
                      ("beta_ssm", beta_ssm)):
        tt[name], vals[name] = to_storage(arr, F32)
    return LayerWeights(torch=tt, **vals)


def gen_activations(dims: LayerDims, case_id: int, batch: int, seq_len: int):
    """meta [M, d] and X [B, L, d] ~ N(0, 1).  Returns (meta_t, meta_np, x_t, x_np)."""
    meta = rng(case_id, 0).standard_normal(size=(dims.n_meta, dims.d_model), dtype=np.float32)
    x = rng(case_id, 1).standard_normal(size=(batch, seq_len, dims.d_model), dtype=np.float32)
    meta_t, meta_np = to_storage(meta, dims.dtype)
    x_t, x_np = to_storage(x, dims.dtype)
    return meta_t, meta_np, x_t, x_np


def gen_decode_inputs(dims: LayerDims, case_id: int, batch: int, step: int):
    """New-token activations for decode step `step`: [B, d] ~ N(0, 1)."""
    x = rng(case_id, 100 + step).standard_normal(size=(batch, dims.d_model), dtype=np.float32)
    return to_storage(x, dims.dtype)


def gen_prior_tokens(dims: LayerDims, case_id: int, seq: int, seq_len: int):
    """The context sequence `seq` of a decode workload saw before decoding: [L, d] ~ N(0, 1),
    one stream per sequence (role 400 + seq), so any subset of the batch can be drawn on
    its own.  Returns (torch tensor in storage dtype, float32 numpy values)."""
    x = rng(case_id, 400 + seq).standard_normal(size=(seq_len, dims.d_model), dtype=np.float32)
    return to_storage(x, dims.dtype)


@dataclasses.dataclass
class BlockWeights:
    """The block wrapper around a layer: RMSNorm weights before the layer and before the
    FFN, and the FFN's two projections (float32 values the device sees, plus torch)."""
    norm1: np.ndarray   # [d] fp32
    norm2: np.ndarray   # [d] fp32
    w_up: np.ndarray    # [I, d]
    w_down: np.ndarray  # [d, I]
    torch: Dict[str, object]


def gen_block_weights(dims: LayerDims, case_id: int, intermediate: int, layer: int = 0,
                      std: float = 0.02) -> BlockWeights:
    """Norm weights ~ 1 + N(0, 0.1); W_up, W_down ~ N(0, std).  Stream role 300 + layer."""
    g = rng(case_id, 300 + layer)
    d = dims.d_model
    n1 = (1.0 + 0.1 * g.standard_normal(size=(d,))).astype(np.float32)
    n2 = (1.0 + 0.1 * g.standard_normal(size=(d,))).astype(np.float32)
    up = _normal(g, (intermediate, d), std)
    down = _normal(g, (d, intermediate), std)
    tt, vals = {}, {}
    for name, arr in (("w_up", up), ("w_down", down)):
        tt[name], vals[name] = to_storage(arr, dims.dtype)
    for name, arr in (("norm1", n1), ("norm2", n2)):
        tt[name], vals[name] = to_storage(arr, F32)
    return BlockWeights(torch=tt, **vals)

