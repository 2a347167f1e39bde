"""Helpers shared by the GPU tests: upload seeded inputs, run the library through its
C ABI, bring results back as float64 numpy arrays, and measure relative errors."""
from __future__ import annotations

import numpy as np
import torch

import hybrid_attention_ssm_proj_amd as hy
from synth import BF16

DEV = "cuda:0"


def max_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def elem_err(got, ref) -> float:
    """max over elements of |got - ref| / (|ref| + rms(ref)): every element is held to its
    own magnitude, with the tensor's root-mean-square as the floor near zero (where a
    purely relative error is ill-posed)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.abs(ref) + (rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / den))


def elem_quantile(got, ref, q=0.999) -> float:
    """The q-quantile of |got - ref| / (|ref| + 1e-3 max|ref|) (reported, not gated)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref) + 1e-3 * max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.quantile(np.abs(got - ref) / den, q))


def h_err(got, ref) -> float:
    """The parity metric of the fp32 SSM state of a bf16 layer: its gate is 1e-3 of the
    tensor's largest element (max_rel_err) and 1e-2 elementwise (elem_err), returned as
    max(max_rel_err, elem_err / 10) so that one threshold of 1e-3 applies to both.  The
    elementwise bound follows from the storage: both sides hold x, delta and G in bf16,
    but the GPU's fp32-accumulated products and the oracle's fp64 products round a few
    elements of them to neighbouring bf16 values (a step of 2^-8 relative), and one such
    step in a token's x or dt moves that channel's state by up to 2^-8 of the token's
    input term."""
    return max(max_rel_err(got, ref), elem_err(got, ref) / 10.0)


def rel_err(got, ref) -> float:
    """The parity metric: the larger of the tensor-normalised error (max |got - ref| /
    max |ref|) and the elementwise error (elem_err).  A gate on it holds every element, so
    an error confined to one head, one channel block or the meta rows cannot hide under
    the tensor's largest value."""
    return max(max_rel_err(got, ref), elem_err(got, ref))


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def storage(dims):
    return torch.bfloat16 if dims.dtype == BF16 else torch.float32


def make_layer(dims, weights) -> hy.HymbaLayer:
    return hy.HymbaLayer(dims, {k: v for k, v in weights.torch.items()}, device=DEV)


def alloc_kv(dims, batch, slots, dtype=None):
    dt = dtype or storage(dims)
    Hkv, M, dh = dims.n_kv_heads, dims.n_meta, dims.head_dim
    k_meta = torch.zeros(Hkv, max(M, 1), dh, dtype=dt, device=DEV)
    v_meta = torch.zeros(Hkv, max(M, 1), dh, dtype=dt, device=DEV)
    k = torch.zeros(batch, Hkv, slots, dh, dtype=dt, device=DEV)
    v = torch.zeros(batch, Hkv, slots, dh, dtype=dt, device=DEV)
    return {"k_meta": k_meta, "v_meta": v_meta, "k": k, "v": v}


def kv_struct(kv) -> hy.KV:
    return hy.make_kv(kv["k_meta"], kv["v_meta"], kv["k"], kv["v"])


def alloc_state(dims, batch):
    h = torch.zeros(batch, dims.d_inner, dims.d_state, dtype=torch.float32, device=DEV)
    pos = torch.zeros(batch, dtype=torch.int32, device=DEV)
    return {"h": h, "pos": pos}


def state_struct(st) -> hy.SSMState:
    return hy.make_state(st["h"], st["pos"])
