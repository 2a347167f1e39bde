"""Helpers shared by the GPU tests: upload seeded inputs, run the library through its
C ABI, bring results back as float64 numpy arrays, and measure relative errors."""
from __future__ import annotations

import numpy as np
import torch

import hybrid_attention_ssm_proj_amd as hy
from synth import BF16

DEV = "cuda:0"


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


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
