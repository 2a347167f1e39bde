"""GPU checks of the meta-prefix cache (hymba_layer_meta_cache_build +
hymba_layer_prefill_cached), through the C ABI.

The cached prefill runs the same kernels on the same values as the plain prefill (the
meta K/V and the post-meta SSM state are what the plain call computes on the way), so
its outputs must equal the plain call's: y, the final state, the ring K/V, and the
cache's meta K/V and y_meta against the plain call's kv_out / y_meta.  The plain call is
itself held to the oracle by the parity tests; here y is also checked against the
oracle once, at the bf16 gate.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from synth import CASES, gen_activations, gen_layer_weights
from tests.gpu_util import (DEV, alloc_kv, alloc_state, kv_struct, make_layer, rel_err,
                            state_struct, to_np)
from tests.test_gpu_parity import TOL_BF16, small_dims

pytestmark = pytest.mark.gpu

SAME = 1e-6  # relative; the two paths perform identical arithmetic


def _both(dims, case, B, L, ring, kv_in=None):
    """Plain prefill and cached prefill of the same inputs; returns both result dicts."""
    w = gen_layer_weights(dims, case)
    meta_t, meta, x_t, x = gen_activations(dims, case, B, L)
    layer = make_layer(dims, w)
    meta_d, x_d = meta_t.to(DEV), x_t.to(DEV)
    out = {}
    for mode in ("plain", "cached"):
        kv = alloc_kv(dims, B, ring) if (ring and not dims.kv_share) else None
        st = alloc_state(dims, B)
        kin = kv_struct(kv_in) if kv_in is not None else None
        if mode == "plain":
            y, ym = layer.prefill(meta_d, x_d, kv_in=kin, kv_out=kv_struct(kv) if kv else None,
                                  state_out=state_struct(st))
            cache_t = None
        else:
            cache_t, cache = layer.build_meta_cache(meta_d, kv_in=kin)
            y = layer.prefill_cached(cache, x_d, kv_in=kin, kv_out=kv_struct(kv) if kv else None,
                                     state_out=state_struct(st))
            ym = cache_t["y_meta"]
        torch.cuda.synchronize()
        out[mode] = dict(y=to_np(y), y_meta=to_np(ym), h=to_np(st["h"]),
                         pos=st["pos"].cpu().numpy(), kv=kv, cache=cache_t, y_t=y, ym_t=ym)
    return w, meta, x, out


def _assert_same(a, b, M, ring):
    errs = {k: rel_err(b[k], a[k]) for k in ("y", "h")}
    if M:
        errs["y_meta"] = rel_err(b["y_meta"][:M], a["y_meta"][:M])
    if ring:
        for k in ("k", "v"):
            errs[k] = rel_err(to_np(b["kv"][k]), to_np(a["kv"][k]))
        if M and b["cache"] is not None and "k_meta" in b["cache"]:
            for k in ("k_meta", "v_meta"):
                errs[k] = rel_err(to_np(b["cache"][k])[:, :M], to_np(a["kv"][k])[:, :M])
    print({k: f"{v:.1e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= SAME, (k, v)
    assert np.all(b["pos"] == a["pos"])


@pytest.mark.parametrize("window,L", [(0, 160), (48, 130)])
def test_cached_prefill_equals_plain_bf16(window, L):
    dims = small_dims(window=window)
    B = 2
    w, meta, x, out = _both(dims, 91 + window, B, L, ring=L)
    _assert_same(out["plain"], out["cached"], dims.n_meta, ring=True)
    ref = orc.prefill(dims, w, meta, x, contract=True)
    e = rel_err(out["cached"]["y"], ref["y"])
    print(f"cached y vs oracle {e:.2e}")
    assert e < TOL_BF16


def test_cached_prefill_equals_plain_fp32():
    dims = CASES[0].dims
    B, L = 1, 64
    _, _, _, out = _both(dims, 92, B, L, ring=L)
    _assert_same(out["plain"], out["cached"], dims.n_meta, ring=True)


def test_cached_prefill_consumer_layer():
    """A kv_share consumer: its meta keys are the producer's, its cache holds h and
    y_meta only."""
    p_dims = small_dims(window=40)
    c_dims = p_dims.replace(kv_share=1)
    B, L = 2, 96
    w1 = gen_layer_weights(p_dims, 93)
    meta_t, _, x_t, _ = gen_activations(p_dims, 93, B, L)
    prod = make_layer(p_dims, w1)
    kv = alloc_kv(p_dims, B, L)
    st = alloc_state(p_dims, B)
    y1, ym1 = prod.prefill(meta_t.to(DEV), x_t.to(DEV), kv_out=kv_struct(kv),
                           state_out=state_struct(st))
    torch.cuda.synchronize()
    w2 = gen_layer_weights(c_dims, 93, layer=1)
    cons = make_layer(c_dims, w2)
    st_a, st_b = alloc_state(c_dims, B), alloc_state(c_dims, B)
    ya, yma = cons.prefill(ym1, y1, kv_in=kv_struct(kv), state_out=state_struct(st_a))
    cache_t, cache = cons.build_meta_cache(ym1, kv_in=kv_struct(kv))
    yb = cons.prefill_cached(cache, y1, kv_in=kv_struct(kv), state_out=state_struct(st_b))
    torch.cuda.synchronize()
    errs = {"y": rel_err(to_np(yb), to_np(ya)), "h": rel_err(to_np(st_b["h"]), to_np(st_a["h"])),
            "y_meta": rel_err(to_np(cache_t["y_meta"]), to_np(yma))}
    print({k: f"{v:.1e}" for k, v in errs.items()})
    assert max(errs.values()) <= SAME


def test_decode_after_cached_prefill_reads_the_cache_meta_kv():
    """Decode after the cached prefill, with kv.k_meta / v_meta pointing at the cache,
    equals decode after the plain prefill."""
    dims = small_dims(window=32)
    B, L, S, steps = 2, 70, 32, 6
    w, meta, x, out = _both(dims, 94, B, L, ring=S)
    layer = make_layer(dims, w)
    _, _, x_t, _ = gen_activations(dims, 94, B, L + steps)
    xb = x_t.to(DEV)
    a, b = out["plain"], out["cached"]
    st_a = {"h": torch.from_numpy(a["h"].astype(np.float32)).to(DEV),
            "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    st_b = {"h": torch.from_numpy(b["h"].astype(np.float32)).to(DEV),
            "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    kv_b = dict(b["kv"])
    kv_b["k_meta"], kv_b["v_meta"] = b["cache"]["k_meta"], b["cache"]["v_meta"]
    for s in range(steps):
        ya = layer.decode(xb[:, L + s].contiguous(), kv_struct(a["kv"]), state_struct(st_a))
        yb = layer.decode(xb[:, L + s].contiguous(), kv_struct(kv_b), state_struct(st_b))
        torch.cuda.synchronize()
        e = rel_err(to_np(yb), to_np(ya))
        assert e <= SAME, (s, e)
