"""GPU parity of layers with the Mamba-2 SSM head (ssm_heads > 0; the chunked
matrix-form scan on MFMA and its decode step), through the C ABI, against the CPU
oracle on the same seeded inputs.

Tolerances as for the Mamba-head layer: bf16 outputs 2e-2 and the fp32 state 1e-3,
relative to the tensor's max magnitude, against the oracle in bf16 storage-contract mode
(it rounds to bf16 where the GPU stores bf16).  The scan multiplies bf16 operands (B, C,
the chunk's decay-weighted C.B products and the previous state for the outputs) with
fp32 accumulation; the carried state takes x (exact in bf16) against w B split into two
bf16 parts, so it keeps about 16 bits per product.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from synth import gen_activations, gen_layer_weights
from tests.gpu_util import (DEV, alloc_kv, alloc_state, h_err, kv_struct, make_layer, rel_err,
                            state_struct, to_np)
from tests.test_gpu_parity import TOL_BF16, TOL_H, check_prefill, gpu_prefill, small_dims

pytestmark = pytest.mark.gpu


def dims2(**kw):
    base = dict(d_inner=512, ssm_heads=8, dt_rank=0)  # 8 heads of 64 channels
    base.update(kw)
    return small_dims(**base)


@pytest.mark.parametrize("d_state,window,M,L,B", [
    (16, 0, 16, 150, 2),    # 166 tokens: two whole chunks and a ragged one
    (16, 48, 16, 64, 3),    # window; 80 tokens
    (32, 0, 5, 59, 1),      # 64 tokens exactly, odd meta count
    (64, 0, 16, 100, 2),
    (128, 32, 8, 70, 2),
    (16, 0, 0, 130, 2),     # no meta tokens
])
def test_head_ssm_prefill_matches_oracle(d_state, window, M, L, B):
    dims = dims2(d_state=d_state, window=window, n_meta=M)
    case = 300 + d_state + window + M
    w = gen_layer_weights(dims, case)
    meta_t, meta, x_t, x = gen_activations(dims, case, B, L)
    ref = orc.prefill(dims, w, meta, x, contract=True, ring_slots=L)
    got = gpu_prefill(dims, w, meta_t, x_t, ring_slots=L)
    check_prefill(dims, got, ref, TOL_BF16, TOL_H, ring=True)


def test_head_ssm_decode_continues_prefill():
    dims = dims2(window=32)
    B, L, S, steps = 2, 70, 32, 8
    w = gen_layer_weights(dims, 311)
    meta_t, meta, x_t, x = gen_activations(dims, 311, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    got = gpu_prefill(dims, w, meta_t, x_t[:, :L].contiguous(), ring_slots=S)
    check_prefill(dims, got, ref, TOL_BF16, TOL_H, ring=True)
    layer = got["layer"]
    kv, st = got["kv_t"], got["state_t"]
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s in range(steps):
        y = layer.decode(xb[:, L + s].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"], o["v"],
                            o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        e = rel_err(to_np(y), o["y"])
        assert e < TOL_BF16, (s, e)
    assert h_err(to_np(st["h"]), o["h"]) < TOL_H
    assert np.all(st["pos"].cpu().numpy() == L + steps)


def test_head_ssm_decode_large_batch_split_k():
    """A batch and widths that take the split-K decode projections (every K a multiple
    of 256) and a state of 64 per channel."""
    dims = dims2(d_model=512, d_inner=1024, ssm_heads=16, d_state=64, window=0)
    B, L, steps = 16, 20, 3
    w = gen_layer_weights(dims, 312)
    meta_t, meta, x_t, x = gen_activations(dims, 312, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=L + steps)
    got = gpu_prefill(dims, w, meta_t, x_t[:, :L].contiguous(), ring_slots=L + steps)
    check_prefill(dims, got, ref, TOL_BF16, TOL_H, ring=True)
    layer, kv, st = got["layer"], got["kv_t"], got["state_t"]
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s in range(steps):
        y = layer.decode(xb[:, L + s].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"], o["v"],
                            o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        assert rel_err(to_np(y), o["y"]) < TOL_BF16
    assert h_err(to_np(st["h"]), o["h"]) < TOL_H


def test_head_ssm_cached_prefill_matches_plain_and_oracle():
    """The meta-prefix cache holds the post-meta state; the cached scan starts from it.
    Its chunks then start at the first X token instead of at the first meta token, so
    the bf16 operands it rounds (the previous state, the chunk products) differ from the
    plain call's: the two agree to fp32 rounding in the state and to bf16 rounding in y,
    and each is held to the oracle."""
    dims = dims2(window=0)
    B, L = 2, 90
    w = gen_layer_weights(dims, 313)
    meta_t, meta, x_t, x = gen_activations(dims, 313, B, L)
    ref = orc.prefill(dims, w, meta, x, contract=True)
    layer = make_layer(dims, w)
    meta_d, x_d = meta_t.to(DEV), x_t.to(DEV)
    st_a, st_b = alloc_state(dims, B), alloc_state(dims, B)
    ya, yma = layer.prefill(meta_d, x_d, state_out=state_struct(st_a))
    cache_t, cache = layer.build_meta_cache(meta_d)
    yb = layer.prefill_cached(cache, x_d, state_out=state_struct(st_b))
    torch.cuda.synchronize()
    errs = {"y": rel_err(to_np(yb), to_np(ya)), "h": rel_err(to_np(st_b["h"]), to_np(st_a["h"])),
            "y_meta": rel_err(to_np(cache_t["y_meta"]), to_np(yma)),
            "y vs oracle": rel_err(to_np(yb), ref["y"]),
            "h vs oracle": h_err(to_np(st_b["h"]), ref["h"])}
    print({k: f"{v:.1e}" for k, v in errs.items()})
    assert errs["h"] <= 1e-4 and errs["y_meta"] <= 1e-6 and errs["y"] < TOL_BF16
    assert errs["y vs oracle"] < TOL_BF16 and errs["h vs oracle"] < TOL_H


def test_head_ssm_full_size_sampled_sequence():
    """The prefill workload's layer shape with the Mamba-2 head (d 2048, Di 4096 in 64
    heads of 64 channels, N 16), B=8, L=2048, 128 meta tokens, run on the whole batch;
    sequence 5 is recomputed by the oracle (y, y_meta and the final state)."""
    from synth import CASES
    case = CASES[1]
    dims = case.dims.replace(ssm_heads=64, dt_rank=0)
    B, L = case.batch, case.seq_len
    w = gen_layer_weights(dims, case.case_id)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, B, L)
    layer = make_layer(dims, w)
    st = alloc_state(dims, B)
    y, ym = layer.prefill(meta_t.to(DEV), x_t.to(DEV), state_out=state_struct(st))
    torch.cuda.synchronize()
    b = 5
    ref = orc.prefill(dims, w, meta, x[b:b + 1], contract=True)
    errs = {"y": rel_err(to_np(y[b]), ref["y"][0]), "y_meta": rel_err(to_np(ym), ref["y_meta"][0]),
            "h": h_err(to_np(st["h"][b]), ref["h"][0])}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] < TOL_BF16 and errs["y_meta"] < TOL_BF16 and errs["h"] < TOL_H
    assert np.all(st["pos"].cpu().numpy() == L)
