"""GPU parity of the group-normalisation fusion variant (norm_group = g > 0: each branch
normalised per group of g channels about the group mean, then beta and the 0.5 average),
through the C ABI, against the oracle.  Tolerances as for the default layer: bf16
outputs 2e-2, the fp32 state 1e-3, fp32 layers 1e-4, relative to the tensor's max
magnitude, the oracle in bf16 storage-contract mode for bf16 layers."""
import numpy as np
import pytest
import torch

import oracle as orc
from synth import CASES, gen_activations, gen_layer_weights
from tests.gpu_util import DEV, h_err, kv_struct, rel_err, state_struct, to_np
from tests.test_gpu_parity import (TOL_BF16, TOL_F32, TOL_H, check_prefill, gpu_prefill,
                                   small_dims)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("g,window,ssm_heads", [(128, 0, 0), (64, 40, 0), (512, 0, 0),
                                               (64, 0, 8)])
def test_group_norm_prefill_matches_oracle(g, window, ssm_heads):
    extra = dict(ssm_heads=ssm_heads, dt_rank=0) if ssm_heads else {}
    dims = small_dims(window=window, norm_group=g, **extra)
    B, L = 2, 100
    case = 400 + g + window + ssm_heads
    w = gen_layer_weights(dims, case)
    meta_t, meta, x_t, x = gen_activations(dims, case, B, L)
    ref = orc.prefill(dims, w, meta, x, contract=True, ring_slots=L)
    got = gpu_prefill(dims, w, meta_t, x_t, ring_slots=L)
    check_prefill(dims, got, ref, TOL_BF16, TOL_H, ring=True)


def test_group_norm_fp32_prefill_matches_oracle():
    dims = CASES[0].dims.replace(norm_group=32)
    w = gen_layer_weights(dims, 401)
    meta_t, meta, x_t, x = gen_activations(dims, 401, 1, 64)
    ref = orc.prefill(dims, w, meta, x)
    got = gpu_prefill(dims, w, meta_t, x_t)
    check_prefill(dims, got, ref, TOL_F32, TOL_F32)


@pytest.mark.parametrize("B,n_kv", [(3, 2), (128, 2)])
def test_group_norm_decode_continues_prefill(B, n_kv):
    """Small batches merge key splits before the group norm; 128 sequences x 2 kv heads
    take the streaming decode attention."""
    dims = small_dims(window=32, norm_group=128, n_kv_heads=n_kv)
    L, S, steps = 40, 32, 3
    w = gen_layer_weights(dims, 402)
    meta_t, meta, x_t, x = gen_activations(dims, 402, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    got = gpu_prefill(dims, w, meta_t, x_t[:, :L].contiguous(), ring_slots=S)
    layer, kv, st = got["layer"], got["kv_t"], got["state_t"]
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


def test_group_norm_full_size_sampled_sequence():
    """The prefill workload's layer (d 2048, 16 x 128 q / 4 kv heads, Di 4096, N 16, 128
    meta tokens) with g = 128, B=8, L=2048, run on the whole batch; sequence 3 is
    recomputed by the oracle (y, y_meta and the final state)."""
    from tests.gpu_util import alloc_state, make_layer
    case = CASES[1]
    dims = case.dims.replace(norm_group=128)
    B, L = case.batch, case.seq_len
    w = gen_layer_weights(dims, case.case_id)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, B, L)
    layer = make_layer(dims, w)
    st = alloc_state(dims, B)
    y, ym = layer.prefill(meta_t.to(DEV), x_t.to(DEV), state_out=state_struct(st))
    torch.cuda.synchronize()
    b = 3
    ref = orc.prefill(dims, w, meta, x[b:b + 1], contract=True)
    errs = {"y": rel_err(to_np(y[b]), ref["y"][0]), "y_meta": rel_err(to_np(ym), ref["y_meta"][0]),
            "h": h_err(to_np(st["h"][b]), ref["h"][0])}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] < TOL_BF16 and errs["y_meta"] < TOL_BF16 and errs["h"] < TOL_H
