"""GPU parity of the block wrapper (hymba_block_prefill / hymba_block_decode: pre-norm,
the layer, residual, FFN with SiLU, residual) through the C ABI against the oracle's
block on the same seeded inputs.  Tolerances as for the layer: bf16 outputs 2e-2, the
fp32 state 1e-3, fp32 layers 1e-4, relative to the tensor's max magnitude, the oracle
in bf16 storage-contract mode for bf16 blocks."""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_proj_amd as hy
import oracle as orc
from synth import CASES, gen_activations, gen_block_weights, gen_layer_weights
from tests.gpu_util import (DEV, alloc_kv, alloc_state, h_err, kv_struct, rel_err, state_struct,
                            to_np)
from tests.test_gpu_parity import TOL_BF16, TOL_F32, TOL_H, small_dims

pytestmark = pytest.mark.gpu


def _block(dims, w, bw):
    return hy.HymbaBlock(dims, dict(w.torch), dict(bw.torch), device=DEV)


@pytest.mark.parametrize("inter,window,L,B", [
    (512, 0, 100, 2),   # intermediate a multiple of 256: few-row down-projections split K
    (768, 40, 70, 3),
    (520, 0, 33, 2),    # not a multiple of 64: generic-K tiles, few rows without split-K
])
def test_block_prefill_and_decode_match_oracle(inter, window, L, B):
    dims = small_dims(window=window)
    S, steps = max(L, 1), 3
    case = 600 + inter + window
    w = gen_layer_weights(dims, case)
    bw = gen_block_weights(dims, case, inter)
    meta_t, meta, x_t, x = gen_activations(dims, case, B, L + steps)
    ref = orc.block_prefill(dims, w, bw, meta, x[:, :L], contract=True, ring_slots=S + steps)
    blk = _block(dims, w, bw)
    kv = alloc_kv(dims, B, S + steps)
    st = alloc_state(dims, B)
    y, ym = blk.prefill(meta_t.to(DEV), x_t[:, :L].contiguous().to(DEV), kv_out=kv_struct(kv),
                        state_out=state_struct(st))
    torch.cuda.synchronize()
    errs = {"y": rel_err(to_np(y), ref["y"]), "y_meta": rel_err(to_np(ym), ref["y_meta"][0]),
            "h": h_err(to_np(st["h"]), ref["h"])}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] < TOL_BF16 and errs["y_meta"] < TOL_BF16 and errs["h"] < TOL_H
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s in range(steps):
        yd = blk.decode(xb[:, L + s].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.block_decode_step(dims, w, bw, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"],
                                  o["v"], o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        e = rel_err(to_np(yd), o["y"])
        assert e < TOL_BF16, (s, e)


def test_block_fp32_prefill_matches_oracle():
    dims = CASES[0].dims
    w = gen_layer_weights(dims, 610)
    bw = gen_block_weights(dims, 610, 256)
    meta_t, meta, x_t, x = gen_activations(dims, 610, 1, 64)
    ref = orc.block_prefill(dims, w, bw, meta, x)
    blk = _block(dims, w, bw)
    y, ym = blk.prefill(meta_t.to(DEV), x_t.to(DEV))
    torch.cuda.synchronize()
    assert rel_err(to_np(y), ref["y"]) < TOL_F32
    assert rel_err(to_np(ym), ref["y_meta"][0]) < TOL_F32


def test_block_full_size_sampled_sequence():
    """The block around the prefill workload's layer with intermediate 5632 (the shape
    the benchmark times), B=8, L=2048, 128 meta tokens, run on the whole batch; sequence 6
    is recomputed by the oracle's block (y, y_meta and the final state)."""
    case = CASES[1]
    dims, inter = case.dims, 5632
    B, L = case.batch, case.seq_len
    w = gen_layer_weights(dims, case.case_id)
    bw = gen_block_weights(dims, case.case_id, inter)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, B, L)
    blk = _block(dims, w, bw)
    st = alloc_state(dims, B)
    y, ym = blk.prefill(meta_t.to(DEV), x_t.to(DEV), state_out=state_struct(st))
    torch.cuda.synchronize()
    b = 6
    ref = orc.block_prefill(dims, w, bw, meta, x[b:b + 1], contract=True)
    errs = {"y": rel_err(to_np(y[b]), ref["y"][0]), "y_meta": rel_err(to_np(ym), ref["y_meta"][0]),
            "h": h_err(to_np(st["h"][b]), ref["h"][0])}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] < TOL_BF16 and errs["y_meta"] < TOL_BF16 and errs["h"] < TOL_H


def test_block_without_meta_tokens():
    """No meta tokens (M = 0: no meta rows, no few-row down-projection), one sequence of
    a ragged length, then two decode steps."""
    dims = small_dims(n_meta=0, window=0)
    B, L, steps = 1, 45, 2
    w = gen_layer_weights(dims, 620)
    bw = gen_block_weights(dims, 620, 512)
    meta_t, meta, x_t, x = gen_activations(dims, 620, B, L + steps)
    ref = orc.block_prefill(dims, w, bw, meta, x[:, :L], contract=True, ring_slots=L + steps)
    blk = _block(dims, w, bw)
    kv = alloc_kv(dims, B, L + steps)
    st = alloc_state(dims, B)
    y, _ = blk.prefill(meta_t.to(DEV), x_t[:, :L].contiguous().to(DEV), kv_out=kv_struct(kv),
                       state_out=state_struct(st))
    torch.cuda.synchronize()
    assert rel_err(to_np(y), ref["y"]) < TOL_BF16
    assert h_err(to_np(st["h"]), ref["h"]) < TOL_H
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s in range(steps):
        yd = blk.decode(xb[:, L + s].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.block_decode_step(dims, w, bw, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"],
                                  o["v"], o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        assert rel_err(to_np(yd), o["y"]) < TOL_BF16, s
