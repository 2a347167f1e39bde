"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Tolerances (relative to the tensor's max magnitude): fp32 layers 1e-4; bf16 outputs
(y, y_meta, K/V cache) 2e-2; the fp32 SSM state 1e-3 against the oracle in bf16
storage-contract mode (it rounds to bf16 where the GPU stores bf16).  bf16 outputs are
also held to 2e-2 against the pure fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from synth import BF16, F32, CASES, LayerDims, gen_activations, gen_layer_weights
from tests.gpu_util import (DEV, alloc_kv, alloc_state, h_err, kv_struct, make_layer, rel_err,
                            state_struct, to_np)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_H = 1e-3


def small_dims(**kw):
    base = dict(d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=128, d_inner=512, d_state=16,
                dt_rank=16, n_meta=16, window=0, kv_share=0, dtype=BF16)
    base.update(kw)
    return LayerDims(**base)


def gpu_prefill(dims, wts, meta_t, x_t, ring_slots=None, kv_in=None):
    layer = make_layer(dims, wts)
    meta, x = meta_t.to(DEV), x_t.to(DEV)
    B = x.shape[0]
    kv = alloc_kv(dims, B, ring_slots) if (ring_slots and not dims.kv_share) else None
    st = alloc_state(dims, B)
    y, ym = layer.prefill(meta, x, kv_in=kv_struct(kv_in) if kv_in is not None else None,
                          kv_out=kv_struct(kv) if kv is not None else None,
                          state_out=state_struct(st))
    torch.cuda.synchronize()
    out = dict(y=to_np(y), y_meta=to_np(ym), h=to_np(st["h"]), pos=st["pos"].cpu().numpy(),
               y_t=y, y_meta_t=ym, kv_t=kv, state_t=st, layer=layer)
    if kv is not None:
        out.update({k: to_np(v) for k, v in kv.items()})
    return out


def check_prefill(dims, g, ref, tol_y, tol_h, pure=None, ring=False):
    M = dims.n_meta
    errs = {"y": rel_err(g["y"], ref["y"]), "h": h_err(g["h"], ref["h"])}
    if M:
        errs["y_meta"] = rel_err(g["y_meta"], ref["y_meta"][0])
    if ring:
        errs["k"] = rel_err(g["k"], ref["k"])
        errs["v"] = rel_err(g["v"], ref["v"])
        if M:
            errs["k_meta"] = rel_err(g["k_meta"][:, :M], ref["k_meta"])
            errs["v_meta"] = rel_err(g["v_meta"][:, :M], ref["v_meta"])
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v < (tol_h if k == "h" else tol_y), (k, v)
    assert np.all(g["pos"] == g["y"].shape[1])
    if pure is not None:
        e = rel_err(g["y"], pure["y"])
        print("pure-oracle y err", f"{e:.2e}")
        assert e < tol_y


# ---------------------------------------------------------------- fp32 configuration

def test_tiny_fp32_prefill_matches_oracle():
    case = CASES[0]
    dims = case.dims
    w = gen_layer_weights(dims, case.case_id)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, case.batch, case.seq_len)
    ref = orc.prefill(dims, w, meta, x, ring_slots=case.seq_len)
    g = gpu_prefill(dims, w, meta_t, x_t, ring_slots=case.seq_len)
    check_prefill(dims, g, ref, TOL_F32, TOL_F32, ring=True)


def test_tiny_fp32_decode_steps_match_oracle():
    case = CASES[0]
    dims = case.dims.replace(window=24)
    B, L, S, steps = 2, 40, 24, 12  # the ring wraps during the steps
    w = gen_layer_weights(dims, case.case_id)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], ring_slots=S)
    layer = make_layer(dims, w)
    kv = {k: torch.from_numpy(ref[k].astype(np.float32)).to(DEV).contiguous()
          for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": torch.from_numpy(ref["h"].astype(np.float32)).to(DEV),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    for s in range(steps):
        xs = torch.from_numpy(x[:, L + s].copy()).to(DEV)
        y = layer.decode(xs, kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"], o["v"],
                            o["h"], o["pos"])
        torch.cuda.synchronize()
        assert rel_err(to_np(y), o["y"]) < TOL_F32, s
    assert rel_err(to_np(st["h"]), o["h"]) < TOL_F32
    assert rel_err(to_np(kv["k"]), o["k"]) < TOL_F32
    assert np.all(st["pos"].cpu().numpy() == L + steps)


def test_fp32_wide_rows_norm_matches_oracle():
    """Rows of F wider than the 8192 values the register-resident row norm holds (128
    attention + 8192 SSM channels): the prefill's in-place branch norm takes its two-pass
    form; decode steps from the oracle's state follow."""
    case = CASES[0]
    dims = case.dims.replace(d_inner=8192)
    B, L, S, steps = 2, 32, 40, 3
    w = gen_layer_weights(dims, 91)
    meta_t, meta, x_t, x = gen_activations(dims, 91, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], ring_slots=S)
    g = gpu_prefill(dims, w, meta_t, x_t[:, :L].contiguous(), ring_slots=S)
    check_prefill(dims, g, ref, TOL_F32, TOL_F32, ring=True)
    layer = g["layer"]
    kv = {k: torch.from_numpy(ref[k].astype(np.float32)).to(DEV).contiguous()
          for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": torch.from_numpy(ref["h"].astype(np.float32)).to(DEV),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    for s_ in range(steps):
        xs = torch.from_numpy(x[:, L + s_].copy()).to(DEV)
        y = layer.decode(xs, kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s_], ref["k_meta"], ref["v_meta"], o["k"],
                            o["v"], o["h"], o["pos"])
        torch.cuda.synchronize()
        assert rel_err(to_np(y), o["y"]) < TOL_F32, s_
    assert rel_err(to_np(st["h"]), o["h"]) < TOL_F32


# ---------------------------------------------------------------- bf16, small shapes

@pytest.mark.parametrize("window,head_dim,n_kv,M,L,B", [
    (0, 128, 2, 16, 200, 2),     # full causal, several 64-key tiles + ragged tail
    (48, 128, 2, 16, 200, 2),    # sliding window smaller than L
    (0, 64, 4, 8, 97, 3),        # head_dim 64, 2 q heads per kv head
    (33, 128, 8, 0, 130, 1),     # no meta tokens, MHA
    (0, 128, 1, 70, 150, 2),     # meta prefix spanning two key tiles, 8 q heads per kv head
])
def test_small_bf16_prefill(window, head_dim, n_kv, M, L, B):
    dims = small_dims(window=window, head_dim=head_dim, n_kv_heads=n_kv, n_meta=M)
    cid = 60 + head_dim + window + M
    w = gen_layer_weights(dims, cid)
    meta_t, meta, x_t, x = gen_activations(dims, cid, B, L)
    ring = 64
    ref = orc.prefill(dims, w, meta, x, contract=True, ring_slots=ring)
    pure = orc.prefill(dims, w, meta, x)
    g = gpu_prefill(dims, w, meta_t, x_t, ring_slots=ring)
    check_prefill(dims, g, ref, TOL_BF16, TOL_H, pure=pure, ring=True)


@pytest.mark.parametrize("d_state", [4, 32, 64, 128])
def test_small_bf16_prefill_state_sizes(d_state):
    dims = small_dims(d_state=d_state, window=40, d_inner=256)
    cid = 70 + d_state
    w = gen_layer_weights(dims, cid)
    meta_t, meta, x_t, x = gen_activations(dims, cid, 2, 77)
    ref = orc.prefill(dims, w, meta, x, contract=True)
    g = gpu_prefill(dims, w, meta_t, x_t)
    check_prefill(dims, g, ref, TOL_BF16, TOL_H)


@pytest.mark.parametrize("d_state,dt_rank,L,M,B", [
    (16, 128, 77, 16, 2),    # ragged last chunk, meta prefix inside the first chunk
    (128, 64, 45, 40, 1),    # meta prefix spanning two chunks
    (32, 64, 64, 8, 3),      # exact chunk multiple
    (64, 128, 100, 0, 2),    # no meta tokens
    (32, 128, 50, 8, 2),     # x_proj of 192 columns (6 column waves)
])
def test_small_bf16_prefill_fused_dt_scan(d_state, dt_rank, L, M, B):
    """Shapes whose dt projection runs inside the scan kernel (dt_rank 64 or 128)."""
    dims = small_dims(d_state=d_state, dt_rank=dt_rank, n_meta=M, window=30, d_inner=512)
    cid = 75 + d_state + dt_rank + M
    w = gen_layer_weights(dims, cid)
    meta_t, meta, x_t, x = gen_activations(dims, cid, B, L)
    ref = orc.prefill(dims, w, meta, x, contract=True)
    g = gpu_prefill(dims, w, meta_t, x_t)
    check_prefill(dims, g, ref, TOL_BF16, TOL_H)


def test_small_bf16_kv_share_pair():
    """Producer then consumer; the consumer reads the producer's cache, takes the
    producer's y as its X and y_meta as its meta rows.

    Strict check: the GPU consumer gets exactly the oracle's inputs (its bf16-rounded
    y, y_meta and K/V), so the 1e-3 state gate measures this layer alone.  Chained
    check: GPU producer -> GPU consumer end to end; the consumer's input then carries
    the producer's own rounding differences, so only the bf16 output gate applies."""
    p_dims = small_dims(window=40)
    c_dims = p_dims.replace(kv_share=1)
    B, L = 2, 150
    w1 = gen_layer_weights(p_dims, 81)
    w2 = gen_layer_weights(c_dims, 81, layer=1)
    meta_t, meta, x_t, x = gen_activations(p_dims, 81, B, L)
    r1 = orc.prefill(p_dims, w1, meta, x, contract=True, ring_slots=L)
    x2 = orc.bf16_round(r1["y"])
    m2 = orc.bf16_round(r1["y_meta"][0])
    r2 = orc.prefill(c_dims, w2, m2, x2, contract=True,
                     kv_src=[{"K": r1["K"][b], "V": r1["V"][b]} for b in range(B)])
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    kv_oracle = {k: bf(r1[k]).to(DEV) for k in ("k_meta", "v_meta", "k", "v")}
    g2s = gpu_prefill(c_dims, w2, bf(m2), bf(x2), kv_in=kv_oracle)
    check_prefill(c_dims, g2s, r2, TOL_BF16, TOL_H)
    g1 = gpu_prefill(p_dims, w1, meta_t, x_t, ring_slots=L)
    check_prefill(p_dims, g1, r1, TOL_BF16, TOL_H, ring=True)
    g2 = gpu_prefill(c_dims, w2, g1["y_meta_t"], g1["y_t"], kv_in=g1["kv_t"])
    e = {k: rel_err(g2[k], r2[k] if k != "y_meta" else r2[k][0]) for k in ("y", "y_meta", "h")}
    print("chained", {k: f"{v:.2e}" for k, v in e.items()})
    assert e["y"] < TOL_BF16 and e["y_meta"] < TOL_BF16


def test_small_bf16_decode_ring_wrap():
    dims = small_dims(window=32)
    B, L, S, steps = 3, 50, 32, 20
    w = gen_layer_weights(dims, 83)
    meta_t, meta, x_t, x = gen_activations(dims, 83, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
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
    assert rel_err(to_np(kv["k"]), o["k"]) < TOL_BF16
    assert rel_err(to_np(kv["v"]), o["v"]) < TOL_BF16
    assert np.all(st["pos"].cpu().numpy() == L + steps)


@pytest.mark.parametrize("B", [9, 40])
def test_small_bf16_decode_fewrow_batches(B):
    """Batches between the one-to-four-row kernel and the streaming attention: the
    projections take the 128-row few-row GEMMs with a partly filled row block (in_proj
    with the ring write, x_proj split-K into atomics in 64-row blocks, out_proj split-K
    partials and their slice sum), and the attention the key-split path (B x 2 kv heads
    below 256)."""
    dims = small_dims(window=48)
    L, S, steps = 60, 48, 5
    w = gen_layer_weights(dims, 87)
    meta_t, meta, x_t, x = gen_activations(dims, 87, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
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
    assert rel_err(to_np(kv["k"]), o["k"]) < TOL_BF16
    assert rel_err(to_np(kv["v"]), o["v"]) < TOL_BF16
    assert np.all(st["pos"].cpu().numpy() == L + steps)


def test_small_bf16_decode_wide_rows_key_splits():
    """bf16 decode with rows of F wider than the register-resident row norm holds (1024
    attention + 7680 SSM channels = 8704 values) and more than 8 key splits (16 meta +
    640 ring keys in splits of 64): the split merge, then the two-pass row norm."""
    dims = small_dims(window=0, d_inner=7680)
    B, L, S, steps = 2, 600, 640, 3
    w = gen_layer_weights(dims, 92)
    meta_t, meta, x_t, x = gen_activations(dims, 92, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s_ in range(steps):
        y = layer.decode(xb[:, L + s_].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s_], ref["k_meta"], ref["v_meta"], o["k"],
                            o["v"], o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        e = rel_err(to_np(y), o["y"])
        assert e < TOL_BF16, (s_, e)
    assert h_err(to_np(st["h"]), o["h"]) < TOL_H


def test_small_bf16_decode_many_key_splits():
    """Global attention over a 2400-slot cache at a small batch: 16 meta + 2400 keys make
    38 key splits of 64 (more than the 8 the fixed-size merge holds, so the grouped merge
    runs), the last ones past every position (empty splits)."""
    dims = small_dims(window=0)
    B, L, S, steps = 2, 2200, 2400, 6
    w = gen_layer_weights(dims, 86)
    meta_t, meta, x_t, x = gen_activations(dims, 86, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
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


def test_bf16_ragged_k_slices():
    """d_model 1024 and out_proj K = 1024 + 3328 = 4352 (17 units of 256): the split-K
    out_proj (meta rows in prefill, the batch in decode) wants 16 slices of its 16 column
    tiles, so it runs 9 slices of 2 units with a last slice of 1 unit."""
    dims = small_dims(d_model=1024, d_inner=3328, window=32)
    B, L, S, steps = 2, 40, 32, 4
    w = gen_layer_weights(dims, 85)
    meta_t, meta, x_t, x = gen_activations(dims, 85, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    got = gpu_prefill(dims, w, meta_t, x_t[:, :L].contiguous(), ring_slots=S)
    check_prefill(dims, got, ref, TOL_BF16, TOL_H, ring=True)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
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


@pytest.mark.parametrize("head_dim,n_kv", [(128, 2), (64, 4)])
def test_bf16_decode_streaming_attention(head_dim, n_kv):
    """Batches whose sequences x kv heads fill the chip (>= 256) take the decode
    attention that streams every key of a (sequence, kv head) in one workgroup; the
    96-slot ring wraps during the steps."""
    dims = small_dims(window=96, head_dim=head_dim, n_kv_heads=n_kv)
    B, L, S, steps = 256 // n_kv, 90, 96, 10
    w = gen_layer_weights(dims, 84)
    meta_t, meta, x_t, x = gen_activations(dims, 84, B, L + steps)
    ref = orc.prefill(dims, w, meta, x[:, :L], contract=True, ring_slots=S)
    layer = make_layer(dims, w)
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(DEV)
    kv = {k: to_dev(ref[k], torch.bfloat16) for k in ("k_meta", "v_meta", "k", "v")}
    st = {"h": to_dev(ref["h"], torch.float32),
          "pos": torch.full((B,), L, dtype=torch.int32, device=DEV)}
    o = dict(k=ref["k"], v=ref["v"], h=ref["h"], pos=np.full(B, L))
    xb = x_t.to(DEV)
    for s in range(steps):
        y = layer.decode(xb[:, L + s].contiguous(), kv_struct(kv), state_struct(st))
        o = orc.decode_step(dims, w, x[:, L + s], ref["k_meta"], ref["v_meta"], o["k"], o["v"],
                            o["h"], o["pos"], contract=True)
        torch.cuda.synchronize()
        e = rel_err(to_np(y), o["y"])
        assert e < TOL_BF16, (s, e)
    print("last step y err", f"{e:.2e}")
    assert h_err(to_np(st["h"]), o["h"]) < TOL_H
    assert rel_err(to_np(kv["k"]), o["k"]) < TOL_BF16
    assert np.all(st["pos"].cpu().numpy() == L + steps)


def test_gemm_op_bf16_ragged():
    import hybrid_attention_ssm_proj_amd as hy
    g = np.random.default_rng(5)
    M, N, K = 300, 200, 264
    a = torch.from_numpy(g.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy(g.standard_normal((N, K)).astype(np.float32)).to(torch.bfloat16)
    ref = a.double().numpy() @ b.double().numpy().T
    ad, bd = a.to(DEV), b.to(DEV)
    c = torch.zeros(M, N, dtype=torch.float32, device=DEV)
    hy.hymba_op_gemm(hy.DTYPE_BF16, ad, K, bd, K, c, N, hy.DTYPE_F32, M, N, K)
    torch.cuda.synchronize()
    assert rel_err(to_np(c), ref) < 1e-5
    cb = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    hy.hymba_op_gemm(hy.DTYPE_BF16, ad, K, bd, K, cb, N, hy.DTYPE_BF16, M, N, K)
    torch.cuda.synchronize()
    assert rel_err(to_np(cb), ref) < 4e-3


def test_zero_values_and_zero_ssm_projection_give_zero_output():
    """With V's projection rows zero every attention output is 0, rms-normalising 0 gives
    0, and with the SSM columns of W_out zero the layer output is exactly 0."""
    dims = small_dims(window=20, n_meta=16)
    w = gen_layer_weights(dims, 84)
    qw, kw = dims.q_width, dims.kv_width
    w.torch["w_in"][qw + kw:qw + 2 * kw] = 0
    w.torch["w_out"][:, qw:] = 0
    meta_t, meta, x_t, x = gen_activations(dims, 84, 2, 90)
    g = gpu_prefill(dims, w, meta_t, x_t)
    assert np.max(np.abs(g["y"])) == 0.0
    assert np.max(np.abs(g["y_meta"])) == 0.0


# ---------------------------------------------------------------- full-size, sampled

def test_config1_full_size_sampled_sequences():
    """The bench workload (B=8, L=2048, 128 meta tokens, full causal): every sequence
    runs on the GPU; sequences 0 and 7 are recomputed by the oracle."""
    case = CASES[1]
    dims = case.dims
    w = gen_layer_weights(dims, case.case_id)
    meta_t, meta, x_t, x = gen_activations(dims, case.case_id, case.batch, case.seq_len)
    g = gpu_prefill(dims, w, meta_t, x_t, ring_slots=1024)
    for b in (0, case.batch - 1):
        ref = orc.prefill(dims, w, meta, x[b:b + 1], contract=True, ring_slots=1024)
        errs = {"y": rel_err(g["y"][b], ref["y"][0]), "y_meta": rel_err(g["y_meta"], ref["y_meta"][0]),
                "h": h_err(g["h"][b], ref["h"][0]), "k": rel_err(g["k"][b], ref["k"][0]),
                "v": rel_err(g["v"][b], ref["v"][0])}
        print(b, {k: f"{v:.2e}" for k, v in errs.items()})
        for k, v in errs.items():
            assert v < (TOL_H if k == "h" else TOL_BF16), (b, k, v)
