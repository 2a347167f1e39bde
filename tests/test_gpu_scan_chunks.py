"""Chunk-size invariance of the chunk-carried scan.

The scan's definition does not depend on how the sequence is cut ("Hymba: A
Hybrid-head Architecture for Small Language Models", Design formulation: the mixing
coefficient alpha_{i,j} is a product over every token between j and i, whatever chunk
they fall in).  The same inputs are scanned with several time-chunk lengths (one chunk,
chunks of 16 tokens, ragged last chunks) through the C ABI: every result is held to the
oracle at the usual tolerances, and the results are held to each other more tightly,
since they differ only in fp32 rounding order (h) and in the bf16 rounding that follows
(y: at most one bf16 step of the element)."""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_proj_amd as hy
import oracle as orc
from synth import BF16, gen_activations, gen_layer_weights, rng, to_storage
from tests.gpu_util import (DEV, alloc_state, elem_err, h_err, make_layer, rel_err, state_struct,
                            to_np)

pytestmark = pytest.mark.gpu


def _normal(g, shape, std=1.0):
    return (g.standard_normal(size=shape) * std).astype(np.float32)


def _op_scan(inputs, Di, N, R, M, L, B, chunk):
    zt, zld, dlt_t, bc, wdt_t, bias, A, D = inputs
    rows = M + B * L
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    y = torch.zeros(rows, Di, dtype=torch.bfloat16, device=DEV)
    h = torch.zeros(B, Di, N, dtype=torch.float32, device=DEV)
    ws_n = hy.hymba_op_scan_workspace_bytes(hy.DTYPE_BF16, M, L, B, Di, N, R, chunk)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=DEV)
    print(f"op_scan Di={Di} N={N} M={M} L={L} B={B} chunk={chunk}", flush=True)
    hy.hymba_op_scan(hy.DTYPE_BF16, zt, zld, 8, 8 + Di, dlt_t, dev(bc), wdt_t, dev(bias), dev(A),
                     dev(D), y, Di, h, M, L, B, Di, N, R, chunk, ws, ws.numel())
    torch.cuda.synchronize()
    return to_np(y), to_np(h)


@pytest.mark.parametrize("Di,N,R,M,L,B", [
    (256, 16, 128, 8, 300, 2),
    (128, 128, 128, 16, 257, 1),
])
def test_op_scan_chunk_size_invariance(Di, N, R, M, L, B):
    g = rng(77 + N, 3)
    rows = M + B * L
    zld = 2 * Di + 16
    zt, z = to_storage(_normal(g, (rows, zld)), BF16)
    dlt_t, dlt = to_storage(_normal(g, (rows, R), 0.5), BF16)
    bc = _normal(g, (rows, 2 * N))
    wdt_t, wdt = to_storage(_normal(g, (Di, R), 0.1), BF16)
    bias = g.uniform(-4, -2, Di).astype(np.float32)
    A = (-np.exp(g.uniform(0, 2, (Di, N)))).astype(np.float32)
    D = _normal(g, (Di,))
    inputs = (zt.to(DEV), zld, dlt_t.to(DEV), bc, wdt_t.to(DEV), bias, A, D)
    # oracle (bf16 storage of the inputs, fp64 arithmetic)
    dt = orc.softplus(dlt.astype(np.float64) @ wdt.astype(np.float64).T + bias)
    ref_y = np.zeros((rows, Di))
    ref_h = np.zeros((B, Di, N))
    for b in range(B):
        idx = np.concatenate([np.arange(M), M + b * L + np.arange(L)]).astype(np.int64)
        yy, hT = orc.selective_scan(z[idx, 8:8 + Di], dt[idx], A, bc[idx, :N], bc[idx, N:], D)
        out = orc.gate(yy, z[idx, 8 + Di:8 + 2 * Di])
        ref_y[idx] = out
        ref_h[b] = hT
    results = {}
    for chunk in (0, 16, 48, 64, 112, 256, ((L + 15) // 16) * 16):
        y, h = _op_scan(inputs, Di, N, R, M, L, B, chunk)
        ey, eh = rel_err(y, ref_y), h_err(h, ref_h)
        print(f"chunk {chunk}: y err {ey:.2e} (elementwise {elem_err(y, ref_y):.2e}) "
              f"h err {eh:.2e}")
        assert ey < 2e-2 and eh < 1e-3, (chunk, ey, eh)
        assert elem_err(y, ref_y) < 2e-2, chunk
        results[chunk] = (y, h)
    y0, h0 = results[((L + 15) // 16) * 16]  # one chunk: the plain serial scan
    for chunk, (y, h) in results.items():
        dh = rel_err(h, h0)
        # y: within one bf16 step (at most 2^-7 of the value) of the one-chunk result,
        # elementwise: a value next to a rounding boundary may round the other way
        step = np.maximum(np.abs(y0), np.abs(y)) * 2.0 ** -7 + 1e-6 * np.max(np.abs(y0))
        bad = np.abs(y - y0) > step
        print(f"chunk {chunk} vs one chunk: h {dh:.2e}, y elements off by more than a bf16 "
              f"step: {int(bad.sum())}")
        assert dh < 2e-5, (chunk, dh)
        assert not bad.any(), chunk


@pytest.mark.parametrize("N", [16, 128])
def test_layer_scan_chunk_size_invariance(N):
    """A whole bf16 layer (d 256, 8x64 q / 2 kv heads, Di 512) over B=1, L=700 with 16
    meta tokens: the library's own chunk choice, chunks of 16 / 128 tokens and one chunk,
    each against the oracle (storage-contract mode) and against each other."""
    from synth import LayerDims
    dims = LayerDims(d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                     d_state=N, dt_rank=64, n_meta=16, window=0, dtype=BF16)
    B, L = 1, 700
    w = gen_layer_weights(dims, 31)
    meta_t, meta, x_t, x = gen_activations(dims, 31, B, L)
    ref = orc.prefill(dims, w, meta, x, contract=True)
    outs = {}
    for chunk in (0, 16, 128, 704):
        d = dims.replace(scan_chunk=chunk)
        print(f"layer N={N} chunk={chunk}", flush=True)
        layer = make_layer(d, w)
        st = alloc_state(d, B)
        y, ym = layer.prefill(meta_t.to(DEV), x_t.to(DEV), state_out=state_struct(st))
        torch.cuda.synchronize()
        yy, hh = to_np(y), to_np(st["h"])
        ey, eh = rel_err(yy, ref["y"]), h_err(hh, ref["h"])
        ee = elem_err(yy, ref["y"])
        print(f"  y {ey:.2e} (elementwise {ee:.2e}) y_meta {rel_err(to_np(ym), ref['y_meta'][0]):.2e}"
              f" h {eh:.2e}")
        assert ey < 2e-2 and ee < 2e-2 and eh < 1e-3
        outs[chunk] = (yy, hh)
    y1, h1 = outs[704]
    for chunk, (yy, hh) in outs.items():
        assert rel_err(hh, h1) < 2e-5, chunk
        assert rel_err(yy, y1) < 1e-2, chunk
