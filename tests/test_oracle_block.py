"""Pins of the oracle's block wrapper (pre-norm, residual, FFN) against things other than
itself: torch's rms_norm / linear / silu on the FFN and the whole block with the layer
taken from the (separately pinned) oracle layer, closed forms with zero weights, and
decode continuing prefill."""
import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import oracle as orc
from synth import F32, LayerDims, gen_activations, gen_block_weights, gen_layer_weights


def tiny(**kw):
    base = dict(d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_inner=12, d_state=3,
                dt_rank=2, n_meta=3, window=0, kv_share=0, dtype=F32)
    base.update(kw)
    return LayerDims(**base)


def _all(dims, B, L, case, inter=24):
    w = gen_layer_weights(dims, case)
    bw = gen_block_weights(dims, case, inter)
    _, meta, _, X = gen_activations(dims, case, B, L)
    return w, bw, meta.astype(np.float64), X.astype(np.float64)


def test_ffn_matches_torch():
    g = np.random.default_rng(3)
    v = g.standard_normal((7, 16))
    up, down = g.standard_normal((24, 16)), g.standard_normal((16, 24))
    ref = TF.linear(TF.silu(TF.linear(torch.from_numpy(v), torch.from_numpy(up))),
                    torch.from_numpy(down)).numpy()
    np.testing.assert_allclose(orc.ffn(v, up, down), ref, rtol=1e-12, atol=1e-12)


def test_block_matches_torch_composition():
    dims = tiny()
    w, bw, meta, X = _all(dims, B=2, L=5, case=501)
    out = orc.block_prefill(dims, w, bw, meta, X)
    f64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    for b in range(2):
        xt = f64(np.concatenate([meta, X[b]]))
        xn = TF.rms_norm(xt, (16,), weight=f64(bw.norm1), eps=dims.rms_eps).numpy()
        lay = orc.prefill(dims, w, xn[:3], xn[3:][None])  # the layer, pinned on its own
        u = xt + f64(np.concatenate([lay["y_meta"][0], lay["y"][0]]))
        v = TF.rms_norm(u, (16,), weight=f64(bw.norm2), eps=dims.rms_eps)
        ref = u + TF.linear(TF.silu(TF.linear(v, f64(bw.w_up))), f64(bw.w_down))
        np.testing.assert_allclose(out["y"][b], ref[3:].numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(out["y_meta"][b], ref[:3].numpy(), rtol=1e-11, atol=1e-12)


def test_block_zero_weights_is_identity():
    """With zero output and FFN projections both residual branches vanish."""
    dims = tiny()
    w, bw, meta, X = _all(dims, B=1, L=4, case=502)
    w.w_out[...] = 0.0
    bw.w_down[...] = 0.0
    out = orc.block_prefill(dims, w, bw, meta, X)
    np.testing.assert_allclose(out["y"], X, rtol=0, atol=0)
    np.testing.assert_allclose(out["y_meta"][0], meta, rtol=0, atol=0)


@pytest.mark.parametrize("window,slots", [(0, 12), (4, 4)])
def test_block_decode_continues_prefill(window, slots):
    dims = tiny(window=window)
    L, k = 6, 4
    w, bw, meta, X = _all(dims, B=2, L=L + k, case=503)
    long = orc.block_prefill(dims, w, bw, meta, X, ring_slots=slots)
    short = orc.block_prefill(dims, w, bw, meta, X[:, :L], ring_slots=slots)
    st = dict(k=short["k"], v=short["v"], h=short["h"], pos=np.full(2, L))
    for s in range(k):
        o = orc.block_decode_step(dims, w, bw, X[:, L + s], short["k_meta"], short["v_meta"],
                                  st["k"], st["v"], st["h"], st["pos"])
        np.testing.assert_allclose(o["y"], long["y"][:, L + s], rtol=1e-11, atol=1e-12)
        st = o
