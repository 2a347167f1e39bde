"""Pins of the oracle's Mamba-2 head (dims.ssm_heads > 0) against things other than
itself: the (already pinned) per-channel selective scan with dt and A held constant
across each head, the summary's explicit mixing-matrix form of the SSM, a hand-worked
example, closed forms, and the whole layer assembled from torch routines."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import oracle as orc
from synth import F32, LayerDims, gen_activations, gen_layer_weights

rs = np.random.default_rng


def _inputs(T, H, P, N, seed):
    g = rs(seed)
    Di = H * P
    x = g.standard_normal((T, Di))
    dt = np.log1p(np.exp(g.uniform(-4, -1, (T, H))))
    A = -np.exp(g.uniform(0, 2, H))
    B = g.standard_normal((T, N))
    C = g.standard_normal((T, N))
    D = g.standard_normal(Di)
    return x, dt, A, B, C, D


def _per_channel(dt, A, P, N):
    """dt [T, H] -> [T, H*P]; A [H] -> [H*P, N]: the head's values on every channel."""
    return np.repeat(dt, P, axis=1), np.repeat(A, P)[:, None] * np.ones((1, N))


@pytest.mark.parametrize("T,H,P,N,seed", [(9, 2, 3, 4, 1), (16, 3, 4, 2, 2), (1, 1, 5, 3, 3)])
def test_head_scan_equals_selective_scan_with_head_constant_parameters(T, H, P, N, seed):
    x, dt, A, B, C, D = _inputs(T, H, P, N, seed)
    dtc, Ac = _per_channel(dt, A, P, N)
    h0 = rs(seed + 10).standard_normal((H * P, N))
    for init in (None, h0):
        y2, s2 = orc.ssm2_scan(x, dt, A, B, C, D, h0=init)
        y1, s1 = orc.selective_scan(x, dtc, Ac, B, C, D, h0=init)
        np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s2, s1, rtol=1e-13, atol=1e-13)


def test_matrix_form_equals_recurrence_and_summary_mixing_form():
    x, dt, A, B, C, D = _inputs(11, 2, 3, 4, 5)
    y_rec, _ = orc.ssm2_scan(x, dt, A, B, C, D)
    y_mat = orc.ssd_matrix_form(x, dt, A, B, C, D)
    dtc, Ac = _per_channel(dt, A, 3, 4)
    y_mix = orc.ssm_mixing_form(x, dtc, Ac, B, C, D)  # the summary's alpha_{i,j} form
    np.testing.assert_allclose(y_mat, y_rec, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y_mix, y_rec, rtol=1e-12, atol=1e-12)


def test_head_scan_hand_worked_example():
    # One head, P = 2, N = 1, A = -ln 2, dt = 1 (decay 1/2), B = (1, 3), C = (5, 7), D = 1/2.
    # t0: S = [2, 1] * 1 = [2, 1];       y0 = 5 S + D x0 = [10 + 1, 5 + 0.5] = [11, 5.5]
    # t1: S = [1, 0.5] + [4, 0] * 3 = [13, 0.5];  y1 = 7 S + D x1 = [91 + 2, 3.5] = [93, 3.5]
    x = np.array([[2.0, 1.0], [4.0, 0.0]])
    dt = np.ones((2, 1))
    A = np.array([-math.log(2.0)])
    B = np.array([[1.0], [3.0]])
    C = np.array([[5.0], [7.0]])
    D = np.array([0.5, 0.5])
    y, s = orc.ssm2_scan(x, dt, A, B, C, D)
    np.testing.assert_allclose(y, [[11.0, 5.5], [93.0, 3.5]], rtol=1e-14)
    np.testing.assert_allclose(s, [[13.0], [0.5]], rtol=1e-14)


def test_head_scan_closed_forms():
    T, H, P, N = 8, 2, 3, 4
    x, dt, A, B, C, D = _inputs(T, H, P, N, 6)
    dtc = np.repeat(dt, P, axis=1)
    # A = 0: the state is the prefix sum of dt_j x_j B_j
    y, s = orc.ssm2_scan(x, dt, np.zeros(H), B, C, D)
    hs = np.cumsum((dtc * x)[:, :, None] * B[:, None, :], axis=0)
    np.testing.assert_allclose(s, hs[-1], rtol=1e-12)
    np.testing.assert_allclose(y, np.einsum("tcn,tn->tc", hs, C) + D * x, rtol=1e-11, atol=1e-12)
    # decay 0: only the current token's input term remains
    y, _ = orc.ssm2_scan(x, dt, np.full(H, -1e300), B, C, D)
    np.testing.assert_allclose(y, dtc * x * np.sum(B * C, axis=1)[:, None] + D * x, rtol=1e-12)


def tiny2(**kw):
    base = dict(d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_inner=12, d_state=3,
                dt_rank=0, n_meta=3, window=0, kv_share=0, dtype=F32, ssm_heads=3)
    base.update(kw)
    return LayerDims(**base)


def _layer(dims, B, L, case):
    w = gen_layer_weights(dims, case)
    _, meta, _, X = gen_activations(dims, case, B, L)
    return w, meta.astype(np.float64), X.astype(np.float64)


def test_layer_with_head_ssm_matches_torch_composition():
    """Attention by torch's SDPA, dt by torch's softplus, the SSM by the alpha mixing
    matrix on the head's values repeated per channel, norms by torch's rms_norm."""
    dims = tiny2(n_meta=2)
    w, meta, X = _layer(dims, B=1, L=6, case=95)
    out = orc.prefill(dims, w, meta, X)
    f64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    xt = f64(np.concatenate([meta, X[0]]))
    z = xt @ f64(w.w_in).T
    qw, kw, Di, H, N = dims.q_width, dims.kv_width, dims.d_inner, dims.ssm_heads, dims.d_state
    T = z.shape[0]
    q = z[:, :qw].reshape(T, 4, 8).permute(1, 0, 2)
    k = z[:, qw:qw + kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    v = z[:, qw + kw:qw + 2 * kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    o = TF.scaled_dot_product_attention(q, k, v, is_causal=True).permute(1, 0, 2).reshape(T, qw)
    xs = z[:, qw + 2 * kw:qw + 2 * kw + Di]
    gg = z[:, qw + 2 * kw + Di:]
    xbc = xs @ f64(w.w_x).T
    dt = TF.softplus(xbc[:, :H] + f64(w.dt_bias), threshold=1e9).numpy()
    dtc, Ac = _per_channel(dt, w.A.astype(np.float64), Di // H, N)
    ymix = orc.ssm_mixing_form(xs.numpy(), dtc, Ac, xbc[:, H:H + N].numpy(),
                               xbc[:, H + N:].numpy(), w.D)
    yssm = torch.from_numpy(ymix) * TF.silu(gg)
    fa = TF.rms_norm(o, (qw,), eps=1e-6) * f64(w.beta_attn)
    fs = TF.rms_norm(yssm, (Di,), eps=1e-6) * f64(w.beta_ssm)
    Y = 0.5 * torch.cat([fa, fs], 1) @ f64(w.w_out).T
    np.testing.assert_allclose(out["y"][0], Y[dims.n_meta:].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["y_meta"][0], Y[:dims.n_meta].numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("window,slots,L,k", [(0, 16, 6, 5), (4, 4, 9, 4)])
def test_head_ssm_decode_continues_prefill(window, slots, L, k):
    dims = tiny2(window=window)
    w, meta, X = _layer(dims, B=2, L=L + k, case=96)
    long = orc.prefill(dims, w, meta, X, ring_slots=slots)
    short = orc.prefill(dims, w, meta, X[:, :L], ring_slots=slots)
    st = dict(k=short["k"], v=short["v"], h=short["h"], pos=np.full(2, L))
    for s in range(k):
        out = orc.decode_step(dims, w, X[:, L + s], short["k_meta"], short["v_meta"],
                              st["k"], st["v"], st["h"], st["pos"])
        np.testing.assert_allclose(out["y"], long["y"][:, L + s], rtol=1e-11, atol=1e-12)
        st = out
    np.testing.assert_allclose(st["h"], long["h"], rtol=1e-12)


# ---------------------------------------------------------------- group-norm fusion

def test_group_normalize_matches_torch_group_norm():
    """The oracle's group normalisation is torch's group_norm (no affine) on rows of
    [batch, channels], and closed forms on tiny groups."""
    g = rs(21)
    x = g.standard_normal((5, 48)) * 3 + 1
    for group in (8, 16, 48):
        ref = TF.group_norm(torch.from_numpy(x), 48 // group, eps=1e-5).numpy()
        np.testing.assert_allclose(orc.group_normalize(x, group, 1e-5), ref, rtol=1e-12, atol=1e-12)
    # a constant group maps to 0; a two-value group (a, b) to (-1, +1) sqrt(v / (v + eps))
    np.testing.assert_allclose(orc.group_normalize(np.full((1, 4), 7.0), 4, 1e-6), 0.0, atol=0)
    v = ((3.0 - 1.0) / 2) ** 2
    np.testing.assert_allclose(orc.group_normalize(np.array([[1.0, 3.0]]), 2, 1e-6),
                               [[-np.sqrt(v / (v + 1e-6)), np.sqrt(v / (v + 1e-6))]], rtol=1e-14)


def test_group_norm_layer_matches_torch_composition():
    """The layer with norm_group = 4: the branch norms by torch's group_norm, the rest as
    in the default layer (SDPA attention, the SSM through the alpha mixing matrix)."""
    dims = LayerDims(d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_inner=12, d_state=3,
                     dt_rank=2, n_meta=2, window=0, kv_share=0, dtype=F32, norm_group=4)
    w, meta, X = _layer(dims, B=1, L=6, case=97)
    out = orc.prefill(dims, w, meta, X)
    f64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    z = f64(np.concatenate([meta, X[0]])) @ f64(w.w_in).T
    qw, kw, Di, N, R = 32, 16, 12, 3, 2
    T = z.shape[0]
    q = z[:, :qw].reshape(T, 4, 8).permute(1, 0, 2)
    k = z[:, qw:qw + kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    v = z[:, qw + kw:qw + 2 * kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    o = TF.scaled_dot_product_attention(q, k, v, is_causal=True).permute(1, 0, 2).reshape(T, qw)
    xs, gg = z[:, qw + 2 * kw:qw + 2 * kw + Di], z[:, qw + 2 * kw + Di:]
    xdbl = xs @ f64(w.w_x).T
    dt = TF.softplus(xdbl[:, :R] @ f64(w.w_dt).T + f64(w.dt_bias), threshold=1e9)
    ymix = orc.ssm_mixing_form(xs.numpy(), dt.numpy(), w.A, xdbl[:, R:R + N].numpy(),
                               xdbl[:, R + N:].numpy(), w.D)
    yssm = torch.from_numpy(ymix) * TF.silu(gg)
    fa = TF.group_norm(o, qw // 4, eps=1e-6) * f64(w.beta_attn)
    fs = TF.group_norm(yssm, Di // 4, eps=1e-6) * f64(w.beta_ssm)
    Y = 0.5 * torch.cat([fa, fs], 1) @ f64(w.w_out).T
    np.testing.assert_allclose(out["y"][0], Y[2:].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["y_meta"][0], Y[:2].numpy(), rtol=1e-10, atol=1e-12)
