"""Pins of the CPU oracle against things other than itself: the mixing-matrix form
of the SSM the Hymba summary prints, closed forms, library routines (torch CPU) on
special cases, brute force on tiny inputs, and invariants the method implies.
No test here retypes the oracle's own formula."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import oracle as orc
from synth import LayerDims, gen_layer_weights, gen_activations, F32

rs = np.random.default_rng


def tiny_dims(**kw):
    base = dict(d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_inner=12,
                d_state=3, dt_rank=2, n_meta=3, window=0, kv_share=0, dtype=F32)
    base.update(kw)
    return LayerDims(**base)


# ---------------------------------------------------------------- elementwise

def test_bf16_round_matches_torch_conversion():
    g = rs(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 10.0 ** g.integers(-6, 6, 20000),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -8 + 2 ** -16,
                  0.0, -0.0, 1.0, 65504.0, 3.0e38], np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = orc.bf16_round(x)
    assert np.array_equal(got, ref)
    # ties go to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert orc.bf16_round(1 + 2 ** -8) == 1.0
    assert orc.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def test_softplus_silu_match_torch():
    z = np.linspace(-40, 40, 4001)
    zt = torch.from_numpy(z)
    sp = TF.softplus(zt, beta=1.0, threshold=1e9).numpy()
    np.testing.assert_allclose(orc.softplus(z), sp, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(orc.silu(z), TF.silu(zt).numpy(), rtol=1e-13, atol=1e-300)
    # softplus at 0 is ln 2; for large z it approaches z
    assert abs(orc.softplus(0.0) - math.log(2.0)) < 1e-15
    assert abs(orc.softplus(30.0) - 30.0) < 1e-12


def test_rms_normalize_closed_forms_and_torch():
    eps = 1e-6
    for c in (-3.0, 0.5, 7.0):
        v = np.full((1, 10), c)
        np.testing.assert_allclose(orc.rms_normalize(v, eps), c / math.sqrt(c * c + eps),
                                   rtol=1e-15)
    v = rs(2).standard_normal((5, 33))
    ref = TF.rms_norm(torch.from_numpy(v), (33,), eps=eps).numpy()
    np.testing.assert_allclose(orc.rms_normalize(v, eps), ref, rtol=1e-13)


# ---------------------------------------------------------------- SSM scan

def _scan_inputs(T, Di, N, seed=3):
    g = rs(seed)
    x = g.standard_normal((T, Di))
    dt = np.log1p(np.exp(g.uniform(-4, -1, (T, Di))))
    A = -np.exp(g.uniform(0, 2, (Di, N)))
    B = g.standard_normal((T, N))
    C = g.standard_normal((T, N))
    D = g.standard_normal(Di)
    return x, dt, A, B, C, D


def test_scan_equals_alpha_mixing_matrix_bruteforce():
    """North-star check 1: the recurrence equals the summary's explicit
    alpha_{i,j} = C_i (prod_{k=j+1..i} exp(A dt_k)) B_j dt_j form."""
    for (T, Di, N, seed) in ((7, 3, 2, 3), (12, 4, 3, 4), (1, 2, 1, 5)):
        x, dt, A, B, C, D = _scan_inputs(T, Di, N, seed)
        y_rec, _ = orc.selective_scan(x, dt, A, B, C, D)
        y_mix = orc.ssm_mixing_form(x, dt, A, B, C, D)
        assert np.max(np.abs(y_rec - y_mix)) < 1e-12 * max(1.0, np.max(np.abs(y_mix)))


def test_scan_hand_worked_example():
    # Di = N = 1, A = -ln 2, dt = 1 -> decay 1/2.  x = (2, 4), B = (1, 3), C = (5, 7), D = 1/2.
    # h0 = 1*2*1 = 2, y0 = 5*2 + 1 = 11;  h1 = 2/2 + 1*4*3 = 13, y1 = 7*13 + 2 = 93.
    x = np.array([[2.0], [4.0]])
    dt = np.ones((2, 1))
    A = np.array([[-math.log(2.0)]])
    B = np.array([[1.0], [3.0]])
    C = np.array([[5.0], [7.0]])
    D = np.array([0.5])
    y, h = orc.selective_scan(x, dt, A, B, C, D)
    np.testing.assert_allclose(y[:, 0], [11.0, 93.0], rtol=1e-14)
    np.testing.assert_allclose(h, [[13.0]], rtol=1e-14)
    alpha = orc.ssm_alpha(dt, A, B, C)
    np.testing.assert_allclose(alpha[:, :, 0], [[5.0, 0.0], [3.5, 21.0]], rtol=1e-14)


def test_scan_closed_forms():
    T, Di, N = 9, 3, 4
    x, dt, A, B, C, D = _scan_inputs(T, Di, N, 6)
    # decay 0 (A -> -inf): only the current input term survives
    y, _ = orc.selective_scan(x, dt, np.full((Di, N), -1e300), B, C, D)
    ref = dt * x * np.sum(B * C, axis=1)[:, None] + D * x
    np.testing.assert_allclose(y, ref, rtol=1e-13)
    # A = 0: the state is a prefix sum of dt_j x_j B_j
    y, h = orc.selective_scan(x, dt, np.zeros((Di, N)), B, C, D)
    hs = np.cumsum((dt * x)[:, :, None] * B[:, None, :], axis=0)  # [T, Di, N]
    np.testing.assert_allclose(h, hs[-1], rtol=1e-13)
    np.testing.assert_allclose(y, np.einsum("tcn,tn->tc", hs, C) + D * x, rtol=1e-12, atol=1e-13)
    # constant dt, B, x: geometric series h_t = b (1 - a^(t+1)) / (1 - a)
    dt_c = np.full((T, Di), 0.3)
    x_c = np.ones((T, Di)) * 2.0
    B_c = np.tile(B[:1], (T, 1))
    _, h = orc.selective_scan(x_c, dt_c, A, B_c, C, D)
    a = np.exp(0.3 * A)
    b = 0.3 * 2.0 * B_c[0][None, :]
    np.testing.assert_allclose(h, b * (1 - a ** T) / (1 - a), rtol=1e-13)


def test_scan_state_chaining():
    x, dt, A, B, C, D = _scan_inputs(15, 3, 2, 7)
    y_all, h_all = orc.selective_scan(x, dt, A, B, C, D)
    y1, h1 = orc.selective_scan(x[:6], dt[:6], A, B[:6], C[:6], D)
    y2, h2 = orc.selective_scan(x[6:], dt[6:], A, B[6:], C[6:], D, h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y_all, rtol=1e-13)
    np.testing.assert_allclose(h2, h_all, rtol=1e-13)


# ---------------------------------------------------------------- attention

def _qkv(T, Hq, Hkv, dh, seed=8):
    g = rs(seed)
    return (g.standard_normal((T, Hq, dh)), g.standard_normal((T, Hkv, dh)),
            g.standard_normal((T, Hkv, dh)))


def test_attention_rows_sum_to_one_and_respect_mask():
    """North-star check 2."""
    T, M = 23, 4
    Q, K, V = _qkv(T, 4, 2, 8)
    pos = np.arange(T)
    for window in (0, 1, 5, 30):
        _, P = orc.attention(Q, K, V, pos, pos, M, window, 0.3, return_probs=True)
        np.testing.assert_allclose(P.sum(axis=2), 1.0, rtol=1e-14)
        for i in range(T):
            for j in range(T):
                allowed = j <= i and (window == 0 or j < M or i - j < window)
                if not allowed:
                    assert np.all(P[:, i, j] == 0.0)
                else:
                    assert np.all(P[:, i, j] > 0.0)


def test_attention_constant_values_give_constant_output():
    T = 17
    Q, K, _ = _qkv(T, 4, 2, 8)
    V = np.ones((T, 2, 8))
    pos = np.arange(T)
    for window in (0, 3):
        O = orc.attention(Q, K, V, pos, pos, 2, window, 0.5)
        np.testing.assert_allclose(O, 1.0, rtol=1e-14)


def test_attention_window_at_least_length_is_full_causal():
    """North-star check 3."""
    T, M = 29, 5
    Q, K, V = _qkv(T, 4, 1, 16)
    pos = np.arange(T)
    full = orc.attention(Q, K, V, pos, pos, M, 0, 0.25)
    for window in (T - M, T, T + 7, 10 ** 6):
        np.testing.assert_allclose(orc.attention(Q, K, V, pos, pos, M, window, 0.25), full,
                                   rtol=1e-14)
    # a window shorter than the span must differ
    assert np.max(np.abs(orc.attention(Q, K, V, pos, pos, M, 4, 0.25) - full)) > 1e-3


def test_attention_matches_torch_sdpa_causal_mha_and_gqa():
    T, dh = 31, 16
    for Hq, Hkv in ((4, 4), (4, 2), (8, 2), (6, 1)):
        Q, K, V = _qkv(T, Hq, Hkv, dh, seed=Hq + Hkv)
        pos = np.arange(T)
        O = orc.attention(Q, K, V, pos, pos, 0, 0, 1.0 / math.sqrt(dh))
        rep = Hq // Hkv
        qt = torch.from_numpy(Q).permute(1, 0, 2)[None]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
        ref = TF.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2)
        np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_attention_window_special_cases():
    T, M = 12, 3
    Q, K, V = _qkv(T, 2, 2, 8, seed=11)
    pos = np.arange(T)
    # window 1, no meta: every query sees only itself
    O = orc.attention(Q, K, V, pos, pos, 0, 1, 0.7)
    np.testing.assert_allclose(O, V, rtol=1e-14)
    # window 1 with M meta keys: query i >= M sees the meta keys and itself: a
    # softmax over M + 1 keys, computed here with torch on the gathered keys.
    O = orc.attention(Q, K, V, pos, pos, M, 1, 0.7)
    for i in range(M, T):
        idx = list(range(M)) + [i]
        for h in range(2):
            s = torch.from_numpy(Q[i, h] @ K[idx, h].T * 0.7)
            ref = torch.softmax(s, 0).numpy() @ V[idx, h]
            np.testing.assert_allclose(O[i, h], ref, rtol=1e-13)
    # a single visible key returns its value: the first query
    np.testing.assert_allclose(O[0], V[0], rtol=1e-14)


# ---------------------------------------------------------------- whole layer

def _layer(dims, B=2, L=9, case=90, **kw):
    w = gen_layer_weights(dims, case, std=kw.pop("std", 0.2))
    _, meta, _, X = gen_activations(dims, case, B, L)
    return w, meta, X


def test_beta_zero_isolates_each_branch():
    """North-star check 4."""
    dims = tiny_dims(window=4)
    w, meta, X = _layer(dims)
    qkv_cols = slice(0, dims.q_width + 2 * dims.kv_width)
    ssm_cols = slice(dims.q_width + 2 * dims.kv_width, dims.n_in)
    g = rs(12)
    # beta1 = 0: output independent of W_Q, W_K, W_V
    w.beta_attn[:] = 0.0
    y0 = orc.prefill(dims, w, meta, X)["y"]
    w.w_in[qkv_cols] += g.standard_normal(w.w_in[qkv_cols].shape).astype(np.float32)
    y1 = orc.prefill(dims, w, meta, X)["y"]
    np.testing.assert_allclose(y1, y0, rtol=1e-13, atol=1e-14)
    # ... but not of the SSM weights
    w.w_x += 0.1 * g.standard_normal(w.w_x.shape).astype(np.float32)
    assert np.max(np.abs(orc.prefill(dims, w, meta, X)["y"] - y0)) > 1e-4
    # beta2 = 0: independent of W_SSM, W_G, W_x, W_dt, b_dt, A, D
    w, meta, X = _layer(dims)
    w.beta_ssm[:] = 0.0
    y0 = orc.prefill(dims, w, meta, X)["y"]
    w.w_in[ssm_cols] += g.standard_normal(w.w_in[ssm_cols].shape).astype(np.float32)
    w.w_x *= 3.0
    w.w_dt *= -2.0
    w.dt_bias += 1.0
    w.A *= 0.5
    w.D += 1.0
    np.testing.assert_allclose(orc.prefill(dims, w, meta, X)["y"], y0, rtol=1e-13, atol=1e-14)
    w.w_in[:dims.q_width] *= 1.5
    assert np.max(np.abs(orc.prefill(dims, w, meta, X)["y"] - y0)) > 1e-4


def test_fusion_reduces_to_shared_out_proj_sum():
    """With equal branch widths and W_out = [W | W] the concatenated form equals the
    summary's W_out(beta1 norm(attn) + beta2 norm(ssm)) up to the 0.5 average."""
    g = rs(13)
    T, wdt, d = 6, 10, 7
    O, Y = g.standard_normal((T, wdt)), g.standard_normal((T, wdt)) * 5
    b1, b2 = g.uniform(0.5, 2, wdt), g.uniform(0.5, 2, wdt)
    W = g.standard_normal((d, wdt))
    got = orc.out_proj(orc.fuse(O, Y, b1, b2, 1e-6), np.concatenate([W, W], axis=1))
    n = lambda v: v / np.sqrt(np.mean(v * v, axis=1, keepdims=True) + 1e-6)
    ref = 0.5 * (b1 * n(O) + b2 * n(Y)) @ W.T
    np.testing.assert_allclose(got, ref, rtol=1e-13)
    # output linear in W_out
    W2 = g.standard_normal((d, 2 * wdt))
    F = orc.fuse(O, Y, b1, b2, 1e-6)
    np.testing.assert_allclose(orc.out_proj(F, 2 * W2 - W2), orc.out_proj(F, W2), rtol=1e-13)


def test_meta_rows_are_batch_invariant():
    dims = tiny_dims(window=5)
    w, meta, X = _layer(dims, B=3, L=7)
    out = orc.prefill(dims, w, meta, X, keep=True)
    M = dims.n_meta
    for b in range(1, 3):
        np.testing.assert_array_equal(out["y_meta"][b], out["y_meta"][0])
        np.testing.assert_array_equal(out["K"][b, :M], out["K"][0, :M])
        np.testing.assert_array_equal(out["V"][b, :M], out["V"][0, :M])
    # the post-meta scan state is batch-shared: scanning the meta rows alone agrees
    s0 = out["seqs"][0]
    _, hm = orc.selective_scan(s0["Xs"][:M], s0["dt"][:M], w.A, s0["B"][:M], s0["C"][:M], w.D)
    s1 = out["seqs"][1]
    _, hm1 = orc.selective_scan(s1["Xs"][:M], s1["dt"][:M], w.A, s1["B"][:M], s1["C"][:M], w.D)
    np.testing.assert_array_equal(hm, hm1)


def test_kv_share_consumer_equals_own_kv_layer():
    """A consumer fed K/V that equal what its own W_K, W_V would give equals a
    non-sharing layer with those projections."""
    prod = tiny_dims(window=4)
    w, meta, X = _layer(prod, B=2, L=8)
    full = orc.prefill(prod, w, meta, X)
    cons = prod.replace(kv_share=1)
    qw, kw = prod.q_width, prod.kv_width
    wc = gen_layer_weights(cons, 90, std=0.2)
    wc.w_in[:] = np.concatenate([w.w_in[:qw], w.w_in[qw + 2 * kw:]], axis=0)
    for name in ("w_x", "w_dt", "dt_bias", "A", "D", "w_out", "beta_attn", "beta_ssm"):
        getattr(wc, name)[...] = getattr(w, name)
    kv_src = [{"K": full["K"][b], "V": full["V"][b]} for b in range(2)]
    shared = orc.prefill(cons, wc, meta, X, kv_src=kv_src)
    np.testing.assert_allclose(shared["y"], full["y"], rtol=1e-13)
    np.testing.assert_allclose(shared["h"], full["h"], rtol=1e-13)


@pytest.mark.parametrize("window,slots,L,k", [(0, 16, 6, 5), (4, 4, 9, 6), (5, 8, 3, 7)])
def test_prefill_then_decode_equals_longer_prefill(window, slots, L, k):
    dims = tiny_dims(window=window)
    w, meta, X = _layer(dims, B=2, L=L + k, case=91)
    long = orc.prefill(dims, w, meta, X, ring_slots=slots)
    short = orc.prefill(dims, w, meta, X[:, :L], ring_slots=slots)
    st = dict(k=short["k"], v=short["v"], h=short["h"], pos=np.full(2, L))
    for s in range(k):
        out = orc.decode_step(dims, w, X[:, L + s], short["k_meta"], short["v_meta"],
                              st["k"], st["v"], st["h"], st["pos"])
        np.testing.assert_allclose(out["y"], long["y"][:, L + s], rtol=1e-11, atol=1e-12)
        st = out
    np.testing.assert_allclose(st["h"], long["h"], rtol=1e-12)
    np.testing.assert_allclose(st["k"], long["k"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(st["v"], long["v"], rtol=1e-13, atol=1e-15)
    assert np.all(st["pos"] == L + k)


def test_contract_rounding_is_small_and_applied():
    dims = tiny_dims(window=0)
    w, meta, X = _layer(dims, B=1, L=10, case=92)
    a = orc.prefill(dims, w, meta, X, keep=True)
    b = orc.prefill(dims, w, meta, X, keep=True, contract=True)
    sb = b["seqs"][0]
    for name in ("z", "O", "Yssm", "F"):
        np.testing.assert_array_equal(orc.bf16_round(sb[name]), sb[name])
    rel = np.max(np.abs(a["y"] - b["y"])) / np.max(np.abs(a["y"]))
    assert 0 < rel < 3e-2


def test_layer_matches_torch_composition_on_full_causal_case():
    """The whole layer, with attention done by torch's SDPA on repeated KV heads and
    the SSM by the alpha mixing matrix: an assembly that shares no step with the
    oracle's recurrent scan or masked softmax."""
    dims = tiny_dims(window=0, n_meta=2)
    w, meta, X = _layer(dims, B=1, L=6, case=93)
    out = orc.prefill(dims, w, meta, X, keep=True)
    s = out["seqs"][0]
    xt = torch.from_numpy(np.concatenate([meta, X[0]]).astype(np.float64))
    z = xt @ torch.from_numpy(w.w_in.astype(np.float64)).T
    qw, kw, Di = dims.q_width, dims.kv_width, dims.d_inner
    T = z.shape[0]
    q = z[:, :qw].reshape(T, 4, 8).permute(1, 0, 2)
    k = z[:, qw:qw + kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    v = z[:, qw + kw:qw + 2 * kw].reshape(T, 2, 8).permute(1, 0, 2).repeat_interleave(2, 0)
    o = TF.scaled_dot_product_attention(q, k, v, is_causal=True).permute(1, 0, 2).reshape(T, qw)
    xs = z[:, qw + 2 * kw:qw + 2 * kw + Di]
    gg = z[:, qw + 2 * kw + Di:]
    xdbl = xs @ torch.from_numpy(w.w_x.astype(np.float64)).T
    R, N = dims.dt_rank, dims.d_state
    dt = TF.softplus(xdbl[:, :R] @ torch.from_numpy(w.w_dt.astype(np.float64)).T
                     + torch.from_numpy(w.dt_bias.astype(np.float64)), threshold=1e9)
    ymix = orc.ssm_mixing_form(xs.numpy(), dt.numpy(), w.A, xdbl[:, R:R + N].numpy(),
                               xdbl[:, R + N:].numpy(), w.D)
    yssm = torch.from_numpy(ymix) * TF.silu(gg)
    fa = TF.rms_norm(o, (qw,), eps=1e-6) * torch.from_numpy(w.beta_attn.astype(np.float64))
    fs = TF.rms_norm(yssm, (Di,), eps=1e-6) * torch.from_numpy(w.beta_ssm.astype(np.float64))
    Y = 0.5 * torch.cat([fa, fs], 1) @ torch.from_numpy(w.w_out.astype(np.float64)).T
    np.testing.assert_allclose(out["y"][0], Y[dims.n_meta:].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["y_meta"][0], Y[:dims.n_meta].numpy(), rtol=1e-10, atol=1e-12)
