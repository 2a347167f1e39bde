"""Plain, slow CPU oracle of the Hymba fused hybrid-head layer forward (numpy, fp64).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the GPU library.  It shares no code with the GPU path.

Sources (web pages on Hymba; cited by title and section):
  [HYMBA-SUM]  "Hymba: A Hybrid-head Architecture for Small Language Models",
               reader's summary (blog.outta.ai), section "A Fused Hybrid Head
               Module / Design formulation": the meta-token prefix equation, the
               five-way in_proj split, the attention-head equation, the SSM mixing
               coefficient alpha_{i,j}, the gated SSM-head equation and the total
               fusion equation.  Sections "Meta Tokens", "Combine global and local
               attention" and "Cross-layer KV sharing" for the mask and the cache.
  [HYMBA-ABS]  the same title, paper abstract (chatpaper.ai): meta tokens prepended
               to the prompt, cross-layer KV sharing, partial sliding-window attention.
  [HYB]        Korean summary of a study of hybrid Transformer-Mamba architectures
               (inter- and intra-layer), section "설계 통찰 / 아키텍처 변형": group
               normalisation and difference / concatenation fusion for intra-layer hybrids.
  [HYMBA-ZH]   Chinese summary "Hymba ... hybrid attention-SSM heads"
               (metaphor-xennon.pages.dev), sections "核心架构" (normalise then average
               the two branches) and "实现细节" (RMSNorm per branch, 0.5 average,
               bias-free projections, meta rows stripped from the output).

What it computes, per sequence b (positions p = 0..T~-1 of X~ = [meta; X_b], meta
first; [HYMBA-SUM] Design formulation):
  Z = X~ W_in^T split by columns into [Q | K | V | Xs | G]   (a KV-sharing consumer
      has no K, V columns and takes K/V from its producer)
  attention per q head h, kv group g = floor(h*Hkv/Hq):
      S_ij = s <Q_i,h, K_j,g>, key j visible to query i iff j <= i and
      (j < M or window == 0 or i - j < window);  O = softmax(S) V
  SSM (Mamba selective scan, diagonal A per channel):
      [delta | B | C] = Xs W_x^T ;  dt = softplus(delta W_dt^T + b_dt)
      h_t = exp(dt_t * A) * h_{t-1} + (dt_t * x_t) B_t ;  y_t = h_t C_t + D * x_t
      Y_ssm = y * SiLU(G)
  F = 0.5 [ beta1 * rms(O) ; beta2 * rms(Y_ssm) ],  rms(v) = v / sqrt(mean(v^2) + eps)
  Y = F W_out^T ;  y = Y[M:], y_meta = Y[:M]

SSM head variant (dims.ssm_heads = H > 0; [HYMBA-ZH] 实现细节, where the layer's SSM head is
a Mamba-2 head built with a number of heads; its internals are not printed).  Reading:
the standard Mamba-2 head with one group: the Di channels form H heads of P = Di / H
channels; x_proj gives [u | B | C] with one u per head, dt = softplus(u + b_dt[h]) is
shared by the head's channels, A is one negative scalar per head, B and C are shared by
all heads; D per channel; no convolution or internal norm (the branch norm follows):
      h_t[c,n] = exp(dt_t[h] A[h]) h_{t-1}[c,n] + dt_t[h] x_t[c] B_t[n],  c in head h
      y_t[c]   = sum_n C_t[n] h_t[c,n] + D[c] x_t[c]
It is the selective scan above with dt and A constant across a head's channels and
states.

Fusion variant (dims.norm_group = g > 0; [HYB] "Hybrid architectures ... design
insights": group normalisation in the intra-layer hybrid, with difference or
concatenation fusion): each branch is normalised in groups of g consecutive channels,
(v - mean) / sqrt(var + eps) per group, then scaled by its beta and averaged as above.
Concatenation is the default fusion; a difference fusion through the concatenated W_out
is the same map with the SSM half of W_out negated, so it needs no code of its own.

Readings where the pages are silent or disagree (each one also listed in the design
notes): softmax scale 1/sqrt(dh); no positional encoding; causal mask; a window of W
keys counts the query itself; contiguous GQA groups; no short convolution before the
scan; dt rank R and the x_proj/dt_proj factorisation of dt, B, C follow Mamba; h = 0
before the first meta token; RMSNorm over each branch's full width; the two branches
of unequal width are concatenated and projected by one W_out (equal to averaging the
two projected branches); only dt_proj has a bias.

`contract=True` rounds to bf16 (round-to-nearest-even) where the bf16 GPU path
rounds to bf16: Z, delta, O, Y_ssm and F.  Everything else stays fp64.  (The GPU's
bf16 prefill rounds beta * O and beta * Y_ssm in place of F and applies the two
per-row norm factors in fp32 inside out_proj: one rounding of a different product, well
inside the bf16 parity tolerance.)

Parity pins: every function here is pinned by tests that do not retype it (closed
forms, brute force, library special cases, invariants).  The conventions above that
no page value fixes (meta rows across layers, layer wiring, dt rank, no convolution,
norm type, concatenated fusion) are "parity unpinned" beyond self-consistency.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_round", "softplus", "silu", "rms_normalize", "in_proj", "split_z",
    "attention", "ssm_params", "selective_scan", "ssm_alpha", "ssm_mixing_form",
    "gate", "fuse", "out_proj", "prefill_sequence", "prefill", "decode_step",
    "visible", "ssm2_params", "ssm2_scan", "ssd_matrix_form", "group_normalize",
    "rms_norm_weighted", "ffn", "block_prefill", "block_decode_step",
]


# ---------------------------------------------------------------------------
# elementwise helpers
# ---------------------------------------------------------------------------

def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.

    Written from the format's definition: a = m * 2^e with 0.5 <= |m| < 1, keep
    round(m * 2^8) / 2^8.  numpy's rint rounds halves to even.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def softplus(z):
    """log(1 + e^z), without a large-z cutoff (stable form log(e^0 + e^z))."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def silu(z):
    """z * sigmoid(z): the output gate nonlinearity."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def rms_normalize(v, eps: float):
    """Per row (last axis): v / sqrt(mean(v^2) + eps).  [HYMBA-ZH] 实现细节: RMSNorm per branch."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def group_normalize(v, group: int, eps: float):
    """Group normalisation of each row (last axis) in consecutive groups of `group`
    channels: (v - mean_g) / sqrt(var_g + eps), the variance taken about the group mean
    ([HYB] design insights: group normalisation in the intra-layer hybrid; reading: no
    affine term of its own, the branch's beta scales afterwards)."""
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    g = v.reshape(shp[:-1] + (shp[-1] // group, group))
    mu = g.mean(axis=-1, keepdims=True)
    var = ((g - mu) ** 2).mean(axis=-1, keepdims=True)
    return ((g - mu) / np.sqrt(var + eps)).reshape(shp)


# ---------------------------------------------------------------------------
# the layer's steps
# ---------------------------------------------------------------------------

def in_proj(xt, w_in):
    """Z = X~ W_in^T.  [HYMBA-SUM] Design formulation: one input projection over the
    meta-prefixed rows, W_in = [W_Q, W_K, W_V, W_SSM, W_G]."""
    return np.asarray(xt, np.float64) @ np.asarray(w_in, np.float64).T


def split_z(z, dims) -> Dict[str, np.ndarray]:
    """Split Z's columns in the order [Q | K | V | Xs | G]; heads are contiguous
    head_dim blocks inside Q, K and V.  A KV-sharing consumer has no K, V blocks."""
    T = z.shape[0]
    qw, kw, Di = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim, dims.d_inner
    c = 0
    out = {"Q": z[:, c:c + qw].reshape(T, dims.n_q_heads, dims.head_dim)}
    c += qw
    if not dims.kv_share:
        out["K"] = z[:, c:c + kw].reshape(T, dims.n_kv_heads, dims.head_dim)
        c += kw
        out["V"] = z[:, c:c + kw].reshape(T, dims.n_kv_heads, dims.head_dim)
        c += kw
    out["Xs"] = z[:, c:c + Di]
    c += Di
    out["G"] = z[:, c:c + Di]
    c += Di
    assert c == z.shape[1]
    return out


def visible(qpos, kpos, n_meta: int, window: int):
    """Mask of keys visible to queries, positions in X~ coordinates (meta first).

    Causal; meta keys are always visible to later queries ([HYMBA-SUM] Meta Tokens:
    meta tokens act as attention backstops); with window > 0 a non-meta key is
    visible iff fewer than `window` positions back, counting the query itself
    ([HYMBA-SUM] Combine global and local attention)."""
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    ok = kpos <= qpos
    if window > 0:
        ok &= (kpos < n_meta) | (qpos - kpos < window)
    return ok


def attention(Q, K, V, qpos, kpos, n_meta: int, window: int, scale: float,
              return_probs: bool = False, q_block: int = 2048):
    """Softmax attention with grouped KV heads.

    Q [Tq, Hq, dh], K/V [Tk, Hkv, dh]; q head h reads kv head floor(h*Hkv/Hq).
    O_i = sum_j P_ij V_j with P_i = softmax_j(scale * <Q_i, K_j>) over visible j.
    [HYMBA-SUM] Design formulation, attention-head equation (an input-dependent
    mixing matrix over tokens); GQA from [HYMBA-ZH] 跨层KV缓存共享.
    Query rows are independent, so they are processed `q_block` at a time only to
    bound memory; each block scores only the keys that the visibility rule can admit
    for some query of the block (meta keys and keys inside the block's causal/window
    span).  Every excluded key is masked for every query of the block, so its softmax
    weight is exactly zero either way: the result is the same definition.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Tq, Hq, dh = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((Tq, Hq, V.shape[2]))
    probs = np.zeros((Hq, Tq, K.shape[0])) if return_probs else None
    qpos = np.asarray(qpos)
    kpos = np.asarray(kpos)
    for q0 in range(0, Tq, q_block):
        q1 = min(Tq, q0 + q_block)
        block_vis = visible(qpos[q0:q1], kpos, n_meta, window).any(axis=0)
        keys = np.nonzero(block_vis)[0]
        mask = visible(qpos[q0:q1], kpos[keys], n_meta, window)
        for h in range(Hq):
            g = (h * Hkv) // Hq
            S = scale * (Q[q0:q1, h, :] @ K[keys, g, :].T)
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            P /= P.sum(axis=1, keepdims=True)
            O[q0:q1, h, :] = P @ V[keys, g, :]
            if return_probs:
                probs[h, q0:q1][:, keys] = P
    if return_probs:
        return O, probs
    return O


def ssm_params(xs, w_x, w_dt, dt_bias, dt_rank: int, d_state: int, contract: bool = False):
    """[delta | B | C] = Xs W_x^T and dt = softplus(delta W_dt^T + b_dt).

    dt, B, C are linear in the SSM input (Mamba's selective parameters, reading of
    [HYMBA-SUM] Design formulation, where the SSM head is Mamba)."""
    xdbl = np.asarray(xs, np.float64) @ np.asarray(w_x, np.float64).T
    delta = xdbl[:, :dt_rank]
    B = xdbl[:, dt_rank:dt_rank + d_state]
    C = xdbl[:, dt_rank + d_state:dt_rank + 2 * d_state]
    if contract:
        delta = bf16_round(delta)
    dt = softplus(delta @ np.asarray(w_dt, np.float64).T + np.asarray(dt_bias, np.float64))
    return dt, B, C


def selective_scan(x, dt, A, B, C, D, h0=None):
    """Recurrent form of the selective SSM, one step per token.

    h_t = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] x_t[c] B_t[n]
    y_t[c] = sum_n C_t[n] h_t[c,n] + D[c] x_t[c]
    x, dt [T, Di]; B, C [T, N]; A [Di, N]; D [Di]; h0 [Di, N] or None (zero).
    Returns (y [T, Di], h_T [Di, N])."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    D = np.asarray(D, np.float64)
    T, Di = x.shape
    h = np.zeros(A.shape) if h0 is None else np.array(h0, np.float64)
    y = np.empty((T, Di))
    for t in range(T):
        h = np.exp(dt[t][:, None] * A) * h + (dt[t] * x[t])[:, None] * B[t][None, :]
        y[t] = h @ C[t] + D * x[t]
    return y, h


def ssm2_params(xs, w_x, dt_bias, n_heads: int, d_state: int):
    """Mamba-2 head: [u | B | C] = Xs W_x^T and dt = softplus(u + b_dt), one dt per
    head (reading of [HYMBA-ZH] 实现细节, see the module docstring).  Returns dt [T, H],
    B, C [T, N]."""
    xbc = np.asarray(xs, np.float64) @ np.asarray(w_x, np.float64).T
    u = xbc[:, :n_heads]
    B = xbc[:, n_heads:n_heads + d_state]
    C = xbc[:, n_heads + d_state:n_heads + 2 * d_state]
    dt = softplus(u + np.asarray(dt_bias, np.float64)[None, :])
    return dt, B, C


def ssm2_scan(x, dt, A, B, C, D, h0=None):
    """Mamba-2 head recurrence, one step per token: head h owns channels
    [h*P, (h+1)*P), P = Di / H, and a P x N state matrix S_h:
        S_h <- exp(dt_t[h] A[h]) S_h + dt_t[h] x_t[head h] B_t^T
        y_t[head h] = S_h C_t + D[head h] * x_t[head h]
    x [T, Di]; dt [T, H]; A [H]; B, C [T, N]; D [Di]; h0 [Di, N] or None (zero).
    Returns (y [T, Di], h_T [Di, N])."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    D = np.asarray(D, np.float64)
    T, Di = x.shape
    H = A.shape[0]
    P = Di // H
    N = B.shape[1]
    S = np.zeros((H, P, N)) if h0 is None else np.array(h0, np.float64).reshape(H, P, N)
    y = np.empty((T, Di))
    for t in range(T):
        xt = x[t].reshape(H, P)
        for h in range(H):
            S[h] = np.exp(dt[t, h] * A[h]) * S[h] + dt[t, h] * np.outer(xt[h], B[t])
            y[t, h * P:(h + 1) * P] = S[h] @ C[t]
        y[t] += D * x[t]
    return y, S.reshape(Di, N)


def ssd_matrix_form(x, dt, A, B, C, D):
    """The same head as one lower-triangular matrix per head (its "dual" form):
        y_i[head h] = sum_{j <= i} exp(A[h] sum_{k=j+1..i} dt_k[h]) (C_i . B_j) dt_j[h] x_j
                      + D x_i.
    Written from the recurrence unrolled from a zero state; O(T^2) per head."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    T, Di = x.shape
    H = A.shape[0]
    P = Di // H
    y = np.asarray(D, np.float64)[None, :] * x
    for h in range(H):
        cols = slice(h * P, (h + 1) * P)
        for i in range(T):
            for j in range(i + 1):
                decay = np.exp(A[h] * dt[j + 1:i + 1, h].sum())
                y[i, cols] += decay * (C[i] @ B[j]) * dt[j, h] * x[j, cols]
    return y


def ssm_alpha(dt, A, B, C):
    """The SSM head's mixing coefficients, straight from [HYMBA-SUM] Design
    formulation: alpha_{i,j}[c] = sum_n C_i[n] (prod_{k=j+1..i} exp(A[c,n] dt_k[c]))
    B_j[n] dt_j[c] for j <= i, 0 otherwise.  Pure-Python loops: tiny inputs only."""
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    T, Di = dt.shape
    N = A.shape[1]
    alpha = np.zeros((T, T, Di))
    for i in range(T):
        for j in range(i + 1):
            for c in range(Di):
                s = 0.0
                for n in range(N):
                    prod = 1.0
                    for k in range(j + 1, i + 1):
                        prod *= np.exp(A[c, n] * dt[k, c])
                    s += C[i, n] * prod * B[j, n] * dt[j, c]
                alpha[i, j, c] = s
    return alpha


def ssm_mixing_form(x, dt, A, B, C, D):
    """y_i = sum_{j<=i} alpha_{i,j} x_j + D x_i: the SSM as an explicit mixing matrix."""
    alpha = ssm_alpha(dt, A, B, C)
    x = np.asarray(x, np.float64)
    y = np.einsum("ijc,jc->ic", alpha, x)
    return y + np.asarray(D, np.float64)[None, :] * x


def gate(y, g):
    """Y_ssm = y * SiLU(G): [HYMBA-SUM] Design formulation, the gate G passes the SSM
    output selectively."""
    return np.asarray(y, np.float64) * silu(g)


def fuse(O, Yssm, beta_attn, beta_ssm, eps: float, norm_group: int = 0):
    """F = 0.5 [beta1 * rms(O) ; beta2 * rms(Y_ssm)].

    [HYMBA-SUM] Design formulation, total fusion equation: each branch normalised
    and rescaled by a learnable vector; [HYMBA-ZH] 核心架构/实现细节: the two are
    averaged.  The branches differ in width, so they are concatenated; projecting
    F with W_out = [W_a | W_s] equals averaging W_a(beta1 rms(O)) and W_s(beta2 rms(Y))."""
    if norm_group:  # the group-normalisation variant of the fusion
        a = np.asarray(beta_attn, np.float64) * group_normalize(O, norm_group, eps)
        s = np.asarray(beta_ssm, np.float64) * group_normalize(Yssm, norm_group, eps)
    else:
        a = np.asarray(beta_attn, np.float64) * rms_normalize(O, eps)
        s = np.asarray(beta_ssm, np.float64) * rms_normalize(Yssm, eps)
    return 0.5 * np.concatenate([a, s], axis=-1)


def out_proj(F, w_out):
    """Y = F W_out^T ([HYMBA-SUM] total fusion equation; bias-free per [HYMBA-ZH])."""
    return np.asarray(F, np.float64) @ np.asarray(w_out, np.float64).T


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def _rnd(a, contract):
    return bf16_round(a) if contract else a


def _ssm_branch(dims, w, xs, h0, contract):
    """dt, B, C and the scan for the layer's SSM head type (ssm_heads = 0: Mamba,
    > 0: Mamba-2 head)."""
    if getattr(dims, "ssm_heads", 0):
        dt, B, C = ssm2_params(xs, w.w_x, w.dt_bias, dims.ssm_heads, dims.d_state)
        y, h = ssm2_scan(xs, dt, w.A, B, C, w.D, h0=h0)
    else:
        dt, B, C = ssm_params(xs, w.w_x, w.w_dt, w.dt_bias, dims.dt_rank, dims.d_state,
                              contract)
        y, h = selective_scan(xs, dt, w.A, B, C, w.D, h0=h0)
    return dt, B, C, y, h


def prefill_sequence(dims, w, meta, x, kv_src: Optional[Dict[str, np.ndarray]] = None,
                     contract: bool = False, keep: bool = False):
    """One sequence through the layer.  meta [M, d], x [L, d].

    kv_src (consumer only): {"K": [T~, Hkv, dh], "V": [T~, Hkv, dh]}, the producer's
    keys and values at every position of this sequence ([HYMBA-SUM] Cross-layer KV
    sharing).  Returns dict with y [L, d], y_meta [M, d], K, V [T~, Hkv, dh],
    h [Di, N] and, with keep=True, the intermediates."""
    M = dims.n_meta
    xt = np.concatenate([np.asarray(meta, np.float64), np.asarray(x, np.float64)], axis=0)
    T = xt.shape[0]
    z = _rnd(in_proj(xt, w.w_in), contract)
    parts = split_z(z, dims)
    if dims.kv_share:
        if kv_src is None:
            raise ValueError("a KV-sharing consumer needs the producer's K/V")
        K, V = np.asarray(kv_src["K"], np.float64), np.asarray(kv_src["V"], np.float64)
    else:
        K, V = parts["K"], parts["V"]
    pos = np.arange(T)
    O = attention(parts["Q"], K, V, pos, pos, M, dims.window, dims.scale)
    O = _rnd(O.reshape(T, -1), contract)
    dt, B, C, y, h = _ssm_branch(dims, w, parts["Xs"], None, contract)
    Yssm = _rnd(gate(y, parts["G"]), contract)
    F = _rnd(fuse(O, Yssm, w.beta_attn, w.beta_ssm, dims.rms_eps,
                         getattr(dims, "norm_group", 0)), contract)
    Y = out_proj(F, w.w_out)
    out = {"y": Y[M:], "y_meta": Y[:M], "K": K, "V": V, "h": h}
    if keep:
        out.update(z=z, O=O, dt=dt, B=B, C=C, y_scan=y, Yssm=Yssm, F=F, Y=Y, **parts)
    return out


def prefill(dims, w, meta, X, kv_src: Optional[Sequence[Dict[str, np.ndarray]]] = None,
            contract: bool = False, ring_slots: Optional[int] = None, keep: bool = False):
    """Batch prefill: each sequence b runs over [meta; X_b] independently.

    Returns y [B, L, d], y_meta [B, M, d] (one copy per sequence, so the batch
    invariance can be checked), per-sequence K/V [B, T~, Hkv, dh], h [B, Di, N],
    and, if ring_slots is given, the cache a producer leaves behind:
    k_meta/v_meta [Hkv, M, dh] and k/v [B, Hkv, S, dh] with X-position p stored at
    slot p mod S for the last min(L, S) positions."""
    X = np.asarray(X, np.float64)
    Bn, L, _ = X.shape
    M = dims.n_meta
    seqs = [prefill_sequence(dims, w, meta, X[b], None if kv_src is None else kv_src[b],
                             contract, keep) for b in range(Bn)]
    out = {
        "y": np.stack([s["y"] for s in seqs]),
        "y_meta": np.stack([s["y_meta"] for s in seqs]),
        "K": np.stack([s["K"] for s in seqs]),
        "V": np.stack([s["V"] for s in seqs]),
        "h": np.stack([s["h"] for s in seqs]),
        "seqs": seqs,
    }
    if ring_slots is not None and not dims.kv_share:
        S = ring_slots
        Hkv, dh = dims.n_kv_heads, dims.head_dim
        k = np.zeros((Bn, Hkv, S, dh))
        v = np.zeros((Bn, Hkv, S, dh))
        for p in range(max(0, L - S), L):
            k[:, :, p % S, :] = out["K"][:, M + p]
            v[:, :, p % S, :] = out["V"][:, M + p]
        out["k_meta"] = out["K"][0, :M].transpose(1, 0, 2).copy()
        out["v_meta"] = out["V"][0, :M].transpose(1, 0, 2).copy()
        out["k"], out["v"] = k, v
    return out


def decode_step(dims, w, x_new, k_meta, v_meta, k_ring, v_ring, h, pos,
                contract: bool = False):
    """One new token per sequence, at X-position pos[b] (X~ position M + pos[b]).

    Steps as in prefill, on one row.  The producer writes its K/V at ring slot
    pos mod S before attending; attention covers the M meta entries and the
    min(pos+1, window) most recent positions held in the ring (all pos+1 with
    window = 0).  One SSM step from the stored h; pos += 1.  k_ring/v_ring and h are
    updated in place on copies that are returned.
    ([HYMBA-SUM] Introduction: attention keeps a KV cache, the SSM a recurrent state;
    Meta Tokens: meta entries are a fixed, precomputable cache prefix.)"""
    x_new = np.asarray(x_new, np.float64)
    k_ring = np.array(k_ring, np.float64)
    v_ring = np.array(v_ring, np.float64)
    h = np.array(h, np.float64)
    pos = np.array(pos, np.int64)
    Bn = x_new.shape[0]
    M, S = dims.n_meta, k_ring.shape[2]
    y = np.zeros((Bn, dims.d_model))
    for b in range(Bn):
        p = int(pos[b])
        z = _rnd(in_proj(x_new[b:b + 1], w.w_in), contract)
        parts = split_z(z, dims)
        if not dims.kv_share:
            k_ring[b, :, p % S, :] = parts["K"][0]
            v_ring[b, :, p % S, :] = parts["V"][0]
        span = p + 1 if dims.window <= 0 else min(p + 1, dims.window)
        if span > S:
            raise ValueError("ring too small for the attended span")
        ring_pos = np.arange(p + 1 - span, p + 1)
        K = np.concatenate([np.asarray(k_meta, np.float64).transpose(1, 0, 2),
                            k_ring[b][:, ring_pos % S, :].transpose(1, 0, 2)], axis=0)
        V = np.concatenate([np.asarray(v_meta, np.float64).transpose(1, 0, 2),
                            v_ring[b][:, ring_pos % S, :].transpose(1, 0, 2)], axis=0)
        kpos = np.concatenate([np.arange(M), M + ring_pos])
        O = attention(parts["Q"], K, V, np.array([M + p]), kpos, M, dims.window, dims.scale)
        O = _rnd(O.reshape(1, -1), contract)
        _, _, _, ys, h[b] = _ssm_branch(dims, w, parts["Xs"], h[b], contract)
        Yssm = _rnd(gate(ys, parts["G"]), contract)
        F = _rnd(fuse(O, Yssm, w.beta_attn, w.beta_ssm, dims.rms_eps,
                         getattr(dims, "norm_group", 0)), contract)
        y[b] = out_proj(F, w.w_out)[0]
        pos[b] = p + 1
    return {"y": y, "k": k_ring, "v": v_ring, "h": h, "pos": pos}


# ---------------------------------------------------------------------------
# block wrapper (pre-norm, residual, FFN)
# ---------------------------------------------------------------------------
# [HYMBA-ZH] 实现细节 prints the layer's configuration with an FFN intermediate size; the
# block around the layer is otherwise not printed.  Reading: a pre-norm residual block,
#     u   = x + Layer(rms(x) * g1)                 (over every row, meta rows included)
#     out = u + FFN(rms(u) * g2),   FFN(v) = W_down SiLU(W_up v)
# with W_up [I, d], W_down [d, I], I the intermediate size, learnable RMSNorm weights
# g1, g2 [d], and SiLU, the one activation the pages use.

def rms_norm_weighted(v, g, eps: float):
    """RMSNorm of each row with a learnable weight: rms(v) * g."""
    return rms_normalize(v, eps) * np.asarray(g, np.float64)


def ffn(v, w_up, w_down):
    """FFN(v) = W_down SiLU(W_up v) per row (the block reading above)."""
    h = silu(np.asarray(v, np.float64) @ np.asarray(w_up, np.float64).T)
    return h @ np.asarray(w_down, np.float64).T


def _ffn_rows(u, bw, eps, contract):
    vn = _rnd(rms_norm_weighted(u, bw.norm2, eps), contract)
    h = _rnd(silu(vn @ np.asarray(bw.w_up, np.float64).T), contract)
    return u + h @ np.asarray(bw.w_down, np.float64).T


def block_prefill(dims, w, bw, meta, X, contract: bool = False,
                  ring_slots: Optional[int] = None):
    """The block over [meta; X_b] for every sequence b.  bw: norm1, norm2 [d], w_up
    [I, d], w_down [d, I].  Returns y [B, L, d], y_meta [B, M, d], and the layer's cache
    and state outputs (as prefill)."""
    eps = dims.rms_eps
    meta = np.asarray(meta, np.float64)
    X = np.asarray(X, np.float64)
    mn = _rnd(rms_norm_weighted(meta, bw.norm1, eps), contract)
    xn = _rnd(rms_norm_weighted(X, bw.norm1, eps), contract)
    out = prefill(dims, w, mn, xn, contract=contract, ring_slots=ring_slots)
    u = _rnd(X + _rnd(out["y"], contract), contract)
    um = _rnd(meta[None] + _rnd(out["y_meta"], contract), contract)
    out["y"] = _ffn_rows(u, bw, eps, contract)
    out["y_meta"] = _ffn_rows(um, bw, eps, contract)
    return out


def block_decode_step(dims, w, bw, x_new, k_meta, v_meta, k_ring, v_ring, h, pos,
                      contract: bool = False):
    """One block step per sequence: the layer's decode step on rms(x_new) * g1, then the
    residual, the FFN and its residual (as block_prefill)."""
    eps = dims.rms_eps
    x_new = np.asarray(x_new, np.float64)
    xn = _rnd(rms_norm_weighted(x_new, bw.norm1, eps), contract)
    out = decode_step(dims, w, xn, k_meta, v_meta, k_ring, v_ring, h, pos, contract=contract)
    u = _rnd(x_new + _rnd(out["y"], contract), contract)
    out["y"] = _ffn_rows(u, bw, eps, contract)
    return out

