"""GPU checks of the layer stack with the partial sliding-window schedule and KV-sharing
pairs (hybrid_attention_ssm_proj_amd.stack), through the C ABI.

Prefill: every layer's output against the oracle run on that layer's own inputs (the
GPU's outputs of the layer below, bf16) and, for a consumer, on the K/V the oracle's
producer computes from its own inputs; bf16 gate 2e-2.  Decode: causality fixes the
next token's output, so decode after a prefill of L tokens must give the last row of a
prefill of L + 1 tokens, through every layer (global caches, sliding-window rings,
shared K/V).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from hybrid_attention_ssm_proj_amd.stack import HymbaStack, schedule
from synth import gen_activations, gen_layer_weights
from tests.gpu_util import DEV, h_err, rel_err, to_np
from tests.test_gpu_parity import TOL_BF16, small_dims

pytestmark = pytest.mark.gpu


def _stack(dims, n_layers, window, case):
    ws = {}

    def weights(l, ld):
        ws[l] = gen_layer_weights(ld, case, layer=l)
        return {k: v for k, v in ws[l].torch.items()}
    return HymbaStack(dims, n_layers, weights, window, device=DEV), ws


def test_schedule_roles():
    assert schedule(6, 40) == [(0, 0, 0), (40, 0, 1), (40, 1, 1), (0, 0, 3), (40, 0, 4), (0, 0, 5)]
    assert schedule(8, 16) == [(0, 0, 0), (16, 0, 1), (16, 1, 1), (16, 0, 3), (0, 0, 4),
                               (16, 0, 5), (16, 1, 5), (0, 0, 7)]
    assert all(s[0] == 0 and s[1] == 0 for s in schedule(5, 0))


def test_stack_prefill_each_layer_matches_oracle():
    dims = small_dims()
    B, L, W = 2, 96, 40
    st, ws = _stack(dims, 6, W, 97)
    st.alloc(B, L, L + 4)
    meta_t, _, x_t, _ = gen_activations(dims, 97, B, L)
    keep = []
    st.prefill(meta_t.to(DEV), x_t.to(DEV), keep=keep)
    torch.cuda.synchronize()
    K = {}
    for l, (m_in, x_in, y, ym) in enumerate(keep):
        win, share, prod = st.sched[l]
        ld = st.layers[l].dims
        m_np, x_np = to_np(m_in), to_np(x_in)
        src = None
        if share:
            src = [{"K": K[prod]["K"][b], "V": K[prod]["V"][b]} for b in range(B)]
        ref = orc.prefill(ld, ws[l], m_np, x_np, kv_src=src, contract=True)
        K[l] = ref
        e_y, e_m = rel_err(to_np(y), ref["y"]), rel_err(to_np(ym), ref["y_meta"][0])
        e_h = h_err(to_np(st.states[l]["h"]), ref["h"])
        print(l, (win, share, prod), f"y {e_y:.2e} y_meta {e_m:.2e} h {e_h:.2e}")
        assert e_y < TOL_BF16 and e_m < TOL_BF16 and e_h < 1e-3, l


def test_stack_decode_continues_the_prefill():
    """decode(prefill(x[:L]), x[L + s]) == prefill(x[:L + s + 1])[L + s] for every layer
    stack role, across a sliding-window ring that wraps."""
    dims = small_dims()
    B, L, W, steps = 2, 60, 24, 3
    meta_t, _, x_t, _ = gen_activations(dims, 98, B, L + steps)
    meta, x = meta_t.to(DEV), x_t.to(DEV)
    a, _ = _stack(dims, 6, W, 98)
    a.alloc(B, L, L + steps)
    a.prefill(meta, x[:, :L].contiguous())
    outs = []
    for s in range(steps):
        outs.append(a.decode(x[:, L + s].contiguous()))
    torch.cuda.synchronize()
    b, _ = _stack(dims, 6, W, 98)
    b.alloc(B, L + steps, L + steps)
    yb, _ = b.prefill(meta, x)
    torch.cuda.synchronize()
    for s in range(steps):
        e = rel_err(to_np(outs[s]), to_np(yb[:, L + s]))
        print(f"step {s}: {e:.2e}")
        assert e < TOL_BF16, (s, e)


def _snapshot(st):
    caches = [None if c is None else {k: v.clone() for k, v in c.items()} for c in st.caches]
    states = [{k: v.clone() for k, v in s_.items()} for s_ in st.states]
    return caches, states


def _restore(st, snap):
    for c, sc in zip(st.caches, snap[0]):
        if c is not None:
            for k in c:
                c[k].copy_(sc[k])
    for s_, ss in zip(st.states, snap[1]):
        for k in s_:
            s_[k].copy_(ss[k])


def test_stack_decode_graph_replays_match_eager():
    """One decode step of a 6-layer stack (global, sliding-window producer, consumer
    roles) captured as a HIP graph and replayed 4 times, with eager work and
    synchronisations between the replays: every replay's y, and the states and caches
    after the last, equal the eager steps from the same state (the x_proj split-K
    accumulates with fp32 atomics, whose order may differ: the gate is one bf16 step)."""
    dims = small_dims()
    B, L, W, steps = 2, 60, 24, 4
    meta_t, _, x_t, _ = gen_activations(dims, 96, B, L + steps)
    meta, x = meta_t.to(DEV), x_t.to(DEV)
    st, _ = _stack(dims, 6, W, 96)
    st.alloc(B, L, L + steps)
    st.prefill(meta, x[:, :L].contiguous())
    torch.cuda.synchronize()
    snap = _snapshot(st)
    eager = [st.decode(x[:, L + s].contiguous()).clone() for s in range(steps)]
    torch.cuda.synchronize()
    after = _snapshot(st)
    _restore(st, snap)
    xs = torch.empty_like(x[:, L])
    g, ys = st.capture_decode(xs)
    for s in range(steps):
        xs.copy_(x[:, L + s])
        g.replay()
        torch.cuda.synchronize()
        junk = (x[:, :L].float() * 2).sum()  # eager work between replays
        e = rel_err(to_np(ys), to_np(eager[s]))
        print(f"replay {s}: y {e:.2e} (junk {float(junk):.1f})")
        assert e < 2 ** -7, (s, e)
    for l, (s_, sa) in enumerate(zip(st.states, after[1])):
        assert torch.equal(s_["pos"], sa["pos"]), l
        assert rel_err(to_np(s_["h"]), to_np(sa["h"])) < 1e-4, l
    for l, (c, ca) in enumerate(zip(st.caches, after[0])):
        if c is not None:
            assert rel_err(to_np(c["k"]), to_np(ca["k"])) < 2 ** -7, l
            assert rel_err(to_np(c["v"]), to_np(ca["v"])) < 2 ** -7, l


def test_cache_bytes_partial_swa_vs_all_global():
    dims = small_dims()
    st, _ = _stack(dims, 6, 40, 99)
    g, _ = _stack(dims, 6, 0, 99)
    B, ctx = 4, 1000
    per = 2 * dims.n_kv_heads * dims.head_dim * 2
    # producers: globals 0, 3, 5 keep ctx positions, sliding-window producers 1 and 4 keep 40
    assert st.decode_cache_bytes(B, ctx) == per * (3 * (B * ctx + dims.n_meta) +
                                                   2 * (B * 40 + dims.n_meta))
    assert g.decode_cache_bytes(B, ctx) == per * 6 * (B * ctx + dims.n_meta)


@pytest.mark.parametrize("L,S,M", [(100, 32, 8), (20, 32, 8), (64, 64, 0)])
def test_kv_ring_fill_matches_gather(L, S, M):
    """hymba_kv_ring_fill: the last min(L, S) positions of a full cache land at slot
    p mod S of the ring, and the meta entries are copied when the arrays differ."""
    import hybrid_attention_ssm_proj_amd as hy
    B, Hkv, dh = 3, 2, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(L + S)
    src = {"k": torch.randn(B, Hkv, L, dh, generator=g, device=DEV).to(torch.bfloat16),
           "v": torch.randn(B, Hkv, L, dh, generator=g, device=DEV).to(torch.bfloat16),
           "k_meta": torch.randn(Hkv, max(M, 1), dh, generator=g, device=DEV).to(torch.bfloat16),
           "v_meta": torch.randn(Hkv, max(M, 1), dh, generator=g, device=DEV).to(torch.bfloat16)}
    dst = {k: torch.zeros(B, Hkv, S, dh, dtype=torch.bfloat16, device=DEV) for k in ("k", "v")}
    dst.update({k: torch.zeros_like(src[k]) for k in ("k_meta", "v_meta")})
    print(f"ring fill L={L} S={S} M={M}", flush=True)
    hy.hymba_kv_ring_fill(hy.make_kv(src["k_meta"], src["v_meta"], src["k"], src["v"], False),
                          hy.make_kv(dst["k_meta"], dst["v_meta"], dst["k"], dst["v"]), B, L, M,
                          Hkv, dh, hy.DTYPE_BF16)
    torch.cuda.synchronize()
    ref = {k: torch.zeros_like(dst[k]) for k in ("k", "v")}
    for p in range(max(0, L - S), L):
        for k in ("k", "v"):
            ref[k][:, :, p % S] = src[k][:, :, p]
    for k in ("k", "v"):
        assert torch.equal(dst[k], ref[k]), k
    for k in ("k_meta", "v_meta"):
        assert torch.equal(dst[k][:, :M], src[k][:, :M]), k
