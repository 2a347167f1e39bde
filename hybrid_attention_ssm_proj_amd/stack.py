"""A stack of hybrid-head layers with the partial sliding-window schedule and
cross-layer KV sharing, run through the C ABI one layer at a time.

Source: "Hymba: A Hybrid-head Architecture for Small Language Models" (outta.ai
summary), "Combine global and local attention" (full attention in only three layers:
the first, the middle and the last; sliding-window attention elsewhere) and "Cross-layer
KV sharing" (two consecutive layers share one KV cache).  Wiring between layers: layer
l + 1 takes layer l's y as its X and its y_meta as its meta rows (no residual, norm or
FFN between them: the block around the layer is outside this library).

Roles.  A global layer is a producer with its own full cache.  Sliding-window layers
are taken in consecutive pairs: the first of a pair is a producer, the second a
consumer (kv_share = 1, no K/V projection) that reads its producer's cache.  A
sliding-window layer left without a partner is a producer on its own.

Caches.  Decode needs, per producer, the meta entries plus: for a global layer every
position so far; for a sliding-window producer the last `window` positions (a ring of
`window` slots).  Consumers hold none.  During prefill a consumer reads every position
of its producer, so a pair runs with one full-length scratch cache (shared by all
pairs, sized for the longest prompt) and the producer's ring is filled from it
afterwards.
"""
from __future__ import annotations

from typing import List, Optional

from . import (DTYPE_BF16, DTYPE_F32, HymbaLayer, KV, SSMState, hymba_kv_ring_fill, make_kv,
               make_state)


def schedule(n_layers: int, window: int, global_layers: Optional[List[int]] = None):
    """Per layer: (window, kv_share, producer index).  window 0 = global attention."""
    if global_layers is None:
        global_layers = sorted({0, n_layers // 2, n_layers - 1}) if n_layers > 0 else []
    out = []
    i = 0
    while i < n_layers:
        if i in global_layers or window <= 0:
            out.append((0, 0, i))
            i += 1
            continue
        out.append((window, 0, i))
        if i + 1 < n_layers and (i + 1) not in global_layers:
            out.append((window, 1, i))
            i += 2
        else:
            i += 1
    return out


class HymbaStack:
    """Layers built from `dims` (the window and kv_share fields are set per layer)
    with the weights `weights_fn(layer_index, layer_dims)` returns (a dict of device
    tensors keyed as hymba_layer_weights)."""

    def __init__(self, dims, n_layers: int, weights_fn, window: int,
                 global_layers: Optional[List[int]] = None, device="cuda"):
        self.sched = schedule(n_layers, window, global_layers)
        self.layers = []
        for l, (win, share, _) in enumerate(self.sched):
            ld = dims.replace(window=win, kv_share=share)
            self.layers.append(HymbaLayer(ld, weights_fn(l, ld), device=device))
        self.device = device
        self.dims = dims
        self.caches = None
        self.states = None

    # ------------------------------------------------------------------ memory
    def cache_slots(self, l: int, context: int) -> int:
        win, share, _ = self.sched[l]
        if share:
            return 0
        return win if win > 0 else context

    def decode_cache_bytes(self, batch: int, context: int) -> int:
        """K/V bytes the stack keeps for decode at `context` positions per sequence."""
        d = self.dims
        es = 2 if d.dtype == "bf16" else 4
        per_slot = 2 * d.n_kv_heads * d.head_dim * es
        total = 0
        for l in range(len(self.layers)):
            s = self.cache_slots(l, context)
            if s:
                total += per_slot * (batch * s + d.n_meta)
        return total

    def alloc(self, batch: int, prompt: int, context: int):
        """Caches for decode up to `context` positions, SSM states, and the prefill
        scratch cache of the sliding-window pairs."""
        import torch
        d = self.dims
        dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
        z = lambda *shape: torch.zeros(*shape, dtype=dt, device=self.device)
        M = max(d.n_meta, 1)
        self.caches = []
        for l in range(len(self.layers)):
            s = self.cache_slots(l, context)
            self.caches.append(None if s == 0 else {
                "k_meta": z(d.n_kv_heads, M, d.head_dim), "v_meta": z(d.n_kv_heads, M, d.head_dim),
                "k": z(batch, d.n_kv_heads, s, d.head_dim),
                "v": z(batch, d.n_kv_heads, s, d.head_dim)})
        self.scratch = {"k": z(batch, d.n_kv_heads, prompt, d.head_dim),
                        "v": z(batch, d.n_kv_heads, prompt, d.head_dim)}
        self.states = [{"h": torch.zeros(batch, d.d_inner, d.d_state, dtype=torch.float32,
                                         device=self.device),
                        "pos": torch.zeros(batch, dtype=torch.int32, device=self.device)}
                       for _ in self.layers]

    def _kv(self, l: int) -> KV:
        c = self.caches[l]
        return make_kv(c["k_meta"], c["v_meta"], c["k"], c["v"])

    def _state(self, l: int) -> SSMState:
        return make_state(self.states[l]["h"], self.states[l]["pos"])

    # ------------------------------------------------------------------ passes
    def prefill(self, meta, x, stream=None, keep: Optional[list] = None):
        """All layers over [meta; x]; returns the last layer's (y, y_meta).  With `keep`
        (a list), every layer's (meta in, x in, y, y_meta) is appended to it."""
        B, L = x.shape[0], x.shape[1]
        for l, layer in enumerate(self.layers):
            win, share, prod = self.sched[l]
            paired = (not share and win > 0 and l + 1 < len(self.layers)
                      and self.sched[l + 1][1] == 1)
            if share:
                c = self.caches[prod]
                kv_in = make_kv(c["k_meta"], c["v_meta"], self.scratch["k"], self.scratch["v"],
                                is_ring=False)
                y, ym = layer.prefill(meta, x, kv_in=kv_in, state_out=self._state(l),
                                      stream=stream)
                self._fill_ring(prod, B, L, stream)
            elif paired:
                c = self.caches[l]
                kv_out = make_kv(c["k_meta"], c["v_meta"], self.scratch["k"], self.scratch["v"],
                                 is_ring=False)
                y, ym = layer.prefill(meta, x, kv_out=kv_out, state_out=self._state(l),
                                      stream=stream)
            else:
                y, ym = layer.prefill(meta, x, kv_out=self._kv(l), state_out=self._state(l),
                                      stream=stream)
            if keep is not None:
                keep.append((meta, x, y, ym))
            meta, x = ym, y
        return x, meta

    def _fill_ring(self, l: int, B: int, L: int, stream=None):
        """Producer l's ring of `window` slots from the scratch cache (the library's ring
        fill, on the layers' stream): position p at slot p mod window, for the last
        min(L, window) positions."""
        ring = self.caches[l]
        src = make_kv(ring["k_meta"], ring["v_meta"], self.scratch["k"], self.scratch["v"],
                      is_ring=False)
        dst = make_kv(ring["k_meta"], ring["v_meta"], ring["k"], ring["v"])
        d = self.dims
        hymba_kv_ring_fill(src, dst, B, L, d.n_meta, d.n_kv_heads, d.head_dim,
                           DTYPE_BF16 if d.dtype == "bf16" else DTYPE_F32, stream)

    def decode(self, x, stream=None):
        """One token per sequence through every layer; returns the last layer's y."""
        for l, layer in enumerate(self.layers):
            _, share, prod = self.sched[l]
            kv = self._kv(prod)
            x = layer.decode(x, kv, self._state(l), stream=stream)
        return x

    def capture_decode(self, x):
        """One decode step of the whole stack captured as a HIP graph (torch's graph
        object, a hipGraph on ROCm): every layer's kernels in order, replayed with no host
        work between them.  `x` [B, d] is the graph's input buffer: copy the next token's
        rows into it, then call replay(); the returned y is the graph's output buffer.
        The kernels take positions, ring slots and the SSM state from device memory, so
        each replay advances every layer's state as an eager decode step does.  Run one
        eager decode at this batch first: the layers' workspaces must exist before the
        capture (the library itself allocates nothing and issues no memset)."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            y = self.decode(x)
        return g, y
