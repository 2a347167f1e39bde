"""hymba_layer_decode_static (the decode entry point that allocates nothing and keeps its
scratch in a static device array) against hymba_layer_decode with a caller's workspace:
the same state, the same inputs, through the C ABI, on two calls in a row, the second
with a smaller batch.  Both run the same kernels on the same data layout, so every output
is compared element for element and must be identical."""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_proj_amd as hy
from synth import gen_activations, gen_decode_inputs, gen_layer_weights
from tests.gpu_util import DEV, alloc_kv, alloc_state, kv_struct, make_layer, state_struct
from tests.test_gpu_parity import small_dims

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    a, b = a.detach().cpu(), b.detach().cpu()
    assert a.shape == b.shape, what
    assert torch.equal(a, b), (what, float((a.float() - b.float()).abs().max()))


@pytest.mark.parametrize("window", [0, 48])
def test_decode_static_matches_decode(window):
    dims = small_dims(dt_rank=64, window=window)
    B, L, S = 6, 70, 64
    w = gen_layer_weights(dims, 91)
    meta_t, _, x_t, _ = gen_activations(dims, 91, B, L)
    layer = make_layer(dims, w)
    kv = alloc_kv(dims, B, S)
    st = alloc_state(dims, B)
    print(f"decode_static window={window}: prefill B={B} L={L}", flush=True)
    layer.prefill(meta_t.to(DEV), x_t.to(DEV), kv_out=kv_struct(kv), state_out=state_struct(st))
    torch.cuda.synchronize()
    kv_a = {k: v.clone() for k, v in kv.items()}
    st_a = {k: v.clone() for k, v in st.items()}
    kv_b = {k: v.clone() for k, v in kv.items()}
    st_b = {k: v.clone() for k, v in st.items()}
    for step, nb in enumerate((B, 3)):
        xt, _ = gen_decode_inputs(dims, 91, nb, step)
        x = xt.to(DEV)
        sub = lambda d: {k: (v[:nb] if k in ("k", "v", "h", "pos") else v) for k, v in d.items()}
        ka, sa, kb, sb = sub(kv_a), sub(st_a), sub(kv_b), sub(st_b)
        ya = torch.empty(nb, dims.d_model, dtype=torch.bfloat16, device=DEV)
        yb = torch.full_like(ya, float("nan"))
        ws_n = hy.hymba_layer_workspace_bytes(layer.desc, nb, S, 1)
        ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
        print(f"  step {step}: batch {nb}, workspace path", flush=True)
        hy.hymba_layer_decode(layer.desc, layer.weights, x, nb, kv_struct(ka), state_struct(sa),
                              ya, ws, ws_n)
        print(f"  step {step}: batch {nb}, static scratch path", flush=True)
        hy.hymba_layer_decode_static(layer.desc, layer.weights, x, nb, kv_struct(kb),
                                     state_struct(sb), yb)
        torch.cuda.synchronize()
        _same(ya, yb, f"y step {step}")
        _same(sa["h"], sb["h"], f"h step {step}")
        _same(sa["pos"], sb["pos"], f"pos step {step}")
        _same(ka["k"], kb["k"], f"ring k step {step}")
        _same(ka["v"], kb["v"], f"ring v step {step}")
        assert np.all(np.isfinite(yb.float().cpu().numpy()))
    # sequences beyond the second call's batch were not touched by it
    _same(st_a["h"][3:], st_b["h"][3:], "untouched h")
