"""Host-side checks of libhymba that need no GPU: the library loads, exports every
symbol include/hymba.h declares, sizes workspaces, and rejects invalid arguments
before anything is launched (error paths return before any HIP call)."""
import ctypes
import os
import re

import pytest

import hybrid_attention_ssm_proj_amd as hy
from synth import CASES, LayerDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "hymba.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hymba_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hy.LIB_PATH):
        pytest.skip("libhymba.so is not built")
    return hy.load_library()


def test_header_declares_the_abi():
    names = header_functions()
    for n in ("hymba_layer_prefill", "hymba_layer_decode", "hymba_layer_workspace_bytes",
              "hymba_op_gemm", "hymba_timer_read"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert hy.hymba_abi_version() == 3
    assert hy.hymba_status_str(0) == "ok"
    assert hy.hymba_status_str(3).startswith("workspace")


def desc_of(k=1, **kw):
    return hy.LayerDesc.from_dims(CASES[k].dims.replace(**kw))


def test_workspace_sizes(lib):
    d = desc_of(1)
    rows = 128 + 8 * 2048
    n_in = 16 * 128 + 2 * 4 * 128 + 2 * 4096
    got = hy.hymba_layer_workspace_bytes(d, 8, 2048, 0)
    # Z, delta (bf16), B|C (fp32), F (bf16); this shape computes dt inside the scan;
    # plus V^T staging for attention: B x Hkv x head_dim x (keys rounded up to 64), bf16
    vt = 8 * 4 * 128 * ((128 + 2048 + 63) // 64 * 64) * 2
    # fp32 partials of the meta-row out_proj: K = 6144 in 8 slices (32 column tiles of 64
    # want 8 workgroups each to fill 256 CUs), one [128, 2048] block per slice
    macc = 8 * 128 * 2048 * 4
    # per-row partial sums of squares (16 heads + 64 scan channel blocks) and the two
    # row factors of the branch norms, all fp32
    ss = rows * (16 + 64) * 4 + rows * 2 * 4
    # the SSM state after the meta rows ([Di, N] fp32), scanned once per call; 8 sequences
    # of 64 channel blocks are 512 workgroups, two per CU, so the sequences' scan runs in
    # one time chunk; the 128 meta rows alone run in 8 chunks of 16 tokens, whose first 7
    # leave a state summary ([Di, N]) and a dt sum ([Di]) each
    hmeta = 4096 * 16 * 4
    msum = 7 * (4096 * 16 * 4 + 4096 * 4)
    floor = rows * (n_in * 2 + 128 * 2 + 32 * 4 + 6144 * 2) + vt + macc + ss + hmeta + msum
    assert floor <= got <= floor + 10 * 256
    # fp32 layers keep a separate fp32 dt buffer
    d0 = desc_of(0)
    rows0 = 8 + 64
    floor0 = rows0 * 4 * (4 * 32 + 2 * 2 * 32 + 2 * 256 + 8 + 32 + 256 + 128 + 256)
    got0 = hy.hymba_layer_workspace_bytes(d0, 1, 64, 0)
    assert floor0 <= got0 <= floor0 + 8 * 256
    assert hy.hymba_layer_workspace_bytes(d, 128, 1024, 1) > 0
    assert hy.hymba_layer_workspace_bytes(d, -1, 10, 0) == 0
    assert hy.hymba_layer_workspace_bytes(d, 1, 10, 7) == 0
    bad = desc_of(1, d_state=24)
    assert hy.hymba_layer_workspace_bytes(bad, 1, 10, 0) == 0


def test_scan_chunk_workspace(lib):
    """The chunk-carried scan's summaries: (chunks - 1) x [Di, N] states and [Di] sums of
    dt per sequence, sized for the larger of the meta launch and the sequence launch."""
    # B = 1, L = 32768, N = 128: 64 channel blocks -> 32 chunks of 1024 (2048 workgroups)
    base = hy.hymba_layer_workspace_bytes(desc_of(3), 1, 32768, 0)
    assert base > 0
    one = hy.hymba_layer_workspace_bytes(desc_of(3, scan_chunk=32768), 1, 32768, 0)
    assert base - one == 31 * 4096 * 128 * 4 + 31 * 4096 * 4
    # a caller's chunk: 2048 tokens -> 16 chunks, 15 summaries
    c16 = hy.hymba_layer_workspace_bytes(desc_of(3, scan_chunk=2048), 1, 32768, 0)
    assert c16 - one == 15 * 4096 * 128 * 4 + 15 * 4096 * 4
    # not a multiple of 16; negative
    assert hy.hymba_layer_workspace_bytes(desc_of(3, scan_chunk=24), 1, 32768, 0) == 0
    assert hy.hymba_layer_workspace_bytes(desc_of(3, scan_chunk=-16), 1, 32768, 0) == 0


def _weights_struct(addr=4096):
    return hy.LayerWeights(*[addr + 256 * i for i in range(9)])


@pytest.mark.parametrize("change,status", [
    (dict(n_kv_heads=3), 1),          # Hq % Hkv != 0
    (dict(head_dim=96), 2),           # no kernel for this head_dim
    (dict(d_state=24), 2),            # state size not a power of two
    (dict(d_state=256), 2),           # beyond the prefill scan's LDS budget
    (dict(d_model=100), 2),           # not a multiple of 8
    (dict(window=-1), 1),
    (dict(kv_share=2), 1),
    (dict(rms_eps=float("nan")), 1),
    (dict(ssm_heads=-1), 1),
    (dict(ssm_heads=32), 2),          # Mamba-2 heads of 128 channels: no kernel
    (dict(ssm_heads=62), 2),          # 4096 / 62 is not a whole head
    (dict(ssm_heads=64, d_state=8), 2),
    (dict(ssm_heads=64, dtype="f32"), 2),
    (dict(dt_rank=0), 1),             # the Mamba head needs a dt rank
    (dict(norm_group=-1), 1),
    (dict(norm_group=24), 2),         # group size not a power of two
    (dict(norm_group=1024), 2),       # wider than one wave's 512 channels
    (dict(norm_group=4), 2),
    (dict(scan_chunk=-16), 1),
    (dict(scan_chunk=40), 2),         # time chunks are whole steps of 16 tokens
])
def test_prefill_rejects_bad_descriptors(lib, change, status):
    d = desc_of(1, **change)
    st = hy.hymba_layer_prefill(d, _weights_struct(), 4096, 8192, 1, 4, None, None, None, 12288,
                                None, 1 << 20, 1 << 40, stream=0, check=False)
    assert st == status


def test_head_ssm_layer_shapes(lib):
    """Mamba-2 heads: dt_rank is ignored, x_proj writes [u | B | C] in fp32 (no delta, no
    dt buffer), w_dt may be NULL, and there is no deferred norm."""
    d = desc_of(1, ssm_heads=64, dt_rank=0)
    rows = 128 + 8 * 2048
    n_in = 16 * 128 + 2 * 4 * 128 + 2 * 4096
    vt = 8 * 4 * 128 * ((128 + 2048 + 63) // 64 * 64) * 2
    macc = 8 * 128 * 2048 * 4
    floor = rows * (n_in * 2 + (64 + 32) * 4 + 6144 * 2) + vt + macc
    got = hy.hymba_layer_workspace_bytes(d, 8, 2048, 0)
    assert floor <= got <= floor + 8 * 256
    # a NULL w_dt passes the weight checks (the too-small workspace then stops the call
    # before any launch); the Mamba head rejects it
    w = hy.LayerWeights(4096, 4096, None, *([4096] * 6))
    assert hy.hymba_layer_prefill(d, w, 4096, 8192, 1, 4, None, None, None, 12288, None,
                                  1 << 20, 1000, stream=0, check=False) == 3
    assert hy.hymba_layer_prefill(desc_of(1), w, 4096, 8192, 1, 4, None, None, None, 12288,
                                  None, 1 << 20, 1000, stream=0, check=False) == 1


def test_prefill_argument_errors(lib):
    d = desc_of(1)
    w = _weights_struct()
    call = lambda **kw: hy.hymba_layer_prefill(**{**dict(
        desc=d, weights=w, meta=4096, x=8192, batch=1, seq_len=4, kv_in=None, kv_out=None,
        state_out=None, y=12288, y_meta=None, workspace=1 << 20, workspace_bytes=1 << 40,
        stream=0, check=False), **kw})
    assert call(meta=None) == 1                      # meta tokens but no meta buffer
    assert call(x=None) == 1
    assert call(batch=-1) == 1
    assert call(workspace_bytes=1000) == 3           # too small
    assert call(workspace=None) == 3
    assert call(x=8192 + 2) == 4                     # misaligned
    assert call(weights=hy.LayerWeights(*([4096] * 8 + [None]))) == 1
    # a producer must not be given a producer's cache
    assert call(kv_in=hy.KV(4096, 4096, 4096, 4096, 16)) == 1
    # a consumer needs one holding every position
    dc = desc_of(1, kv_share=1)
    assert call(desc=dc) == 1
    assert call(desc=dc, kv_in=hy.KV(4096, 4096, 4096, 4096, 3)) == 1
    assert call(desc=dc, kv_in=hy.KV(4096, 4096, 4096, 4096, 4),
                kv_out=hy.KV(4096, 4096, 4096, 4096, 4)) == 1
    assert call(kv_out=hy.KV(4096, 4096, 4096, None, 4)) == 1
    assert call(state_out=hy.SSMState(None, None)) == 1
    # more than 65 time chunks per sequence: the carry scan spans one wavefront
    assert call(desc=desc_of(1, scan_chunk=16), seq_len=2048) == 2
    assert call(desc=desc_of(1, scan_chunk=32), seq_len=2048,
                workspace_bytes=1000) == 3                            # 64 chunks: valid
    # row counts must stay below 2^31 (int32 shapes inside)
    assert call(desc=desc_of(1, n_meta=0), batch=2, seq_len=1 << 30) == 2
    assert call(desc=desc_of(1, n_meta=0), batch=1, seq_len=(1 << 31) - 1,
                workspace_bytes=1000) == 3
    # nothing to do: zero rows is a successful no-op that launches nothing
    assert hy.hymba_layer_prefill(desc_of(1, n_meta=0), w, None, None, 0, 0, None, None, None,
                                  None, None, None, 0, stream=0, check=False) == 0


def test_decode_argument_errors(lib):
    d = desc_of(4)
    w = _weights_struct()
    kv = hy.KV(4096, 4096, 4096, 4096, 1024)
    state = hy.SSMState(4096, 4096)
    call = lambda **kw: hy.hymba_layer_decode(**{**dict(
        desc=d, weights=w, x=4096, batch=2, kv=kv, state=state, y=4096, workspace=4096,
        workspace_bytes=1 << 40, stream=0, check=False), **kw})
    assert call(kv=None) == 1
    assert call(state=None) == 1
    assert call(kv=hy.KV(4096, 4096, 4096, 4096, 512)) == 1   # ring shorter than the window
    assert call(state=hy.SSMState(4096, None)) == 1
    assert call(workspace_bytes=16) == 3
    assert call(y=4100) == 4
    assert call(batch=0) == 0


def test_decode_static_rejects_before_any_launch(lib):
    """The static-scratch decode: a batch whose workspace exceeds the fixed array is
    refused with HYMBA_ERR_WORKSPACE, bad arguments with HYMBA_ERR_INVALID_ARG, before
    the device is touched."""
    d = desc_of(4)
    w = _weights_struct()
    kv = hy.KV(4096, 4096, 4096, 4096, 1024)
    state = hy.SSMState(4096, 4096)
    call = lambda **kw: hy.hymba_layer_decode_static(**{**dict(
        desc=d, weights=w, x=4096, batch=2, kv=kv, state=state, y=4096), **kw}, stream=0,
        check=False)
    big = 4096  # 4096 sequences: about 0.6 GB of decode workspace
    assert hy.hymba_layer_workspace_bytes(d, big, 1024, 1) > (64 << 20)
    assert call(batch=big) == 3
    assert 0 < hy.hymba_layer_workspace_bytes(d, 128, 1024, 1) <= (64 << 20)
    assert call(kv=None) == 1
    assert call(batch=-1) == 1
    assert call(kv=hy.KV(4096, 4096, 4096, 4096, 0)) == 1
    assert call(desc=desc_of(4, d_state=24)) == 2       # the descriptor's own error


def test_kv_ring_fill_and_ring_flag_checks(lib):
    """The ring fill and the is_ring contract are validated on the host: a non-ring
    prefill cache must hold every position, a ring fill's source must hold the copied
    positions; bad flags and sizes are refused before anything is launched."""
    bf = hy.DTYPE_BF16
    full = hy.KV(4096, 4096, 8192, 8192, 64, 0)
    ring = hy.KV(4096, 4096, 16384, 16384, 16, 1)
    fill = lambda **kw: hy.hymba_kv_ring_fill(**{**dict(
        src=full, dst=ring, batch=2, seq_len=64, n_meta=8, n_kv_heads=2, head_dim=128,
        dtype=bf), **kw}, stream=0, check=False)
    assert fill(src=hy.KV(4096, 4096, 8192, 8192, 32, 0)) == 1   # source misses positions
    assert fill(src=hy.KV(4096, 4096, 8192, 8192, 8, 1)) == 1    # a ring shorter than 16
    assert fill(dst=hy.KV(4096, 4096, 16384, 16384, 16, 0)) == 1  # non-ring dst too short
    assert fill(dst=hy.KV(4096, 4096, 16384, 16384, 16, 2)) == 1  # is_ring is 0 or 1
    assert fill(dtype=5) == 1
    assert fill(head_dim=12) == 2
    assert fill(dst=hy.KV(4096, 4096, 16390, 16384, 16, 1)) == 4
    assert fill(batch=-1) == 1
    assert fill(batch=0, n_meta=0) == 0                          # nothing to copy
    # a producer's non-ring cache must hold all L positions
    d = desc_of(1)
    call = lambda **kw: hy.hymba_layer_prefill(**{**dict(
        desc=d, weights=_weights_struct(), meta=4096, x=8192, batch=1, seq_len=64, kv_in=None,
        kv_out=None, state_out=None, y=12288, y_meta=None, workspace=1 << 20,
        workspace_bytes=1000), **kw}, stream=0, check=False)
    assert call(kv_out=hy.KV(4096, 4096, 4096, 4096, 32, 0)) == 1
    assert call(kv_out=hy.KV(4096, 4096, 4096, 4096, 32, 1)) == 3  # a ring: valid
    assert call(kv_out=hy.KV(4096, 4096, 4096, 4096, 64, 0)) == 3


def test_op_gemm_argument_errors(lib):
    call = lambda **kw: lib.hymba_op_gemm(*[{**dict(
        dtype=1, a=4096, lda=64, b=4096, ldb=64, c=4096, ldc=64, c_dtype=1, m=4, n=4, k=64,
        stream=None), **kw}[n] for n in ("dtype", "a", "lda", "b", "ldb", "c", "ldc", "c_dtype",
                                         "m", "n", "k", "stream")])
    assert call(dtype=7) == 1
    assert call(k=60, lda=60, ldb=60) == 2
    assert call(lda=32) == 1
    assert call(a=4098) == 4
    assert call(m=0) == 0
    assert lib.hymba_op_copy(4096, 8192, 17, None) == 2
    probe = lambda kind, blocks, iters, src, nbytes, out: lib.hymba_op_probe(
        kind, blocks, iters, src, nbytes, out, None)
    assert probe(4, 8, 8, None, 0, 4096) == 1
    assert probe(3, 8, 8, None, 0, 4096) == 1        # kind 3 needs its operands
    assert probe(3, 8, 8, 4096, 1 << 20, 4096) == 1  # fewer than 4 MiB of them
    assert probe(0, 0, 8, None, 0, 4096) == 1
    assert probe(0, 8, 8, None, 0, None) == 1
    assert probe(2, 0, 0, 4096, 17, 4096) == 2
    assert probe(2, 0, 0, None, 16, 4096) == 1
    assert probe(1, 8, 8, None, 0, 4100) == 4


def test_op_attn_and_op_scan_reject_bad_arguments_before_any_launch(lib):
    """Validation of the single-step entry points returns a status and launches nothing
    (every case below fails before the first HIP call, so this runs without a GPU)."""
    bf, f32 = hy.DTYPE_BF16, hy.DTYPE_F32
    p = 4096  # a 16-byte aligned stand-in address; nothing is dereferenced
    attn = lambda **kw: hy.hymba_op_attn(**{**dict(
        dtype=bf, q=p, q_ld=1024, k=p, v=p, kv_ld=256, o=p, o_ld=1024, n_meta=8, seq_len=64,
        batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=0, scale=0.0, workspace=p,
        workspace_bytes=0), **kw}, stream=0, check=False)
    assert attn(dtype=7) == 1
    assert attn(n_q_heads=6, n_kv_heads=4) == 1          # Hq % Hkv != 0
    assert attn(head_dim=96, q_ld=768, o_ld=768, kv_ld=192) == 2
    assert attn(dtype=f32, head_dim=128) == 2             # fp32 kernels: 32 or 64
    assert attn(q_ld=1000) == 1                           # stride below the heads' width
    assert attn(q=p + 8) == 4
    assert attn(q=None) == 1
    assert attn(workspace_bytes=0) == 3                   # V^T staging needed for bf16
    assert attn(seq_len=0, n_meta=0) == 0                 # nothing to do
    need = hy.hymba_op_attn_workspace_bytes(bf, 8, 64, 2, 2, 128)
    assert need == 2 * 2 * 128 * 128 * 2                  # B x Hkv x dh x keys rounded to 64
    assert hy.hymba_op_attn_workspace_bytes(f32, 8, 64, 2, 2, 64) == 0
    scan = lambda **kw: hy.hymba_op_scan(**{**dict(
        dtype=bf, z=p, z_ld=1024, xs_col=0, g_col=512, delta=p, bc=p, w_dt=p, dt_bias=p, A=p,
        D=p, y=p, y_ld=512, h_out=None, n_meta=8, seq_len=64, batch=2, d_inner=512, d_state=16,
        dt_rank=64, chunk_tokens=0, workspace=None, workspace_bytes=0), **kw}, stream=0,
        check=False)
    assert scan(dtype=3) == 1
    assert scan(d_state=24) == 2
    assert scan(g_col=600) == 1                           # G columns past the row
    assert scan(delta=None) == 1
    assert scan(y=p + 4) == 4
    assert scan(dt_rank=16) == 3                          # unfused: needs the fp32 dt buffer
    assert scan(batch=0, n_meta=0) == 0
    assert scan() == 3                                    # the post-meta state needs room
    assert scan(chunk_tokens=24) == 2
    assert scan(chunk_tokens=-16) == 1
    assert scan(n_meta=(1 << 31) - 128, seq_len=64) == 2  # rows reach 2^31
    assert attn(n_meta=(1 << 31) - 128, seq_len=64) == 2
    # bf16 chunked scan: the post-meta state [Di, N] fp32; with 512 workgroups (8
    # sequences x 64 channel blocks) the sequences run in one chunk, and so do 8 meta rows
    assert hy.hymba_op_scan_workspace_bytes(bf, 8, 2048, 8, 4096, 16, 64) == 4096 * 16 * 4
    assert hy.hymba_op_scan_workspace_bytes(bf, 0, 64, 2, 512, 16, 64, 64) == 0
    # chunks of 16 tokens: 4 per sequence, 3 summaries each ([Di, N] states + [Di] sums);
    # a short sequence on few workgroups gets the same by default
    for chunk in (16, 0):
        assert hy.hymba_op_scan_workspace_bytes(bf, 8, 64, 2, 512, 16, 64, chunk) == (
            512 * 16 * 4 + 6 * 512 * 16 * 4 + 6 * 512 * 4)
    assert hy.hymba_op_scan_workspace_bytes(bf, 8, 64, 2, 512, 16, 16) == (8 + 128) * 512 * 4


def test_block_workspace_sizes(lib):
    """Block workspace: the layer's, then xn and v ([rows, d] each), h ([rows, I]) and the
    fp32 partial slices of the few-row FFN projections, the larger of: the down-projection's
    8 slices of [few rows, d] (K = 5632 in 22 units of 256, 3 units a slice) and the
    up-projection's 3 slices of [few rows, I] (K = 2048 in 8 units, 3 units a slice)."""
    d = desc_of(1)
    rows, inter = 128 + 8 * 2048, 5632
    acc = max(8 * 2048, 3 * inter) * 128 * 4
    floor = (hy.hymba_layer_workspace_bytes(d, 8, 2048, 0) + rows * (2048 * 2 * 2 + inter * 2)
             + acc)
    got = hy.hymba_block_workspace_bytes(d, inter, 8, 2048, 0)
    assert floor <= got <= floor + 4 * 256
    d4 = desc_of(4)
    floor = (hy.hymba_layer_workspace_bytes(d4, 128, 1024, 1) + 128 * (2048 * 2 * 2 + inter * 2)
             + acc)
    got = hy.hymba_block_workspace_bytes(d4, inter, 128, 1024, 1)
    assert floor <= got <= floor + 4 * 256
    assert hy.hymba_block_workspace_bytes(d, 5630, 8, 2048, 0) == 0   # not a multiple of 8
    assert hy.hymba_block_workspace_bytes(d, 0, 8, 2048, 0) == 0
    assert hy.hymba_block_workspace_bytes(d, inter, 8, 2048, 2) == 0  # no such mode


def test_block_argument_errors(lib):
    """Every rejection happens before a launch; valid arguments with a workspace that is
    too small stop at the workspace check."""
    d = desc_of(1)
    w = _weights_struct()
    bw = hy.BlockWeights(4096, 4352, 4608, 4864, 5632)
    call = lambda **kw: hy.hymba_block_prefill(**{**dict(
        desc=d, weights=w, block=bw, meta=4096, x=8192, batch=1, seq_len=4, kv_in=None,
        kv_out=None, state_out=None, y=12288, y_meta=None, workspace=1 << 20,
        workspace_bytes=1000, stream=0, check=False), **kw})
    assert call() == 3
    assert call(block=hy.BlockWeights(4096, None, 4608, 4864, 5632)) == 1
    assert call(block=hy.BlockWeights(4096, 4352, 4608, 4864, 0)) == 1
    assert call(block=hy.BlockWeights(4096, 4352, 4608, 4864, 5630)) == 2
    assert call(block=hy.BlockWeights(4104, 4352, 4608, 4864, 5632)) == 4
    assert call(batch=-1) == 1
    assert call(x=None) == 1
    assert call(meta=None) == 1
    assert call(y=12290) == 4
    assert call(desc=desc_of(1, head_dim=96)) == 2
    assert hy.hymba_block_prefill(desc_of(1, n_meta=0), w, bw, None, None, 0, 0, None, None,
                                  None, None, None, None, 0, stream=0, check=False) == 0
    kv = hy.KV(4096, 4096, 4096, 4096, 1024)
    state = hy.SSMState(4096, 4096)
    dcall = lambda **kw: hy.hymba_block_decode(**{**dict(
        desc=desc_of(4), weights=w, block=bw, x=4096, batch=2, kv=kv, state=state, y=4096,
        workspace=4096, workspace_bytes=16, stream=0, check=False), **kw})
    assert dcall() == 3
    assert dcall(block=hy.BlockWeights(None, 4352, 4608, 4864, 5632)) == 1
    assert dcall(kv=None) == 1
    assert dcall(batch=-1) == 1
    assert dcall(x=4100) == 4
    assert dcall(batch=0) == 0
