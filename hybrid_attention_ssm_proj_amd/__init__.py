"""Python binding of libhymba, the gfx950 Hymba hybrid-head layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libhymba.so; torch is used for device memory and streams.  The functions named
hymba_* mirror the C ABI in include/hymba.h one to one.  Importing this module does
not touch the GPU; the first call loads the library and raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MetaCache", "hymba_layer_meta_cache_build", "hymba_layer_prefill_cached",
    "BlockWeights", "HymbaBlock", "hymba_block_workspace_bytes", "hymba_block_prefill",
    "hymba_block_decode",
    "hymba_op_attn", "hymba_op_attn_workspace_bytes", "hymba_op_scan",
    "hymba_op_scan_workspace_bytes",
    "HymbaError", "LayerDesc", "LayerWeights", "KV", "SSMState", "load_library",
    "hymba_layer_prefill", "hymba_layer_decode", "hymba_layer_decode_static",
    "hymba_kv_ring_fill",
    "hymba_layer_workspace_bytes",
    "hymba_status_str", "hymba_abi_version", "hymba_last_hip_error", "hymba_timer_enable",
    "hymba_timer_read", "hymba_op_gemm", "hymba_op_copy", "hymba_op_probe", "HymbaLayer",
    "STAGES",
    "DTYPE_F32", "DTYPE_BF16", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhymba.so")
DTYPE_F32, DTYPE_BF16 = 0, 1
STATUS = {0: "OK", 1: "ERR_INVALID_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE",
          4: "ERR_ALIGNMENT", 5: "ERR_HIP"}
STAGES = ["in_proj", "attn", "x_proj", "dt_proj", "scan", "norm", "out_proj", "kv_write",
          "meta", "misc", "block"]


class HymbaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {STATUS.get(status, status)}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "n_q_heads", "n_kv_heads", "head_dim", "d_inner", "d_state", "dt_rank",
        "n_meta", "window", "kv_share", "dtype")] + [
        ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("ssm_heads", ctypes.c_int32), ("norm_group", ctypes.c_int32),
        ("scan_chunk", ctypes.c_int32)]

    @classmethod
    def from_dims(cls, dims) -> "LayerDesc":
        return cls(dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.d_inner,
                   dims.d_state, dims.dt_rank, dims.n_meta, dims.window, dims.kv_share,
                   DTYPE_BF16 if dims.dtype == "bf16" else DTYPE_F32, dims.rms_eps,
                   dims.softmax_scale, getattr(dims, "ssm_heads", 0),
                   getattr(dims, "norm_group", 0), getattr(dims, "scan_chunk", 0))


class BlockWeights(ctypes.Structure):
    _fields_ = [("norm1", ctypes.c_void_p), ("norm2", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("intermediate", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_in", "w_x", "w_dt", "w_out", "dt_bias", "A", "D", "beta_attn", "beta_ssm")]


class KV(ctypes.Structure):
    _fields_ = [("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("slots", ctypes.c_int32),
                ("is_ring", ctypes.c_int32)]


class SSMState(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


class MetaCache(ctypes.Structure):
    _fields_ = [("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("y_meta", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def load_library() -> ctypes.CDLL:
    """Load libhymba.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libhymba.so not built at {LIB_PATH}; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int64
    sig = {
        "hymba_layer_prefill": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P,
                                      P, I32, I32, ctypes.POINTER(KV), ctypes.POINTER(KV),
                                      ctypes.POINTER(SSMState), P, P, P, SZ, P]),
        "hymba_layer_decode": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P,
                                     I32, ctypes.POINTER(KV), ctypes.POINTER(SSMState), P, P, SZ,
                                     P]),
        "hymba_layer_decode_static": (I32, [ctypes.POINTER(LayerDesc),
                                            ctypes.POINTER(LayerWeights), P, I32,
                                            ctypes.POINTER(KV), ctypes.POINTER(SSMState), P,
                                            P]),
        "hymba_layer_workspace_bytes": (SZ, [ctypes.POINTER(LayerDesc), I32, I32, I32]),
        "hymba_op_probe": (I32, [I32, I32, I32, P, SZ, P, P]),
        "hymba_kv_ring_fill": (I32, [ctypes.POINTER(KV), ctypes.POINTER(KV), I32, I32, I32, I32,
                                     I32, I32, P]),
        "hymba_layer_meta_cache_build": (I32, [ctypes.POINTER(LayerDesc),
                                               ctypes.POINTER(LayerWeights), P, ctypes.POINTER(KV),
                                               ctypes.POINTER(MetaCache), P, SZ, P]),
        "hymba_layer_prefill_cached": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                             ctypes.POINTER(MetaCache), P, I32, I32,
                                             ctypes.POINTER(KV), ctypes.POINTER(KV),
                                             ctypes.POINTER(SSMState), P, P, SZ, P]),
        "hymba_block_workspace_bytes": (SZ, [ctypes.POINTER(LayerDesc), I32, I32, I32, I32]),
        "hymba_block_prefill": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                      ctypes.POINTER(BlockWeights), P, P, I32, I32,
                                      ctypes.POINTER(KV), ctypes.POINTER(KV),
                                      ctypes.POINTER(SSMState), P, P, P, SZ, P]),
        "hymba_block_decode": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                     ctypes.POINTER(BlockWeights), P, I32, ctypes.POINTER(KV),
                                     ctypes.POINTER(SSMState), P, P, SZ, P]),
        "hymba_status_str": (ctypes.c_char_p, [I32]),
        "hymba_abi_version": (I32, []),
        "hymba_last_hip_error": (I32, []),
        "hymba_timer_enable": (I32, [I32]),
        "hymba_timer_read": (I32, [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
        "hymba_op_gemm": (I32, [I32, P, I64, P, I64, P, I64, I32, I32, I32, I32, P]),
        "hymba_op_copy": (I32, [P, P, SZ, P]),
        "hymba_op_attn_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "hymba_op_attn": (I32, [I32, P, I64, P, P, I64, P, I64, I32, I32, I32, I32, I32, I32,
                                I32, ctypes.c_float, P, SZ, P]),
        "hymba_op_scan_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32, I32, I32]),
        "hymba_op_scan": (I32, [I32, P, I64, I32, I32, P, P, P, P, P, P, P, I64, P, I32, I32, I32,
                                I32, I32, I32, I32, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None for None); ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise HymbaError(status, where, load_library().hymba_last_hip_error())


def _ref(obj):
    return ctypes.byref(obj) if obj is not None else None


# ----------------------------------------------------------------- raw ABI mirrors

def hymba_abi_version() -> int:
    return load_library().hymba_abi_version()


def hymba_status_str(status: int) -> str:
    return load_library().hymba_status_str(status).decode()


def hymba_last_hip_error() -> int:
    return load_library().hymba_last_hip_error()


def hymba_layer_workspace_bytes(desc: LayerDesc, batch: int, seq_len: int, mode: int) -> int:
    return load_library().hymba_layer_workspace_bytes(ctypes.byref(desc), batch, seq_len, mode)


def hymba_layer_prefill(desc, weights, meta, x, batch, seq_len, kv_in, kv_out, state_out, y,
                        y_meta, workspace, workspace_bytes, stream=None, check=True) -> int:
    st = load_library().hymba_layer_prefill(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(meta), _ptr(x), batch, seq_len,
        _ref(kv_in), _ref(kv_out), _ref(state_out), _ptr(y), _ptr(y_meta), _ptr(workspace),
        workspace_bytes, _stream(stream))
    if check:
        _check(st, "hymba_layer_prefill")
    return st


def hymba_layer_decode(desc, weights, x, batch, kv, state, y, workspace, workspace_bytes,
                       stream=None, check=True) -> int:
    st = load_library().hymba_layer_decode(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(x), batch, _ref(kv), _ref(state), _ptr(y),
        _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "hymba_layer_decode")
    return st


def hymba_layer_decode_static(desc, weights, x, batch, kv, state, y, stream=None,
                              check=True) -> int:
    st = load_library().hymba_layer_decode_static(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(x), batch, _ref(kv), _ref(state), _ptr(y),
        _stream(stream))
    if check:
        _check(st, "hymba_layer_decode_static")
    return st


def hymba_kv_ring_fill(src, dst, batch, seq_len, n_meta, n_kv_heads, head_dim, dtype,
                       stream=None, check=True) -> int:
    st = load_library().hymba_kv_ring_fill(ctypes.byref(src), ctypes.byref(dst), batch, seq_len,
                                           n_meta, n_kv_heads, head_dim, dtype, _stream(stream))
    if check:
        _check(st, "hymba_kv_ring_fill")
    return st


def hymba_layer_meta_cache_build(desc, weights, meta, kv_in, cache, workspace, workspace_bytes,
                                 stream=None, check=True) -> int:
    st = load_library().hymba_layer_meta_cache_build(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(meta), _ref(kv_in), ctypes.byref(cache),
        _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "hymba_layer_meta_cache_build")
    return st


def hymba_layer_prefill_cached(desc, weights, cache, x, batch, seq_len, kv_in, kv_out, state_out,
                               y, workspace, workspace_bytes, stream=None, check=True) -> int:
    st = load_library().hymba_layer_prefill_cached(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(cache), _ptr(x), batch, seq_len,
        _ref(kv_in), _ref(kv_out), _ref(state_out), _ptr(y), _ptr(workspace), workspace_bytes,
        _stream(stream))
    if check:
        _check(st, "hymba_layer_prefill_cached")
    return st


def hymba_block_workspace_bytes(desc: LayerDesc, intermediate: int, batch: int, seq_len: int,
                                mode: int) -> int:
    return load_library().hymba_block_workspace_bytes(ctypes.byref(desc), intermediate, batch,
                                                      seq_len, mode)


def hymba_block_prefill(desc, weights, block, meta, x, batch, seq_len, kv_in, kv_out, state_out,
                        y, y_meta, workspace, workspace_bytes, stream=None, check=True) -> int:
    st = load_library().hymba_block_prefill(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(block), _ptr(meta), _ptr(x),
        batch, seq_len, _ref(kv_in), _ref(kv_out), _ref(state_out), _ptr(y), _ptr(y_meta),
        _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "hymba_block_prefill")
    return st


def hymba_block_decode(desc, weights, block, x, batch, kv, state, y, workspace, workspace_bytes,
                       stream=None, check=True) -> int:
    st = load_library().hymba_block_decode(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(block), _ptr(x), batch, _ref(kv),
        _ref(state), _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "hymba_block_decode")
    return st


def hymba_timer_enable(stage_mask) -> None:
    """stage_mask: bit i selects stage i (STAGES order); True = all, False/0 = off."""
    if stage_mask is True:
        stage_mask = -1
    elif stage_mask is False:
        stage_mask = 0
    _check(load_library().hymba_timer_enable(int(stage_mask)), "hymba_timer_enable")


def hymba_timer_read(stage: int):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(load_library().hymba_timer_read(stage, ctypes.byref(ms), ctypes.byref(n)),
           "hymba_timer_read")
    return ms.value, n.value


def hymba_op_gemm(dtype, a, lda, b, ldb, c, ldc, c_dtype, m, n, k, stream=None) -> None:
    _check(load_library().hymba_op_gemm(dtype, _ptr(a), lda, _ptr(b), ldb, _ptr(c), ldc, c_dtype,
                                        m, n, k, _stream(stream)), "hymba_op_gemm")


def hymba_op_probe(kind, blocks, iters, src, nbytes, out, stream=None) -> None:
    _check(load_library().hymba_op_probe(kind, blocks, iters, _ptr(src), nbytes, _ptr(out),
                                         _stream(stream)), "hymba_op_probe")


def hymba_op_copy(src, dst, nbytes, stream=None) -> None:
    _check(load_library().hymba_op_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "hymba_op_copy")


def hymba_op_attn_workspace_bytes(dtype, n_meta, seq_len, batch, n_kv_heads, head_dim) -> int:
    return load_library().hymba_op_attn_workspace_bytes(dtype, n_meta, seq_len, batch,
                                                        n_kv_heads, head_dim)


def hymba_op_attn(dtype, q, q_ld, k, v, kv_ld, o, o_ld, n_meta, seq_len, batch, n_q_heads,
                  n_kv_heads, head_dim, window, scale, workspace, workspace_bytes, stream=None,
                  check=True) -> int:
    st = load_library().hymba_op_attn(dtype, _ptr(q), q_ld, _ptr(k), _ptr(v), kv_ld, _ptr(o),
                                      o_ld, n_meta, seq_len, batch, n_q_heads, n_kv_heads,
                                      head_dim, window, scale, _ptr(workspace), workspace_bytes,
                                      _stream(stream))
    if check:
        _check(st, "hymba_op_attn")
    return st


def hymba_op_scan_workspace_bytes(dtype, n_meta, seq_len, batch, d_inner, d_state,
                                  dt_rank, chunk_tokens=0) -> int:
    return load_library().hymba_op_scan_workspace_bytes(dtype, n_meta, seq_len, batch, d_inner,
                                                        d_state, dt_rank, chunk_tokens)


def hymba_op_scan(dtype, z, z_ld, xs_col, g_col, delta, bc, w_dt, dt_bias, A, D, y, y_ld, h_out,
                  n_meta, seq_len, batch, d_inner, d_state, dt_rank, chunk_tokens, workspace,
                  workspace_bytes, stream=None, check=True) -> int:
    st = load_library().hymba_op_scan(dtype, _ptr(z), z_ld, xs_col, g_col, _ptr(delta), _ptr(bc),
                                      _ptr(w_dt), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(y), y_ld,
                                      _ptr(h_out), n_meta, seq_len, batch, d_inner, d_state,
                                      dt_rank, chunk_tokens, _ptr(workspace), workspace_bytes,
                                      _stream(stream))
    if check:
        _check(st, "hymba_op_scan")
    return st


# ----------------------------------------------------------------- convenience

class HymbaLayer:
    """One layer's weights on the device plus the descriptor; allocates workspace and
    outputs with torch and calls the ABI.  `w` maps the weight names of
    hymba_layer_weights to device tensors."""

    def __init__(self, dims, w: dict, device="cuda"):
        import torch
        self.dims = dims
        self.desc = LayerDesc.from_dims(dims)
        self.w = {k: v.to(device).contiguous() for k, v in w.items()}
        # an empty tensor (w_dt of a Mamba-2 head layer) is passed as NULL
        self.weights = LayerWeights(*[self.w[n].data_ptr() if self.w[n].numel() else None
                                      for n, _ in LayerWeights._fields_])
        self.device = device
        self.store = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        self._ws = None

    def workspace(self, nbytes: int):
        import torch
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def prefill(self, meta, x, kv_in: Optional[KV] = None, kv_out: Optional[KV] = None,
                state_out: Optional[SSMState] = None, y=None, y_meta=None, stream=None):
        import torch
        B, L = x.shape[0], x.shape[1]
        d = self.dims.d_model
        if y is None:
            y = torch.empty(B, L, d, dtype=self.store, device=self.device)
        if y_meta is None:
            y_meta = torch.empty(self.dims.n_meta, d, dtype=self.store, device=self.device)
        nb = hymba_layer_workspace_bytes(self.desc, B, L, 0)
        ws = self.workspace(nb)
        hymba_layer_prefill(self.desc, self.weights, meta, x, B, L, kv_in, kv_out, state_out, y,
                            y_meta, ws, ws.numel(), stream)
        return y, y_meta

    def build_meta_cache(self, meta, kv_in: Optional[KV] = None, stream=None):
        """The layer over its meta tokens alone, once per weight set.  Returns (dict of
        device tensors, MetaCache struct pointing at them)."""
        import torch
        dm = self.dims
        M = dm.n_meta
        t = {"h": torch.zeros(dm.d_inner, dm.d_state, dtype=torch.float32, device=self.device),
             "y_meta": torch.empty(max(M, 1), dm.d_model, dtype=self.store, device=self.device)}
        if not dm.kv_share:
            for n in ("k_meta", "v_meta"):
                t[n] = torch.zeros(dm.n_kv_heads, max(M, 1), dm.head_dim, dtype=self.store,
                                   device=self.device)
        cache = MetaCache(_ptr(t.get("k_meta")), _ptr(t.get("v_meta")), _ptr(t["h"]),
                          _ptr(t["y_meta"]))
        nb = hymba_layer_workspace_bytes(self.desc, 0, 0, 0)
        ws = self.workspace(nb)
        hymba_layer_meta_cache_build(self.desc, self.weights, meta, kv_in, cache, ws, ws.numel(),
                                     stream)
        return t, cache

    def prefill_cached(self, cache: "MetaCache", x, kv_in: Optional[KV] = None,
                       kv_out: Optional[KV] = None, state_out: Optional[SSMState] = None, y=None,
                       stream=None):
        import torch
        B, L = x.shape[0], x.shape[1]
        if y is None:
            y = torch.empty(B, L, self.dims.d_model, dtype=self.store, device=self.device)
        nb = hymba_layer_workspace_bytes(self.desc, B, L, 2)
        ws = self.workspace(nb)
        hymba_layer_prefill_cached(self.desc, self.weights, cache, x, B, L, kv_in, kv_out,
                                   state_out, y, ws, ws.numel(), stream)
        return y

    def decode(self, x, kv: KV, state: SSMState, y=None, stream=None):
        import torch
        B = x.shape[0]
        if y is None:
            y = torch.empty(B, self.dims.d_model, dtype=self.store, device=self.device)
        nb = hymba_layer_workspace_bytes(self.desc, B, kv.slots, 1)
        ws = self.workspace(nb)
        hymba_layer_decode(self.desc, self.weights, x, B, kv, state, y, ws, ws.numel(), stream)
        return y


class HymbaBlock(HymbaLayer):
    """The layer inside its block wrapper (pre-norm, residual, FFN).  `bw` maps norm1,
    norm2, w_up, w_down to device tensors."""

    def __init__(self, dims, w: dict, bw: dict, device="cuda"):
        super().__init__(dims, w, device=device)
        self.bw = {k: v.to(device).contiguous() for k, v in bw.items()}
        self.inter = int(self.bw["w_up"].shape[0])
        self.block = BlockWeights(self.bw["norm1"].data_ptr(), self.bw["norm2"].data_ptr(),
                                  self.bw["w_up"].data_ptr(), self.bw["w_down"].data_ptr(),
                                  self.inter)

    def prefill(self, meta, x, kv_in: Optional[KV] = None, kv_out: Optional[KV] = None,
                state_out: Optional[SSMState] = None, y=None, y_meta=None, stream=None):
        import torch
        B, L = x.shape[0], x.shape[1]
        d = self.dims.d_model
        if y is None:
            y = torch.empty(B, L, d, dtype=self.store, device=self.device)
        if y_meta is None:
            y_meta = torch.empty(self.dims.n_meta, d, dtype=self.store, device=self.device)
        nb = hymba_block_workspace_bytes(self.desc, self.inter, B, L, 0)
        ws = self.workspace(nb)
        hymba_block_prefill(self.desc, self.weights, self.block, meta, x, B, L, kv_in, kv_out,
                            state_out, y, y_meta, ws, ws.numel(), stream)
        return y, y_meta

    def decode(self, x, kv: KV, state: SSMState, y=None, stream=None):
        import torch
        B = x.shape[0]
        if y is None:
            y = torch.empty(B, self.dims.d_model, dtype=self.store, device=self.device)
        nb = hymba_block_workspace_bytes(self.desc, self.inter, B, kv.slots, 1)
        ws = self.workspace(nb)
        hymba_block_decode(self.desc, self.weights, self.block, x, B, kv, state, y, ws,
                           ws.numel(), stream)
        return y


def make_kv(k_meta, v_meta, k, v, is_ring: bool = True) -> KV:
    """A cache over tensors k/v [B, Hkv, slots, dh]: a ring of the last `slots` positions
    (is_ring) or one slot per position."""
    return KV(_ptr(k_meta), _ptr(v_meta), _ptr(k), _ptr(v), int(k.shape[2]), int(bool(is_ring)))


def make_state(h, pos) -> SSMState:
    return SSMState(_ptr(h), _ptr(pos))
