"""Python binding of libphi (ctypes): argument marshalling only.

Every step of the prefill and decode paths runs in the HIP kernels of
``libphi.so``; torch provides device memory and the stream.  The functions
carry the names of the C entry points declared in ``include/phi.h``.
Importing works without a GPU; calling an entry point needs the built
library (``logits_parity_amd.build.build()``) and a GPU, and raises if the
library is missing - there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PHI_LIB names another build of the library (the host-sanitizer test uses it)
LIB_PATH = os.environ.get("PHI_LIB") or os.path.join(HERE, "libphi.so")

PHI_WT_F32, PHI_WT_F16, PHI_WT_I8 = 0, 1, 2
PROF_STAGES = ("embed", "qkv", "attn", "o_proj", "norm", "gate_up", "down", "lm_head")
PROF_N = len(PROF_STAGES)
WTYPES = {"f32": PHI_WT_F32, "f16": PHI_WT_F16, "i8": PHI_WT_I8}

EXPORTS = ("phi_state_bytes", "phi_load_fused", "phi_workspace_bytes", "phi_prefill_logits", "phi_free",
           "phi_strerror", "phi_linear_f32out", "phi_gate_up_silu", "phi_attention_vt_stride", "phi_attention_prefill",
           "attn_decode_k16v8_workspace_bytes", "attn_decode_k16v8", "phi_kv_pool_slots", "phi_profile_enable",
           "phi_profile_read", "kv_append_k16v8", "phi_prefill_fill_k16v8", "phi_decode_workspace_bytes",
           "phi_decode_step_k16v8", "attn_decode_k16v8_noalloc", "phi_prefill_logits_host_ids")


class PhiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class phi_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_pos", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("wtype", ctypes.c_int32)]


class phi_linear(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class phi_kv_cache(ctypes.Structure):
    _fields_ = [("k_pools", ctypes.POINTER(ctypes.c_void_p)), ("v_pools", ctypes.POINTER(ctypes.c_void_p)),
                ("v_scale", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("n_pages", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class phi_layer_weights(ctypes.Structure):
    _fields_ = [("ln1", ctypes.c_void_p), ("qkv", phi_linear), ("o", phi_linear), ("ln2", ctypes.c_void_p),
                ("gate_up", phi_linear), ("down", phi_linear), ("qkv_bias", ctypes.c_void_p)]


class phi_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("layers", ctypes.POINTER(phi_layer_weights)),
                ("final_norm", ctypes.c_void_p), ("lm_head", phi_linear)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run logits_parity_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "phi_state_bytes": (sz, [ctypes.POINTER(phi_config)]),
        "phi_load_fused": (i32, [ctypes.POINTER(phi_config), ctypes.POINTER(phi_weights), P, sz, P,
                                 ctypes.POINTER(P)]),
        "phi_workspace_bytes": (sz, [P, i32, i32]),
        "phi_prefill_logits": (i32, [P, P, i32, i32, P, P, sz, P]),
        "phi_prefill_logits_host_ids": (i32, [P, P, i32, i32, P, P, sz, P]),
        "phi_free": (None, [P]),
        "phi_strerror": (ctypes.c_char_p, [i32]),
        "phi_linear_f32out": (i32, [i32, P, P, P, P, i32, i32, i32, P]),
        "phi_gate_up_silu": (i32, [i32, P, P, P, P, i32, i32, i32, P]),
        "phi_attention_vt_stride": (sz, [i32]),
        "phi_attention_prefill": (i32, [i32, P, P, P, P, i32, i32, i32, i32, i32, P]),
        "attn_decode_k16v8_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "attn_decode_k16v8": (i32, [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f32, P, P, sz, P]),
        "attn_decode_k16v8_noalloc": (i32, [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f32, P, P]),
        "kv_append_k16v8": (i32, [P, P, P, P, P, i32, i32, i32, i32, i32, i32, P, P, P]),
        "phi_prefill_fill_k16v8": (i32, [P, P, i32, i32, P, ctypes.POINTER(phi_kv_cache), P, sz, P]),
        "phi_decode_workspace_bytes": (sz, [P, i32, i32]),
        "phi_decode_step_k16v8": (i32, [P, P, P, i32, i32, ctypes.POINTER(phi_kv_cache), P, P, sz, P]),
        "phi_kv_pool_slots": (i64, [i64, i32, i32, i32, i32, i32, i32]),
        "phi_profile_enable": (i32, [P, i32]),
        "phi_profile_read": (i32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().phi_strerror(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise PhiError(status, where)


def _ptr(t) -> int | None:
    """Device address of a tensor the library reads or writes as a dense
    row-major array: a strided view (a transpose, a broadcast, a slice with
    steps) would be read in the wrong layout, so it is refused."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} and strides {tuple(t.stride())} is not contiguous; "
                         "pass .contiguous()")
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_config(cfg) -> phi_config:
    """phi_config from any object with the PhiConfig fields."""
    return phi_config(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate,
                      cfg.vocab, cfg.max_pos, cfg.rms_eps, cfg.rope_theta, WTYPES[cfg.wtype])


def _lin(x) -> phi_linear:
    if isinstance(x, tuple):
        return phi_linear(_ptr(x[0]), _ptr(x[1]))
    return phi_linear(_ptr(x), None)


class Model:
    """A loaded model: borrowed device weights + RoPE state, released on del."""

    def __init__(self, cfg, weights: dict, stream=None):
        import torch
        self.cfg = cfg
        self._c = make_config(cfg)
        self._weights = weights  # keep the device tensors alive
        layers = (phi_layer_weights * cfg.n_layers)()
        for i, lw in enumerate(weights["layers"]):
            layers[i] = phi_layer_weights(_ptr(lw["ln1"]), _lin(lw["qkv"]), _lin(lw["o"]), _ptr(lw["ln2"]),
                                          _lin(lw["gate_up"]), _lin(lw["down"]), _ptr(lw.get("qkv_bias")))
        w = phi_weights(_ptr(weights["embed"]), layers, _ptr(weights["final_norm"]), _lin(weights["lm_head"]))
        nbytes = lib().phi_state_bytes(ctypes.byref(self._c))
        dev = weights["embed"].device
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p()
        _check(lib().phi_load_fused(ctypes.byref(self._c), ctypes.byref(w), _ptr(self.state), nbytes,
                                    _stream(stream), ctypes.byref(h)), "phi_load_fused")
        self.handle = h

    def workspace_bytes(self, batch: int, seq: int) -> int:
        return lib().phi_workspace_bytes(self.handle, batch, seq)

    def prefill_logits(self, ids, logits=None, workspace=None, stream=None):
        return phi_prefill_logits(self, ids, logits, workspace, stream)

    def prefill_fill_k16v8(self, ids, cache: "KVCache", logits=None, workspace=None, stream=None):
        """Prefill logits [B, S, V] that also writes every layer's keys and
        values of the B sequences into `cache` (pages from its block table)."""
        import torch
        B, S = ids.shape
        if ids.dtype != torch.int32 or not ids.is_contiguous():
            raise ValueError("ids must be a contiguous int32 tensor")
        if logits is None:
            logits = torch.empty((B, S, self.cfg.vocab), dtype=torch.float32, device=ids.device)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(B, S), dtype=torch.uint8, device=ids.device)
        c = cache.struct()
        _check(lib().phi_prefill_fill_k16v8(self.handle, _ptr(ids), B, S, _ptr(logits), ctypes.byref(c),
                                            _ptr(workspace), workspace.numel(), _stream(stream)),
               "phi_prefill_fill_k16v8")
        return logits

    def decode_step_k16v8(self, ids, positions, cache: "KVCache", max_ctx: int, logits=None, workspace=None,
                          stream=None):
        """One decode step: ids, positions int32 device [B] -> logits [B, V]."""
        import torch
        B = ids.shape[0]
        if logits is None:
            logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=ids.device)
        if workspace is None:
            need = lib().phi_decode_workspace_bytes(self.handle, B, max_ctx)
            workspace = torch.empty(need, dtype=torch.uint8, device=ids.device)
        c = cache.struct()
        _check(lib().phi_decode_step_k16v8(self.handle, _ptr(ids), _ptr(positions), B, max_ctx, ctypes.byref(c),
                                           _ptr(logits), _ptr(workspace), workspace.numel(), _stream(stream)),
               "phi_decode_step_k16v8")
        return logits

    def profile_enable(self, enable: bool = True):
        _check(lib().phi_profile_enable(self.handle, int(enable)), "phi_profile_enable")

    def profile_read(self) -> dict:
        """Per-stage device milliseconds and launch counts since the last read."""
        ms = (ctypes.c_double * PROF_N)()
        n = (ctypes.c_int64 * PROF_N)()
        _check(lib().phi_profile_read(self.handle, ms, n), "phi_profile_read")
        return {name: (ms[i], n[i]) for i, name in enumerate(PROF_STAGES)}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.phi_free(h)
            self.handle = None


class KVCache:
    """Device tensors of a K16/V8 paged cache for every layer (see
    phi_kv_cache in include/phi.h): k_pools / v_pools lists of
    [n_pages, n_kv_heads, 16, head_dim] binary16 / uint8 tensors, v_scale
    float32 [n_layers, n_kv_heads], block_table int32 [B, max_pages]."""

    def __init__(self, k_pools, v_pools, v_scale, block_table):
        self.k_pools, self.v_pools = list(k_pools), list(v_pools)
        self.v_scale, self.block_table = v_scale, block_table

    @classmethod
    def empty(cls, cfg, n_pages: int, block_table, v_scale, device="cuda"):
        import torch
        shape = (n_pages, cfg.n_kv_heads, 16, cfg.head_dim)
        k = [torch.zeros(shape, dtype=torch.float16, device=device) for _ in range(cfg.n_layers)]
        v = [torch.zeros(shape, dtype=torch.uint8, device=device) for _ in range(cfg.n_layers)]
        return cls(k, v, v_scale, block_table)

    def struct(self, block_table=None) -> phi_kv_cache:
        bt = self.block_table if block_table is None else block_table
        self._kp = (ctypes.c_void_p * len(self.k_pools))(*[_ptr(t) for t in self.k_pools])
        self._vp = (ctypes.c_void_p * len(self.v_pools))(*[_ptr(t) for t in self.v_pools])
        return phi_kv_cache(ctypes.cast(self._kp, ctypes.POINTER(ctypes.c_void_p)),
                            ctypes.cast(self._vp, ctypes.POINTER(ctypes.c_void_p)), _ptr(self.v_scale),
                            _ptr(bt), self.k_pools[0].shape[0], bt.shape[1], 16)

    def with_table(self, block_table) -> "KVCache":
        """The same pools seen through another block table (e.g. one row)."""
        return KVCache(self.k_pools, self.v_pools, self.v_scale, block_table)


def phi_load_fused(cfg, weights: dict, stream=None) -> Model:
    return Model(cfg, weights, stream)


def phi_prefill_logits(model: Model, ids, logits=None, workspace=None, stream=None):
    """ids: int32 device tensor [B, S] -> float32 logits [B, S, V]."""
    import torch
    B, S = ids.shape
    if ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 tensor")
    if logits is None:
        logits = torch.empty((B, S, model.cfg.vocab), dtype=torch.float32, device=ids.device)
    need = model.workspace_bytes(B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=ids.device)
    _check(lib().phi_prefill_logits(model.handle, _ptr(ids), B, S, _ptr(logits), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "phi_prefill_logits")
    return logits


def phi_prefill_logits_host_ids(model: Model, ids, logits, workspace=None, stream=None):
    """ids: int32 host array or CPU tensor [B, S], checked against the
    vocabulary by the library before anything is enqueued -> float32 logits
    [B, S, V] on the device of `logits`.  The ids buffer must stay unchanged
    until the stream has run the copy."""
    import numpy as np
    import torch
    if isinstance(ids, np.ndarray):
        if ids.dtype != np.int32 or not ids.flags["C_CONTIGUOUS"]:
            raise ValueError("ids must be a C-contiguous int32 array")
        B, S = ids.shape
        ids_addr = ids.ctypes.data
    else:
        if ids.dtype != torch.int32 or ids.device.type != "cpu":
            raise ValueError("ids must be an int32 CPU tensor")
        B, S = ids.shape
        ids_addr = _ptr(ids)
    need = model.workspace_bytes(B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    _check(lib().phi_prefill_logits_host_ids(model.handle, ids_addr, B, S, _ptr(logits), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)),
           "phi_prefill_logits_host_ids")
    return logits


def phi_linear_f32out(a, w, scale=None, out=None, stream=None):
    """y[M, N] float32 = a[M, K] w[N, K]^T (w float16, int8 with scale, or float32)."""
    import torch
    M, K = a.shape
    N = w.shape[0]
    wt = {torch.float16: PHI_WT_F16, torch.int8: PHI_WT_I8, torch.float32: PHI_WT_F32}[w.dtype]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _check(lib().phi_linear_f32out(wt, _ptr(a), _ptr(w), _ptr(scale), _ptr(out), M, N, K, _stream(stream)),
           "phi_linear_f32out")
    return out


def phi_gate_up_silu(a, w, scale=None, out=None, stream=None):
    """act[M, I] = silu(a w[:I]^T) * (a w[I:]^T) for the fused gate/up weight w [2I, K]."""
    import torch
    M, K = a.shape
    I = w.shape[0] // 2
    wt = {torch.float16: PHI_WT_F16, torch.int8: PHI_WT_I8, torch.float32: PHI_WT_F32}[w.dtype]
    if out is None:
        out = torch.empty((M, I), dtype=a.dtype, device=a.device)
    _check(lib().phi_gate_up_silu(wt, _ptr(a), _ptr(w), _ptr(scale), _ptr(out), M, I, K, _stream(stream)),
           "phi_gate_up_silu")
    return out


def phi_attention_vt_stride(seq: int) -> int:
    return lib().phi_attention_vt_stride(seq)


def phi_attention_prefill(q, k, vt, out=None, stream=None):
    """q [B, Hq, S, D], k [B, Hkv, S, D], vt [B, Hkv, D, s_pad] -> out [B, S, Hq * D]; D = 96, or 128
    for binary16."""
    import torch
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty((B, S, Hq * D), dtype=q.dtype, device=q.device)
    _check(lib().phi_attention_prefill(int(q.dtype == torch.float32), _ptr(q), _ptr(k), _ptr(vt), _ptr(out),
                                       B, S, Hq, Hkv, D, _stream(stream)), "phi_attention_prefill")
    return out


def attn_decode_k16v8_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_ctx) -> int:
    return lib().attn_decode_k16v8_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_ctx)


def attn_decode_k16v8(q, k_pool, v_pool, v_scale, block_table, ctx_lens, max_ctx: int, sm_scale: float,
                      out=None, workspace=None, stream=None):
    """One K16/V8 decode-attention step; see include/phi.h for layouts."""
    import torch
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pool.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    if workspace is None:
        workspace = torch.empty(attn_decode_k16v8_workspace_bytes(B, Hq, Hkv, D, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().attn_decode_k16v8(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(v_scale), _ptr(block_table),
                                   _ptr(ctx_lens), B, Hq, Hkv, D, page, P, block_table.shape[1], max_ctx,
                                   float(sm_scale), _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_decode_k16v8")
    return out


def attn_decode_k16v8_noalloc(q, k_pool, v_pool, v_scale, block_table, ctx_lens, max_ctx: int, sm_scale: float,
                              out=None, stream=None):
    """attn_decode_k16v8 with its partials in the library's fixed scratch array
    (no workspace); see include/phi.h."""
    import torch
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pool.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    _check(lib().attn_decode_k16v8_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(v_scale), _ptr(block_table),
                                           _ptr(ctx_lens), B, Hq, Hkv, D, page, P, block_table.shape[1], max_ctx,
                                           float(sm_scale), _ptr(out), _stream(stream)),
           "attn_decode_k16v8_noalloc")
    return out


def kv_append_k16v8(k_new, v_new, v_scale, block_table, positions, k_pool, v_pool, stream=None):
    """Append one token per sequence to the K16/V8 pools in place; see include/phi.h."""
    B, Hkv, D = k_new.shape
    P, _, page, _ = k_pool.shape
    _check(lib().kv_append_k16v8(_ptr(k_new), _ptr(v_new), _ptr(v_scale), _ptr(block_table), _ptr(positions), B,
                                 Hkv, D, page, P, block_table.shape[1], _ptr(k_pool), _ptr(v_pool),
                                 _stream(stream)), "kv_append_k16v8")


def phi_kv_pool_slots(budget_bytes: int, n_layers: int, n_kv_heads: int, head_dim: int, k_bytes: int,
                      v_bytes: int, page_size: int) -> int:
    return lib().phi_kv_pool_slots(budget_bytes, n_layers, n_kv_heads, head_dim, k_bytes, v_bytes, page_size)
