"""ctypes binding of liblte.so (the C ABI in include/lte.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The library
is loaded on first use; if it is missing or fails to load, every call raises
-- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblte.so")
_lib = None

LTE_OK = 0
STATUS_NAMES = {0: "LTE_OK", 1: "LTE_ERR_INVALID_ARG", 2: "LTE_ERR_UNSUPPORTED",
                3: "LTE_ERR_STATE", 4: "LTE_ERR_HIP", 5: "LTE_ERR_WORKSPACE",
                6: "LTE_ERR_SCRATCH"}


class LTEError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().lte_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "q_heads", "kv_heads", "head_dim", "sink", "window", "capacity",
                 "hidden")]


class _CNN(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p)]


class _CacheLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("k", "v", "ret_idx", "ret_score", "ring_score", "count", "pos",
                 "next_unscored", "flags", "weak", "nx_slot", "nx_score", "arrive", "total")]


class _LinConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "heads", "head_dim")]


class _WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("scores", "rank", "thr", "ncand", "total")]


# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_CFG = ctypes.POINTER(_Config)
_CNNP = ctypes.POINTER(_CNN)
_LCFG = ctypes.POINTER(_LinConfig)
SIGNATURES = {
    "lte_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lte_version": (ctypes.c_int, []),
    "lte_check_config": (ctypes.c_int, [_CFG]),
    "lte_cache_bytes": (_SZ, [_CFG]),
    "lte_cache_get_layout": (ctypes.c_int, [_CFG, ctypes.POINTER(_CacheLayout)]),
    "lte_workspace_bytes": (_SZ, [_CFG, _I64]),
    "lte_workspace_get_layout": (ctypes.c_int, [_CFG, _I64, ctypes.POINTER(_WsLayout)]),
    "lte_cache_init": (ctypes.c_int, [_CFG, _P, _P]),
    "lte_prefill": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _CNNP, _P, _P, _P, _SZ, _P, _P]),
    "lte_prefill_varlen": (ctypes.c_int,
                           [_CFG, _I64, _P, _P, _P, _P, _CNNP, _P, _P, _P, _SZ, _P, _P]),
    "lte_chunk_workspace_bytes": (_SZ, [_CFG, _I64]),
    "lte_linear_check_config": (ctypes.c_int, [_LCFG]),
    "lte_linear_state_bytes": (_SZ, [_LCFG]),
    "lte_linear_prefill": (ctypes.c_int, [_LCFG, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "lte_linear_decode_step": (ctypes.c_int, [_LCFG, _P, _P, _P, _P, _P, _P, _P]),
    "lte_prefill_chunk": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _CNNP, _P, _P, _SZ, _P, _P]),
    "lte_prefill_score": (ctypes.c_int, [_CFG, _I64, _P, _P, _CNNP, _P, _SZ, _P]),
    "lte_prefill_select": (ctypes.c_int, [_CFG, _I64, _P, _P, _SZ, _P]),
    "lte_prefill_attend": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _P, _SZ, _P, _P]),
    "lte_prefill_build_cache": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _SZ, _P, _P]),
    "lte_prefill_build_cache_background": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _SZ, _P, _P]),
    "lte_score_evict": (ctypes.c_int, [_CFG, _CNNP, _P, _P, _P, _P]),
    "lte_decode_attend": (ctypes.c_int, [_CFG, _P, _P, _P, _SZ, _P, _P]),
    "lte_decode_step": (ctypes.c_int, [_CFG, _P, _P, _P, _CNNP, _P, _P, _SZ, _P, _P]),
    "lte_decode_step_static": (ctypes.c_int, [_CFG, _P, _P, _P, _CNNP, _P, _P, _P]),
    "lte_cache_export": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P]),
}


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m learnable_kv_cache_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != LTE_OK:
        raise LTEError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclass(frozen=True)
class Config:
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    sink: int
    window: int
    capacity: int
    hidden: int = 32

    def c(self):
        return _Config(self.batch, self.q_heads, self.kv_heads, self.head_dim, self.sink,
                       self.window, self.capacity, self.hidden)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


class CNN:
    """Device copies of the scoring-CNN parameters (fp32)."""

    def __init__(self, params: dict, device="cuda"):
        self.t = {k: torch.as_tensor(params[k], dtype=torch.float32).contiguous().to(device)
                  for k in ("W1", "b1", "W2", "b2")}
        self.c = _CNN(self.t["W1"].data_ptr(), self.t["b1"].data_ptr(),
                      self.t["W2"].data_ptr(), self.t["b2"].data_ptr())


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous device {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


class Layer:
    """One LTE layer of a given shape: cache/workspace sizing and the ABI calls."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._c = cfg.c()
        _check(lib().lte_check_config(ctypes.byref(self._c)), "lte_check_config")

    # -- sizes and layouts ------------------------------------------------------
    def cache_bytes(self) -> int:
        return int(lib().lte_cache_bytes(ctypes.byref(self._c)))

    def workspace_bytes(self, T: int) -> int:
        return int(lib().lte_workspace_bytes(ctypes.byref(self._c), int(T)))

    def cache_layout(self) -> dict:
        L = _CacheLayout()
        _check(lib().lte_cache_get_layout(ctypes.byref(self._c), ctypes.byref(L)),
               "lte_cache_get_layout")
        return {n: int(getattr(L, n)) for n, _ in _CacheLayout._fields_}

    def workspace_layout(self, T: int) -> dict:
        L = _WsLayout()
        _check(lib().lte_workspace_get_layout(ctypes.byref(self._c), int(T), ctypes.byref(L)),
               "lte_workspace_get_layout")
        return {n: int(getattr(L, n)) for n, _ in _WsLayout._fields_}

    def alloc_cache(self, device="cuda") -> torch.Tensor:
        cache = torch.empty(self.cache_bytes(), dtype=torch.uint8, device=device)
        self.cache_init(cache)
        return cache

    def alloc_workspace(self, T: int, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_bytes(T), dtype=torch.uint8, device=device)

    # -- prefill -------------------------------------------------------------------
    def prefill(self, q, k, v, cnn: CNN | None = None, score_override=None, cache=None,
                workspace=None, out=None, seq_lens=None):
        """Prefill of [B, T] prompts; seq_lens (int32 [B] on the device) gives each
        sequence's length when they differ (rows at or past it are padding)."""
        c = self.cfg
        B, T = q.shape[0], q.shape[1]
        _need(q, torch.bfloat16, (c.batch, T, c.q_heads, c.head_dim), "q")
        _need(k, torch.bfloat16, (c.batch, T, c.kv_heads, c.head_dim), "k")
        _need(v, torch.bfloat16, (c.batch, T, c.kv_heads, c.head_dim), "v")
        if score_override is not None:
            _need(score_override, torch.float32, (c.batch, c.kv_heads, T), "score_override")
        if workspace is None:
            workspace = self.alloc_workspace(T, q.device)
        if out is None:
            out = torch.empty_like(q)
        cnn_p = ctypes.byref(cnn.c) if cnn is not None else None
        if seq_lens is None:
            _check(lib().lte_prefill(
                ctypes.byref(self._c), int(T), _ptr(q), _ptr(k), _ptr(v), cnn_p,
                _ptr(score_override), _ptr(cache), _ptr(workspace), int(workspace.numel()),
                _ptr(out), _stream()), "lte_prefill")
        else:
            _need(seq_lens, torch.int32, (c.batch,), "seq_lens")
            _check(lib().lte_prefill_varlen(
                ctypes.byref(self._c), int(T), _ptr(seq_lens), _ptr(q), _ptr(k), _ptr(v), cnn_p,
                _ptr(score_override), _ptr(cache), _ptr(workspace), int(workspace.numel()),
                _ptr(out), _stream()), "lte_prefill_varlen")
        return out

    def chunk_workspace_bytes(self, n: int) -> int:
        return int(lib().lte_chunk_workspace_bytes(ctypes.byref(self._c), int(n)))

    def alloc_chunk_workspace(self, n: int, device="cuda") -> torch.Tensor:
        nbytes = self.chunk_workspace_bytes(n)
        if nbytes == 0:
            raise ValueError(f"chunk of {n} tokens not supported for this layer")
        return torch.empty(nbytes, dtype=torch.uint8, device=device)

    def prefill_chunk(self, q, k, v, cnn: CNN, cache, workspace=None, out=None):
        """Appends n tokens per sequence to the cache and returns their outputs."""
        c = self.cfg
        n = q.shape[1]
        _need(q, torch.bfloat16, (c.batch, n, c.q_heads, c.head_dim), "q")
        _need(k, torch.bfloat16, (c.batch, n, c.kv_heads, c.head_dim), "k")
        _need(v, torch.bfloat16, (c.batch, n, c.kv_heads, c.head_dim), "v")
        if workspace is None:
            workspace = self.alloc_chunk_workspace(n, q.device)
        if out is None:
            out = torch.empty_like(q)
        _check(lib().lte_prefill_chunk(
            ctypes.byref(self._c), int(n), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cnn.c),
            _ptr(cache), _ptr(workspace), int(workspace.numel()), _ptr(out), _stream()),
            "lte_prefill_chunk")
        return out

    def prefill_score(self, k, v, cnn: CNN, workspace):
        T = k.shape[1]
        _check(lib().lte_prefill_score(ctypes.byref(self._c), int(T), _ptr(k), _ptr(v),
                                       ctypes.byref(cnn.c), _ptr(workspace),
                                       int(workspace.numel()), _stream()), "lte_prefill_score")

    def prefill_select(self, T, workspace, score_override=None):
        _check(lib().lte_prefill_select(ctypes.byref(self._c), int(T), _ptr(score_override),
                                        _ptr(workspace), int(workspace.numel()), _stream()),
               "lte_prefill_select")

    def prefill_attend(self, q, k, v, workspace, out):
        T = q.shape[1]
        _check(lib().lte_prefill_attend(ctypes.byref(self._c), int(T), _ptr(q), _ptr(k),
                                        _ptr(v), _ptr(workspace), int(workspace.numel()),
                                        _ptr(out), _stream()), "lte_prefill_attend")

    def prefill_build_cache(self, k, v, workspace, cache):
        T = k.shape[1]
        _check(lib().lte_prefill_build_cache(ctypes.byref(self._c), int(T), _ptr(k), _ptr(v),
                                             _ptr(workspace), int(workspace.numel()),
                                             _ptr(cache), _stream()), "lte_prefill_build_cache")

    def prefill_build_cache_background(self, k, v, workspace, cache):
        """prefill_build_cache with a low-bandwidth row copy, for a second stream beside
        prefill_attend."""
        T = k.shape[1]
        _check(lib().lte_prefill_build_cache_background(
            ctypes.byref(self._c), int(T), _ptr(k), _ptr(v), _ptr(workspace),
            int(workspace.numel()), _ptr(cache), _stream()), "lte_prefill_build_cache_background")

    def workspace_views(self, workspace, T: int) -> dict:
        """Device views of the last prefill's scores [B,Hkv,T], rank, thr, ncand."""
        c = self.cfg
        L = self.workspace_layout(T)
        n = c.batch * c.kv_heads * T

        def view(off, count, dtype):
            nbytes = count * torch.empty((), dtype=dtype).element_size()
            return workspace[off:off + nbytes].view(dtype)

        return {
            "scores": view(L["scores"], n, torch.float32).view(c.batch, c.kv_heads, T),
            "rank": view(L["rank"], n, torch.int32).view(c.batch, c.kv_heads, T),
            "thr": view(L["thr"], n, torch.int32).view(c.batch, c.kv_heads, T),
            "ncand": view(L["ncand"], c.batch * c.kv_heads, torch.int32).view(c.batch, c.kv_heads),
        }

    # -- cache and decode -------------------------------------------------------------
    def cache_init(self, cache):
        _check(lib().lte_cache_init(ctypes.byref(self._c), _ptr(cache), _stream()),
               "lte_cache_init")

    def score_evict(self, k_t, v_t, cnn: CNN, cache):
        _check(lib().lte_score_evict(ctypes.byref(self._c), ctypes.byref(cnn.c), _ptr(k_t),
                                     _ptr(v_t), _ptr(cache), _stream()), "lte_score_evict")

    def decode_attend(self, q_t, cache, workspace, out_t=None):
        if out_t is None:
            out_t = torch.empty_like(q_t)
        _check(lib().lte_decode_attend(ctypes.byref(self._c), _ptr(q_t), _ptr(cache),
                                       _ptr(workspace), int(workspace.numel()), _ptr(out_t),
                                       _stream()), "lte_decode_attend")
        return out_t

    def decode_step(self, q_t, k_t, v_t, cnn: CNN, cache, workspace, out_t=None):
        c = self.cfg
        _need(q_t, torch.bfloat16, (c.batch, c.q_heads, c.head_dim), "q_t")
        _need(k_t, torch.bfloat16, (c.batch, c.kv_heads, c.head_dim), "k_t")
        _need(v_t, torch.bfloat16, (c.batch, c.kv_heads, c.head_dim), "v_t")
        if out_t is None:
            out_t = torch.empty_like(q_t)
        _check(lib().lte_decode_step(ctypes.byref(self._c), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                     ctypes.byref(cnn.c), _ptr(cache), _ptr(workspace),
                                     int(workspace.numel()), _ptr(out_t), _stream()),
               "lte_decode_step")
        return out_t

    def decode_step_static(self, q_t, k_t, v_t, cnn: CNN, cache, out_t):
        """lte_decode_step_static: one decode step with no workspace (the split partials
        live in the library's static device array); out_t is caller-provided."""
        c = self.cfg
        _need(q_t, torch.bfloat16, (c.batch, c.q_heads, c.head_dim), "q_t")
        _need(k_t, torch.bfloat16, (c.batch, c.kv_heads, c.head_dim), "k_t")
        _need(v_t, torch.bfloat16, (c.batch, c.kv_heads, c.head_dim), "v_t")
        _need(out_t, torch.bfloat16, (c.batch, c.q_heads, c.head_dim), "out_t")
        _check(lib().lte_decode_step_static(ctypes.byref(self._c), _ptr(q_t), _ptr(k_t),
                                            _ptr(v_t), ctypes.byref(cnn.c), _ptr(cache),
                                            _ptr(out_t), _stream()), "lte_decode_step_static")
        return out_t

    def cache_views(self, cache) -> dict:
        """Device views of every section of a cache blob."""
        c = self.cfg
        L = self.cache_layout()
        S = c.sink + c.capacity + c.window
        bg = c.batch * c.kv_heads

        def view(name, count, dtype, shape):
            nbytes = count * torch.empty((), dtype=dtype).element_size()
            return cache[L[name]:L[name] + nbytes].view(dtype).view(*shape)

        return {
            "k": view("k", bg * S * c.head_dim, torch.bfloat16, (c.batch, c.kv_heads, S, c.head_dim)),
            "v": view("v", bg * S * c.head_dim, torch.bfloat16, (c.batch, c.kv_heads, S, c.head_dim)),
            "ret_idx": view("ret_idx", bg * c.capacity, torch.int32, (c.batch, c.kv_heads, c.capacity)),
            "ret_score": view("ret_score", bg * c.capacity, torch.float32,
                              (c.batch, c.kv_heads, c.capacity)),
            "ring_score": view("ring_score", bg * c.window, torch.float32,
                               (c.batch, c.kv_heads, c.window)),
            "count": view("count", bg, torch.int32, (c.batch, c.kv_heads)),
            "pos": view("pos", bg, torch.int64, (c.batch, c.kv_heads)),
            "next_unscored": view("next_unscored", bg, torch.int64, (c.batch, c.kv_heads)),
            "flags": view("flags", bg, torch.int32, (c.batch, c.kv_heads)),
            "weak": view("weak", bg, torch.int32, (c.batch, c.kv_heads)),
            "nx_slot": view("nx_slot", bg, torch.int32, (c.batch, c.kv_heads)),
            "nx_score": view("nx_score", bg, torch.float32, (c.batch, c.kv_heads)),
            "arrive": view("arrive", bg, torch.int32, (c.batch, c.kv_heads)),
        }

    def cache_export(self, cache) -> dict:
        """Host copies of the retained-segment bookkeeping (via lte_cache_export)."""
        c = self.cfg
        dev = cache.device
        ret_idx = torch.empty((c.batch, c.kv_heads, c.capacity), dtype=torch.int32, device=dev)
        ret_score = torch.empty((c.batch, c.kv_heads, c.capacity), dtype=torch.float32, device=dev)
        count = torch.empty((c.batch, c.kv_heads), dtype=torch.int32, device=dev)
        pos = torch.empty((c.batch, c.kv_heads), dtype=torch.int64, device=dev)
        _check(lib().lte_cache_export(ctypes.byref(self._c), _ptr(cache), _ptr(ret_idx),
                                      _ptr(ret_score), _ptr(count), _ptr(pos), _stream()),
               "lte_cache_export")
        return {"ret_idx": ret_idx.cpu(), "ret_score": ret_score.cpu(), "count": count.cpu(),
                "pos": pos.cpu()}


class LinearLayer:
    """The hybrid's linear-attention layer (S_t = a_t S_{t-1} + v_t k_t^T, o_t = S_t q_t):
    argument marshalling for the ABI calls."""

    def __init__(self, batch: int, heads: int, head_dim: int):
        self.batch, self.heads, self.head_dim = batch, heads, head_dim
        self._c = _LinConfig(batch, heads, head_dim)
        _check(lib().lte_linear_check_config(ctypes.byref(self._c)), "lte_linear_check_config")

    def alloc_state(self, device="cuda") -> torch.Tensor:
        D = self.head_dim
        return torch.zeros((self.batch, self.heads, D, D), dtype=torch.float32, device=device)

    def prefill(self, q, k, v, log_a, state_in=None, state_out=None, out=None):
        """q, k, v [B, T, H, D] bf16, log_a [B, T, H] fp32; returns (out, state_out)."""
        B, H, D = self.batch, self.heads, self.head_dim
        T = q.shape[1]
        for t, nm in ((q, "q"), (k, "k"), (v, "v")):
            _need(t, torch.bfloat16, (B, T, H, D), nm)
        _need(log_a, torch.float32, (B, T, H), "log_a")
        if state_in is not None:
            _need(state_in, torch.float32, (B, H, D, D), "state_in")
        if state_out is None:
            state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        _check(lib().lte_linear_prefill(ctypes.byref(self._c), int(T), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(log_a), _ptr(state_in), _ptr(state_out), _ptr(out),
                                        _stream()), "lte_linear_prefill")
        return out, state_out

    def decode_step(self, q_t, k_t, v_t, log_a_t, state, out=None):
        """q_t, k_t, v_t [B, H, D] bf16, log_a_t [B, H] fp32; state updated in place."""
        B, H, D = self.batch, self.heads, self.head_dim
        for t, nm in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
            _need(t, torch.bfloat16, (B, H, D), nm)
        _need(log_a_t, torch.float32, (B, H), "log_a_t")
        _need(state, torch.float32, (B, H, D, D), "state")
        if out is None:
            out = torch.empty_like(q_t)
        _check(lib().lte_linear_decode_step(ctypes.byref(self._c), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                            _ptr(log_a_t), _ptr(state), _ptr(out), _stream()),
               "lte_linear_decode_step")
        return out
