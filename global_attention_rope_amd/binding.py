"""ctypes binding of ``libmimo_attn.so`` (declared in ``include/mimo_attn.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI.
torch supplies device memory and the current stream.  If the library is not built, loading it
raises; there is no other execution path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmimo_attn.so")

MIMO_OK, MIMO_ERR_INVALID_ARG, MIMO_ERR_UNSUPPORTED, MIMO_ERR_WORKSPACE, MIMO_ERR_HIP = 0, -1, -2, -3, -4
LAYER_GLOBAL, LAYER_SWA = 0, 1
F32, BF16 = 0, 1
CACHE_SAME, CACHE_FP8_E4M3 = 0, 2

EXPORTS = ("mimo_attn_prefill", "mimo_attn_prefill_workspace_size", "mimo_attn_extend",
           "mimo_attn_extend_workspace_size", "mimo_attn_decode",
           "mimo_attn_decode_workspace_size", "mimo_attn_decode_noalloc",
           "mimo_attn_decode_noalloc_max_bytes", "mimo_attn_layer_prefill",
           "mimo_attn_layer_workspace_size", "mimo_attn_check_params", "mimo_attn_last_error",
           "mimo_attn_abi_version", "mimo_router_topk", "mimo_router_check_params")


class MimoAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mimo_attn error {code}: {msg}")
        self.code = code


class CParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("qk_head_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
        ("layer_kind", ctypes.c_int32), ("window", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("v_scale", ctypes.c_float),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32), ("k_cache_scale", ctypes.c_float),
        ("v_cache_scale", ctypes.c_float),
    ]


class CRouterParams(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


@dataclasses.dataclass
class RouterParams:
    num_experts: int = 256
    n_group: int = 8
    topk_group: int = 4
    top_k: int = 8
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 1.0

    def c(self, num_tokens: int) -> CRouterParams:
        return CRouterParams(num_tokens, self.num_experts, self.n_group, self.topk_group,
                             self.top_k, int(self.norm_topk_prob),
                             float(self.routed_scaling_factor), 0)


@dataclasses.dataclass
class Params:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    qk_head_dim: int
    v_head_dim: int
    rope_dims: int
    layer_kind: int
    window: int
    rope_theta: float
    v_scale: float = 1.0
    softmax_scale: float = 0.0
    dtype: int = BF16
    cache_dtype: int = CACHE_SAME      # CACHE_FP8_E4M3: caches are uint8 e4m3 codes
    k_cache_scale: float = 1.0
    v_cache_scale: float = 1.0

    def c(self) -> CParams:
        return CParams(self.batch, self.num_q_heads, self.num_kv_heads, self.qk_head_dim,
                       self.v_head_dim, self.rope_dims, self.layer_kind, self.window,
                       float(self.rope_theta), float(self.v_scale), float(self.softmax_scale),
                       self.dtype, self.cache_dtype, float(self.k_cache_scale),
                       float(self.v_cache_scale))


_lock = threading.Lock()
_lib = None


def lib(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m global_attention_rope_amd.build`")
            L = ctypes.CDLL(path)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            P = ctypes.POINTER(CParams)
            L.mimo_attn_prefill.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
            L.mimo_attn_prefill.restype = ctypes.c_int
            L.mimo_attn_prefill_workspace_size.argtypes = [P, i32]
            L.mimo_attn_prefill_workspace_size.restype = sz
            L.mimo_attn_extend.argtypes = [P, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, sz,
                                           vp]
            L.mimo_attn_extend.restype = ctypes.c_int
            L.mimo_attn_extend_workspace_size.argtypes = [P, i32, i32]
            L.mimo_attn_extend_workspace_size.restype = sz
            L.mimo_attn_decode.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
            L.mimo_attn_decode.restype = ctypes.c_int
            L.mimo_attn_decode_workspace_size.argtypes = [P, i32]
            L.mimo_attn_decode_workspace_size.restype = sz
            L.mimo_attn_decode_noalloc.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp]
            L.mimo_attn_decode_noalloc.restype = ctypes.c_int
            L.mimo_attn_decode_noalloc_max_bytes.argtypes = []
            L.mimo_attn_decode_noalloc_max_bytes.restype = sz
            L.mimo_attn_layer_prefill.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                                  vp, vp, i32, vp, sz, vp]
            L.mimo_attn_layer_prefill.restype = ctypes.c_int
            L.mimo_attn_layer_workspace_size.argtypes = [P, i32, i32]
            L.mimo_attn_layer_workspace_size.restype = sz
            R = ctypes.POINTER(CRouterParams)
            L.mimo_router_topk.argtypes = [R, vp, vp, vp, vp, vp]
            L.mimo_router_topk.restype = ctypes.c_int
            L.mimo_router_check_params.argtypes = [R]
            L.mimo_router_check_params.restype = ctypes.c_int
            L.mimo_attn_check_params.argtypes = [P]
            L.mimo_attn_check_params.restype = ctypes.c_int
            L.mimo_attn_last_error.argtypes = []
            L.mimo_attn_last_error.restype = ctypes.c_char_p
            L.mimo_attn_abi_version.argtypes = []
            L.mimo_attn_abi_version.restype = ctypes.c_int
            _lib = L
    return _lib


def last_error() -> str:
    return lib().mimo_attn_last_error().decode()


def _raise(code: int):
    if code != MIMO_OK:
        raise MimoAttnError(code, last_error())


def check_params(p: Params) -> int:
    cp = p.c()
    return lib().mimo_attn_check_params(ctypes.byref(cp))


def prefill_workspace_size(p: Params, seq_len: int) -> int:
    cp = p.c()
    return int(lib().mimo_attn_prefill_workspace_size(ctypes.byref(cp), seq_len))


def extend_workspace_size(p: Params, seq_len: int, max_start: int) -> int:
    cp = p.c()
    return int(lib().mimo_attn_extend_workspace_size(ctypes.byref(cp), seq_len, max_start))


def decode_workspace_size(p: Params, max_position: int) -> int:
    cp = p.c()
    return int(lib().mimo_attn_decode_workspace_size(ctypes.byref(cp), max_position))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tdtype(p: Params):
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def _cdtype(p: Params):
    """torch dtype of the caches: uint8 codes for fp8 caches, else the layer dtype."""
    return torch.uint8 if p.cache_dtype == CACHE_FP8_E4M3 else _tdtype(p)


def prefill(p: Params, q, k, v, start_pos, sinks=None, out=None, k_cache=None, v_cache=None,
            workspace=None, stream=None):
    """mimo_attn_prefill on torch device tensors (shapes as in include/mimo_attn.h).

    start_pos: int32 [B] device tensor.  Returns out [B,S,Hq,dv]."""
    B, S = q.shape[0], q.shape[1]
    dev, dt = q.device, _tdtype(p)
    if p.batch != B:
        raise ValueError(f"params.batch {p.batch} != q.shape[0] {B}")
    _expect(q, "q", (B, S, p.num_q_heads, p.qk_head_dim), dt, dev)
    _expect(k, "k", (B, S, p.num_kv_heads, p.qk_head_dim), dt, dev)
    _expect(v, "v", (B, S, p.num_kv_heads, p.v_head_dim), dt, dev)
    _expect(start_pos, "start_pos", (B,), torch.int32, dev)
    if sinks is not None:
        _expect(sinks, "sinks", (p.num_q_heads,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, S, p.num_q_heads, p.v_head_dim), dtype=dt, device=dev)
    _expect(out, "out", (B, S, p.num_q_heads, p.v_head_dim), dt, dev)
    cap = 0
    if k_cache is not None or v_cache is not None:
        cap = k_cache.shape[2]
        _expect(k_cache, "k_cache", (B, p.num_kv_heads, cap, p.qk_head_dim), _cdtype(p), dev)
        _expect(v_cache, "v_cache", (B, p.num_kv_heads, cap, p.v_head_dim), _cdtype(p), dev)
    need = prefill_workspace_size(p, S)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cp = p.c()
    _raise(lib().mimo_attn_prefill(ctypes.byref(cp), S, _ptr(q), _ptr(k), _ptr(v), _ptr(start_pos),
                                   _ptr(sinks), _ptr(out), _ptr(k_cache), _ptr(v_cache), cap,
                                   _ptr(workspace), wbytes, _stream(stream)))
    return out


def extend(p: Params, q, k, v, start_pos, max_start: int, k_cache, v_cache, sinks=None, out=None,
           workspace=None, stream=None):
    """mimo_attn_extend on torch device tensors: S new tokens per sequence against the cache,
    which holds each sequence's positions before start_pos[b] and receives the new tokens.

    start_pos: int32 [B] device tensor; max_start: host bound of every start_pos[b].
    Returns out [B,S,Hq,dv]."""
    B, S = q.shape[0], q.shape[1]
    dev, dt = q.device, _tdtype(p)
    if p.batch != B:
        raise ValueError(f"params.batch {p.batch} != q.shape[0] {B}")
    _expect(q, "q", (B, S, p.num_q_heads, p.qk_head_dim), dt, dev)
    _expect(k, "k", (B, S, p.num_kv_heads, p.qk_head_dim), dt, dev)
    _expect(v, "v", (B, S, p.num_kv_heads, p.v_head_dim), dt, dev)
    _expect(start_pos, "start_pos", (B,), torch.int32, dev)
    if sinks is not None:
        _expect(sinks, "sinks", (p.num_q_heads,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, S, p.num_q_heads, p.v_head_dim), dtype=dt, device=dev)
    _expect(out, "out", (B, S, p.num_q_heads, p.v_head_dim), dt, dev)
    if k_cache is None or v_cache is None:
        raise ValueError("extend needs k_cache and v_cache")
    cap = k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, p.num_kv_heads, cap, p.qk_head_dim), _cdtype(p), dev)
    _expect(v_cache, "v_cache", (B, p.num_kv_heads, cap, p.v_head_dim), _cdtype(p), dev)
    need = extend_workspace_size(p, S, max_start)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cp = p.c()
    _raise(lib().mimo_attn_extend(ctypes.byref(cp), S, _ptr(q), _ptr(k), _ptr(v), _ptr(start_pos),
                                  max_start, _ptr(sinks), _ptr(out), _ptr(k_cache), _ptr(v_cache),
                                  cap, _ptr(workspace), wbytes, _stream(stream)))
    return out


def decode(p: Params, q, k_new, v_new, positions, max_position: int, k_cache, v_cache,
           sinks=None, out=None, workspace=None, stream=None):
    """mimo_attn_decode on torch device tensors.  positions: int32 [B] device tensor."""
    B = q.shape[0]
    dev, dt = q.device, _tdtype(p)
    if p.batch != B:
        raise ValueError(f"params.batch {p.batch} != q.shape[0] {B}")
    _expect(q, "q", (B, p.num_q_heads, p.qk_head_dim), dt, dev)
    _expect(k_new, "k_new", (B, p.num_kv_heads, p.qk_head_dim), dt, dev)
    _expect(v_new, "v_new", (B, p.num_kv_heads, p.v_head_dim), dt, dev)
    _expect(positions, "positions", (B,), torch.int32, dev)
    cap = k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, p.num_kv_heads, cap, p.qk_head_dim), _cdtype(p), dev)
    _expect(v_cache, "v_cache", (B, p.num_kv_heads, cap, p.v_head_dim), _cdtype(p), dev)
    if sinks is not None:
        _expect(sinks, "sinks", (p.num_q_heads,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, p.num_q_heads, p.v_head_dim), dtype=dt, device=dev)
    _expect(out, "out", (B, p.num_q_heads, p.v_head_dim), dt, dev)
    need = decode_workspace_size(p, max_position)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cp = p.c()
    _raise(lib().mimo_attn_decode(ctypes.byref(cp), _ptr(q), _ptr(k_new), _ptr(v_new),
                                  _ptr(positions), max_position, _ptr(k_cache), _ptr(v_cache), cap,
                                  _ptr(sinks), _ptr(out), _ptr(workspace), wbytes,
                                  _stream(stream)))
    return out


def decode_noalloc_max_bytes() -> int:
    return int(lib().mimo_attn_decode_noalloc_max_bytes())


def decode_noalloc(p: Params, q, k_new, v_new, positions, max_position: int, k_cache, v_cache,
                   sinks=None, out=None, stream=None):
    """mimo_attn_decode_noalloc on torch device tensors: decode without a workspace (the library's
    own per-device scratch array holds the split partials).  out is required to be preallocated
    by callers that cannot allocate; when None it is allocated here."""
    B = q.shape[0]
    dev, dt = q.device, _tdtype(p)
    if p.batch != B:
        raise ValueError(f"params.batch {p.batch} != q.shape[0] {B}")
    _expect(q, "q", (B, p.num_q_heads, p.qk_head_dim), dt, dev)
    _expect(k_new, "k_new", (B, p.num_kv_heads, p.qk_head_dim), dt, dev)
    _expect(v_new, "v_new", (B, p.num_kv_heads, p.v_head_dim), dt, dev)
    _expect(positions, "positions", (B,), torch.int32, dev)
    cap = k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, p.num_kv_heads, cap, p.qk_head_dim), _cdtype(p), dev)
    _expect(v_cache, "v_cache", (B, p.num_kv_heads, cap, p.v_head_dim), _cdtype(p), dev)
    if sinks is not None:
        _expect(sinks, "sinks", (p.num_q_heads,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, p.num_q_heads, p.v_head_dim), dtype=dt, device=dev)
    _expect(out, "out", (B, p.num_q_heads, p.v_head_dim), dt, dev)
    cp = p.c()
    _raise(lib().mimo_attn_decode_noalloc(ctypes.byref(cp), _ptr(q), _ptr(k_new), _ptr(v_new),
                                          _ptr(positions), max_position, _ptr(k_cache),
                                          _ptr(v_cache), cap, _ptr(sinks), _ptr(out),
                                          _stream(stream)))
    return out


def layer_workspace_size(p: Params, hidden: int, seq_len: int) -> int:
    cp = p.c()
    return int(lib().mimo_attn_layer_workspace_size(ctypes.byref(cp), hidden, seq_len))


def layer_prefill(p: Params, x, w_q, w_k, w_v, w_o, start_pos, sinks=None, out=None, k_cache=None,
                  v_cache=None, workspace=None, stream=None):
    """mimo_attn_layer_prefill on torch device tensors: x [B,S,hidden]; w_q [hidden, Hq*dqk],
    w_k [hidden, Hkv*dqk], w_v [hidden, Hkv*dv], w_o [Hq*dv, out_dim] (bf16).  Returns
    out [B,S,out_dim]."""
    B, S, hidden = x.shape
    dev, dt = x.device, _tdtype(p)
    if p.batch != B:
        raise ValueError(f"params.batch {p.batch} != x.shape[0] {B}")
    _expect(x, "x", (B, S, hidden), dt, dev)
    _expect(w_q, "w_q", (hidden, p.num_q_heads * p.qk_head_dim), dt, dev)
    _expect(w_k, "w_k", (hidden, p.num_kv_heads * p.qk_head_dim), dt, dev)
    _expect(w_v, "w_v", (hidden, p.num_kv_heads * p.v_head_dim), dt, dev)
    if w_o is None or w_o.dim() != 2:
        raise ValueError("w_o must be a [Hq*dv, out_dim] matrix")
    out_dim = w_o.shape[1]
    _expect(w_o, "w_o", (p.num_q_heads * p.v_head_dim, out_dim), dt, dev)
    _expect(start_pos, "start_pos", (B,), torch.int32, dev)
    if sinks is not None:
        _expect(sinks, "sinks", (p.num_q_heads,), torch.float32, dev)
    if out is None:
        out = torch.empty((B, S, out_dim), dtype=dt, device=dev)
    _expect(out, "out", (B, S, out_dim), dt, dev)
    cap = 0
    if k_cache is not None or v_cache is not None:
        cap = k_cache.shape[2]
        _expect(k_cache, "k_cache", (B, p.num_kv_heads, cap, p.qk_head_dim), _cdtype(p), dev)
        _expect(v_cache, "v_cache", (B, p.num_kv_heads, cap, p.v_head_dim), _cdtype(p), dev)
    need = layer_workspace_size(p, hidden, S)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cp = p.c()
    _raise(lib().mimo_attn_layer_prefill(
        ctypes.byref(cp), hidden, S, _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), out_dim,
        _ptr(start_pos), _ptr(sinks), _ptr(out), _ptr(k_cache), _ptr(v_cache), cap,
        _ptr(workspace), wbytes, _stream(stream)))
    return out


def router_check_params(p: RouterParams, num_tokens: int = 1) -> int:
    cp = p.c(num_tokens)
    return lib().mimo_router_check_params(ctypes.byref(cp))


def router_topk(p: RouterParams, logits, bias=None, expert_idx=None, weights=None, stream=None):
    """mimo_router_topk on torch device tensors: logits fp32 [T, E], bias fp32 [E] or None.
    Returns (expert_idx int32 [T, top_k], weights fp32 [T, top_k])."""
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    dev = logits.device
    if E != p.num_experts:
        raise ValueError(f"logits have {E} experts, params {p.num_experts}")
    _expect(logits, "logits", (T, E), torch.float32, dev)
    if bias is not None:
        _expect(bias, "bias", (E,), torch.float32, dev)
    if expert_idx is None:
        expert_idx = torch.empty((T, p.top_k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((T, p.top_k), dtype=torch.float32, device=dev)
    _expect(expert_idx, "expert_idx", (T, p.top_k), torch.int32, dev)
    _expect(weights, "weights", (T, p.top_k), torch.float32, dev)
    cp = p.c(T)
    _raise(lib().mimo_router_topk(ctypes.byref(cp), _ptr(logits), _ptr(bias), _ptr(expert_idx),
                                  _ptr(weights), _stream(stream)))
    return expert_idx, weights
