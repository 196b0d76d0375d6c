"""ctypes binding of the fp64 oracle (``mimo_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the benchmark).

Every array argument is converted to a C-contiguous float32 (inputs: bf16 and fp32 values are
exact in float32) or int32 array; results are float64 numpy arrays.  Errors raise ValueError.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mimo_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "router_oracle.c")]
_LIB = os.path.join(_HERE, "libmimo_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE fp64: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or any(
            os.path.getmtime(_LIB) < os.path.getmtime(f) for f in _SRCS):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             *_SRCS, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _CParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("qk_head_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
        ("layer_kind", ctypes.c_int32), ("window", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("v_scale", ctypes.c_double),
        ("softmax_scale", ctypes.c_double),
    ]


@dataclasses.dataclass
class OracleParams:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    qk_head_dim: int
    v_head_dim: int
    rope_dims: int
    layer_kind: int  # 0 global causal, 1 sliding window
    window: int
    rope_theta: float
    v_scale: float = 1.0
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(qk_head_dim)

    def c(self) -> _CParams:
        return _CParams(self.batch, self.num_q_heads, self.num_kv_heads, self.qk_head_dim,
                        self.v_head_dim, self.rope_dims, self.layer_kind, self.window,
                        float(self.rope_theta), float(self.v_scale), float(self.softmax_scale))


class _CRouterParams(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_double),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.POINTER
            f32, f64, i32 = P(ctypes.c_float), P(ctypes.c_double), P(ctypes.c_int32)
            lib.oracle_rope_omega.argtypes = [ctypes.c_int32, ctypes.c_double, f64]
            lib.oracle_rope_rotate.argtypes = [f64, f64, ctypes.c_int64, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_double, i32]
            lib.oracle_prefill.argtypes = [P(_CParams), ctypes.c_int32, f32, f32, f32, i32, f32,
                                           f64, i32, ctypes.c_int32, f64]
            lib.oracle_prefill_f64.argtypes = [P(_CParams), ctypes.c_int32, f64, f64, f64, i32,
                                               f32, f64, i32, ctypes.c_int32, f64]
            lib.oracle_scores.argtypes = [P(_CParams), ctypes.c_int32, f32, f32, i32,
                                          ctypes.c_int32, ctypes.c_int32, f64]
            lib.oracle_decode.argtypes = [P(_CParams), f32, f32, f32, i32, f32, f32, i32, i32,
                                          ctypes.c_int32, f32, f64, f64, i32, ctypes.c_int32]
            lib.oracle_extend.argtypes = [P(_CParams), ctypes.c_int32, f32, f32, f32, i32, f32,
                                          f32, i32, i32, ctypes.c_int32, f32, f64, i32,
                                          ctypes.c_int32, f64]
            u8 = P(ctypes.c_uint8)
            lib.oracle_e4m3_encode.argtypes = [f32, ctypes.c_int64, ctypes.c_float, u8]
            lib.oracle_e4m3_decode.argtypes = [u8, ctypes.c_int64, ctypes.c_double, f64]
            lib.oracle_decode_fp8.argtypes = [P(_CParams), f32, f32, f32, i32, u8, u8, i32, i32,
                                              ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                              f32, f64, f64, u8, u8, i32, ctypes.c_int32]
            lib.oracle_router.argtypes = [P(_CRouterParams), f32, f32, i32, f64]
            lib.oracle_router_sigmoid.argtypes = [ctypes.c_float]
            lib.oracle_router_sigmoid.restype = ctypes.c_float
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            for fn in ("oracle_rope_omega", "oracle_rope_rotate", "oracle_prefill",
                       "oracle_scores", "oracle_decode", "oracle_extend", "oracle_e4m3_encode",
                       "oracle_e4m3_decode", "oracle_decode_fp8", "oracle_prefill_f64",
                       "oracle_router"):
                getattr(lib, fn).restype = ctypes.c_int
            _lib = lib
    return _lib


def _f32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def _u8(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def omega(rope_dims: int, theta: float) -> np.ndarray:
    out = np.zeros(max(rope_dims // 2, 1), dtype=np.float64)
    _check(_load().oracle_rope_omega(rope_dims, theta, _ptr(out, ctypes.c_double)), "omega")
    return out[: rope_dims // 2]


def rotate(x, rope_dims: int, theta: float, positions) -> np.ndarray:
    """Rotate rows x[..., dim] at positions[...] (same leading shape)."""
    x = _f64(x)
    pos = _i32(positions)
    assert pos.shape == x.shape[:-1]
    y = np.empty_like(x)
    n = int(np.prod(x.shape[:-1]))
    _check(_load().oracle_rope_rotate(_ptr(x, ctypes.c_double), _ptr(y, ctypes.c_double), n,
                                      x.shape[-1], rope_dims, theta, _ptr(pos, ctypes.c_int32)),
           "rotate")
    return y


def prefill(p: OracleParams, q, k, v, positions, sinks=None, rows=None, want_k_rot=False):
    """Attention over S new tokens: q [B,S,Hq,dqk], k [B,S,Hkv,dqk], v [B,S,Hkv,dv],
    positions [B,S], sinks [Hq] or None.  Returns out [B,S,Hq,dv] (rows not listed are NaN),
    plus the rotated keys [B,S,Hkv,dqk] when want_k_rot."""
    q, k, v, sinks = _f32(q), _f32(k), _f32(v), _f32(sinks)
    pos = _i32(positions)
    B, S = pos.shape
    assert q.shape == (B, S, p.num_q_heads, p.qk_head_dim), q.shape
    assert k.shape == (B, S, p.num_kv_heads, p.qk_head_dim), k.shape
    assert v.shape == (B, S, p.num_kv_heads, p.v_head_dim), v.shape
    out = np.full((B, S, p.num_q_heads, p.v_head_dim), np.nan, dtype=np.float64)
    rows_a = _i32(rows)
    krot = np.empty(k.shape, dtype=np.float64) if want_k_rot else None
    cp = p.c()
    _check(_load().oracle_prefill(
        ctypes.byref(cp), S, _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
        _ptr(v, ctypes.c_float), _ptr(pos, ctypes.c_int32), _ptr(sinks, ctypes.c_float),
        _ptr(out, ctypes.c_double), _ptr(rows_a, ctypes.c_int32),
        0 if rows_a is None else len(rows_a), _ptr(krot, ctypes.c_double)), "prefill")
    return (out, krot) if want_k_rot else out


def scores(p: OracleParams, q, k, positions, b: int, h: int) -> np.ndarray:
    """Unmasked scaled score matrix [S,S] of sequence b, query head h."""
    q, k = _f32(q), _f32(k)
    pos = _i32(positions)
    S = pos.shape[1]
    z = np.empty((S, S), dtype=np.float64)
    cp = p.c()
    _check(_load().oracle_scores(ctypes.byref(cp), S, _ptr(q, ctypes.c_float),
                                 _ptr(k, ctypes.c_float), _ptr(pos, ctypes.c_int32), b, h,
                                 _ptr(z, ctypes.c_double)), "scores")
    return z


def decode(p: OracleParams, q, k_new, v_new, pos, kc=None, vc=None, kpos=None, count=None,
           sinks=None, batch_rows=None, want_k_rot=False):
    """One new token per sequence against a position->(rotated key, value) map.

    q [B,Hq,dqk], k_new [B,Hkv,dqk] (raw), v_new [B,Hkv,dv], pos [B];
    kc [B,Hkv,L,dqk] rotated keys, vc [B,Hkv,L,dv], kpos [B,L], count [B] (or None for L=0).
    Returns out [B,Hq,dv] (sequences not listed in batch_rows are NaN), plus the rotated new
    keys [B,Hkv,dqk] when want_k_rot."""
    q, k_new, v_new, sinks = _f32(q), _f32(k_new), _f32(v_new), _f32(sinks)
    pos = _i32(pos)
    B = pos.shape[0]
    assert q.shape == (B, p.num_q_heads, p.qk_head_dim)
    assert k_new.shape == (B, p.num_kv_heads, p.qk_head_dim)
    assert v_new.shape == (B, p.num_kv_heads, p.v_head_dim)
    if kc is None:
        L = 0
        kc_a = vc_a = kpos_a = cnt_a = None
    else:
        kc_a, vc_a, kpos_a, cnt_a = _f32(kc), _f32(vc), _i32(kpos), _i32(count)
        L = kc_a.shape[2]
        assert kc_a.shape == (B, p.num_kv_heads, L, p.qk_head_dim)
        assert vc_a.shape == (B, p.num_kv_heads, L, p.v_head_dim)
        assert kpos_a.shape == (B, L) and cnt_a.shape == (B,)
    out = np.full((B, p.num_q_heads, p.v_head_dim), np.nan, dtype=np.float64)
    krot = np.full(k_new.shape, np.nan, dtype=np.float64) if want_k_rot else None
    br = _i32(batch_rows)
    cp = p.c()
    _check(_load().oracle_decode(
        ctypes.byref(cp), _ptr(q, ctypes.c_float), _ptr(k_new, ctypes.c_float),
        _ptr(v_new, ctypes.c_float), _ptr(pos, ctypes.c_int32), _ptr(kc_a, ctypes.c_float),
        _ptr(vc_a, ctypes.c_float), _ptr(kpos_a, ctypes.c_int32), _ptr(cnt_a, ctypes.c_int32), L,
        _ptr(sinks, ctypes.c_float), _ptr(out, ctypes.c_double), _ptr(krot, ctypes.c_double),
        _ptr(br, ctypes.c_int32), 0 if br is None else len(br)), "decode")
    return (out, krot) if want_k_rot else out


def extend(p: OracleParams, q, k, v, start, kc=None, vc=None, kpos=None, count=None, sinks=None,
           rows=None, want_k_rot=False):
    """Chunked prefill: S new tokens per sequence (positions start[b] + i) against a
    position->(rotated key, value) map of earlier tokens.

    q [B,S,Hq,dqk], k [B,S,Hkv,dqk] (raw), v [B,S,Hkv,dv], start [B];
    kc [B,Hkv,L,dqk] rotated keys, vc [B,Hkv,L,dv], kpos [B,L], count [B] (or None for L=0).
    Returns out [B,S,Hq,dv] (rows not listed are NaN), plus the rotated new keys [B,S,Hkv,dqk]
    when want_k_rot."""
    q, k, v, sinks = _f32(q), _f32(k), _f32(v), _f32(sinks)
    st = _i32(start)
    B, S = q.shape[0], q.shape[1]
    assert st.shape == (B,)
    assert q.shape == (B, S, p.num_q_heads, p.qk_head_dim), q.shape
    assert k.shape == (B, S, p.num_kv_heads, p.qk_head_dim), k.shape
    assert v.shape == (B, S, p.num_kv_heads, p.v_head_dim), v.shape
    if kc is None:
        L = 0
        kc_a = vc_a = kpos_a = cnt_a = None
    else:
        kc_a, vc_a, kpos_a, cnt_a = _f32(kc), _f32(vc), _i32(kpos), _i32(count)
        L = kc_a.shape[2]
        assert kc_a.shape == (B, p.num_kv_heads, L, p.qk_head_dim)
        assert vc_a.shape == (B, p.num_kv_heads, L, p.v_head_dim)
        assert kpos_a.shape == (B, L) and cnt_a.shape == (B,)
    out = np.full((B, S, p.num_q_heads, p.v_head_dim), np.nan, dtype=np.float64)
    rows_a = _i32(rows)
    krot = np.empty(k.shape, dtype=np.float64) if want_k_rot else None
    cp = p.c()
    _check(_load().oracle_extend(
        ctypes.byref(cp), S, _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
        _ptr(v, ctypes.c_float), _ptr(st, ctypes.c_int32), _ptr(kc_a, ctypes.c_float),
        _ptr(vc_a, ctypes.c_float), _ptr(kpos_a, ctypes.c_int32), _ptr(cnt_a, ctypes.c_int32), L,
        _ptr(sinks, ctypes.c_float), _ptr(out, ctypes.c_double), _ptr(rows_a, ctypes.c_int32),
        0 if rows_a is None else len(rows_a), _ptr(krot, ctypes.c_double)), "extend")
    return (out, krot) if want_k_rot else out


# ----------------------------------------------------------------------------- fp8 KV cache


def e4m3_encode(x, inv_scale: float = 1.0) -> np.ndarray:
    """e4m3 codes (uint8) of fp32(x) * fp32(inv_scale), clamped to +-448, nearest, ties even."""
    xa = _f32(x)
    out = np.empty(xa.shape, dtype=np.uint8)
    _check(_load().oracle_e4m3_encode(_ptr(xa, ctypes.c_float), xa.size, float(inv_scale),
                                      _ptr(out, ctypes.c_uint8)), "e4m3_encode")
    return out


def e4m3_decode(codes, scale: float = 1.0) -> np.ndarray:
    """Stored values code -> e4m3(code) * scale (float64; NaN codes give NaN)."""
    ca = _u8(codes)
    out = np.empty(ca.shape, dtype=np.float64)
    _check(_load().oracle_e4m3_decode(_ptr(ca, ctypes.c_uint8), ca.size, float(scale),
                                      _ptr(out, ctypes.c_double)), "e4m3_decode")
    return out


def decode_fp8(p: OracleParams, q, k_new, v_new, pos, kc8=None, vc8=None, kpos=None, count=None,
               k_scale: float = 1.0, v_scale: float = 1.0, sinks=None, batch_rows=None):
    """decode() against fp8 caches: kc8 [B,Hkv,L,dqk] / vc8 [B,Hkv,L,dv] e4m3 codes with one
    scale each; the new token is quantized as the cache stores it before it is attended.

    Returns (out [B,Hq,dv], rotated new keys [B,Hkv,dqk] (exact, before quantization),
    new key codes [B,Hkv,dqk], new value codes [B,Hkv,dv])."""
    q, k_new, v_new, sinks = _f32(q), _f32(k_new), _f32(v_new), _f32(sinks)
    pos = _i32(pos)
    B = pos.shape[0]
    assert q.shape == (B, p.num_q_heads, p.qk_head_dim)
    assert k_new.shape == (B, p.num_kv_heads, p.qk_head_dim)
    assert v_new.shape == (B, p.num_kv_heads, p.v_head_dim)
    if kc8 is None:
        L = 0
        kc_a = vc_a = kpos_a = cnt_a = None
    else:
        kc_a, vc_a, kpos_a, cnt_a = _u8(kc8), _u8(vc8), _i32(kpos), _i32(count)
        L = kc_a.shape[2]
        assert kc_a.shape == (B, p.num_kv_heads, L, p.qk_head_dim)
        assert vc_a.shape == (B, p.num_kv_heads, L, p.v_head_dim)
        assert kpos_a.shape == (B, L) and cnt_a.shape == (B,)
    out = np.full((B, p.num_q_heads, p.v_head_dim), np.nan, dtype=np.float64)
    krot = np.full(k_new.shape, np.nan, dtype=np.float64)
    kcode = np.zeros(k_new.shape, dtype=np.uint8)
    vcode = np.zeros(v_new.shape, dtype=np.uint8)
    br = _i32(batch_rows)
    cp = p.c()
    _check(_load().oracle_decode_fp8(
        ctypes.byref(cp), _ptr(q, ctypes.c_float), _ptr(k_new, ctypes.c_float),
        _ptr(v_new, ctypes.c_float), _ptr(pos, ctypes.c_int32), _ptr(kc_a, ctypes.c_uint8),
        _ptr(vc_a, ctypes.c_uint8), _ptr(kpos_a, ctypes.c_int32), _ptr(cnt_a, ctypes.c_int32), L,
        float(k_scale), float(v_scale), _ptr(sinks, ctypes.c_float), _ptr(out, ctypes.c_double),
        _ptr(krot, ctypes.c_double), _ptr(kcode, ctypes.c_uint8), _ptr(vcode, ctypes.c_uint8),
        _ptr(br, ctypes.c_int32), 0 if br is None else len(br)), "decode_fp8")
    return out, krot, kcode, vcode


# ----------------------------------------------------------------------------- layer


def prefill_f64(p: OracleParams, q, k, v, positions, sinks=None, rows=None):
    """prefill() with q, k, v taken in float64 (no rounding of the inputs)."""
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f32(sinks)
    pos = _i32(positions)
    B, S = pos.shape
    assert q.shape == (B, S, p.num_q_heads, p.qk_head_dim), q.shape
    assert k.shape == (B, S, p.num_kv_heads, p.qk_head_dim), k.shape
    assert v.shape == (B, S, p.num_kv_heads, p.v_head_dim), v.shape
    out = np.full((B, S, p.num_q_heads, p.v_head_dim), np.nan, dtype=np.float64)
    rows_a = _i32(rows)
    cp = p.c()
    _check(_load().oracle_prefill_f64(
        ctypes.byref(cp), S, _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
        _ptr(v, ctypes.c_double), _ptr(pos, ctypes.c_int32), _ptr(sinks, ctypes.c_float),
        _ptr(out, ctypes.c_double), _ptr(rows_a, ctypes.c_int32),
        0 if rows_a is None else len(rows_a), None), "prefill_f64")
    return out


def layer_prefill(p: OracleParams, x, wq, wk, wv, wo, positions, sinks=None, rows=None):
    """The attention layer with its projections, in fp64:
    q = x Wq, k = x Wk, v = x Wv (x [B,S,hidden]; Wq [hidden, Hq*dqk], Wk [hidden, Hkv*dqk],
    Wv [hidden, Hkv*dv], heads contiguous in the columns), attention as prefill() (v_scale
    included), out = attn Wo (attn [B,S,Hq*dv], Wo [Hq*dv, hidden_out]).  Matrix products are
    numpy's fp64 matmul.  Returns out [B,S,hidden_out] (rows not listed are NaN)."""
    x = _f64(x)
    B, S, H = x.shape
    wq, wk, wv, wo = _f64(wq), _f64(wk), _f64(wv), _f64(wo)
    assert wq.shape == (H, p.num_q_heads * p.qk_head_dim), wq.shape
    assert wk.shape == (H, p.num_kv_heads * p.qk_head_dim), wk.shape
    assert wv.shape == (H, p.num_kv_heads * p.v_head_dim), wv.shape
    assert wo.shape[0] == p.num_q_heads * p.v_head_dim, wo.shape
    q = (x @ wq).reshape(B, S, p.num_q_heads, p.qk_head_dim)
    k = (x @ wk).reshape(B, S, p.num_kv_heads, p.qk_head_dim)
    v = (x @ wv).reshape(B, S, p.num_kv_heads, p.v_head_dim)
    attn = prefill_f64(p, q, k, v, positions, sinks, rows).reshape(B, S, -1)
    out = np.full((B, S, wo.shape[1]), np.nan, dtype=np.float64)
    sel = np.arange(S) if rows is None else np.asarray(rows)
    out[:, sel] = attn[:, sel] @ wo
    return out


# ----------------------------------------------------------------------------- MoE router


@dataclasses.dataclass
class RouterParams:
    num_experts: int = 256
    n_group: int = 8
    topk_group: int = 4
    top_k: int = 8
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 1.0


def router(p: RouterParams, logits, bias=None):
    """Grouped sigmoid top-k routing of logits [T, E] (float32) with an optional correction bias
    [E].  Returns (expert indices int32 [T, top_k] in rank order, weights float64 [T, top_k])."""
    x = _f32(logits)
    T, E = x.shape
    assert E == p.num_experts
    b = _f32(bias)
    idx = np.zeros((T, p.top_k), np.int32)
    w = np.zeros((T, p.top_k), np.float64)
    cp = _CRouterParams(T, E, p.n_group, p.topk_group, p.top_k, int(p.norm_topk_prob),
                        float(p.routed_scaling_factor))
    _check(_load().oracle_router(ctypes.byref(cp), _ptr(x, ctypes.c_float), _ptr(b, ctypes.c_float),
                                 _ptr(idx, ctypes.c_int32), _ptr(w, ctypes.c_double)), "router")
    return idx, w


def router_sigmoid(x: float) -> float:
    """The float32 score of one logit (fp64 sigmoid rounded to fp32)."""
    return float(_load().oracle_router_sigmoid(float(x)))
