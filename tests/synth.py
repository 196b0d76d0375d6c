"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds shapes and random draws only; none of the layer's arithmetic lives here, so the
oracle side and the HIP side both take their inputs from it without sharing any computation.

Recipe: ``torch.Generator`` seeded per (workload, layer), values drawn as float32 N(0,1) in the
fixed order q, k, v, sinks, then cast round-to-nearest-even to bf16 (fp32 workloads stay fp32).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    num_q_heads: int
    num_kv_heads: int
    qk_head_dim: int
    v_head_dim: int
    rope_dims: int
    rope_theta: float
    layer_kind: int  # 0 global causal, 1 sliding window
    window: int
    sinks: bool
    hidden: int
    dtype: torch.dtype

    @property
    def v_scale(self) -> float:
        return math.sqrt(self.hidden / (self.num_q_heads * self.v_head_dim))


# Head configurations of the two layer kinds at full size (hidden 4096, 64 query heads,
# QK head dim 192 with 64 rotated dims, V head dim 128).
SWA_HEADS = dict(num_q_heads=64, num_kv_heads=8, qk_head_dim=192, v_head_dim=128, rope_dims=64,
                 rope_theta=1.0e4, layer_kind=1, window=128, sinks=True, hidden=4096)
GA_HEADS = dict(num_q_heads=64, num_kv_heads=4, qk_head_dim=192, v_head_dim=128, rope_dims=64,
                rope_theta=5.0e6, layer_kind=0, window=0, sinks=False, hidden=4096)

TINY_SWA = Workload("tiny_swa_fp32", batch=1, seq=64, num_q_heads=4, num_kv_heads=1,
                    qk_head_dim=32, v_head_dim=16, rope_dims=int(0.33 * 32), rope_theta=1.0e4,
                    layer_kind=1, window=16, sinks=True, hidden=64, dtype=torch.float32)
SWA_PREFILL = Workload("swa_prefill_s4096", batch=1, seq=4096, dtype=torch.bfloat16, **SWA_HEADS)
GA_PREFILL = Workload("ga_prefill_s8192", batch=1, seq=8192, dtype=torch.bfloat16, **GA_HEADS)

DECODE_BATCH = 64
DECODE_MIN_LEN, DECODE_MAX_LEN = 1024, 32768
STACK_LAYERS, STACK_BATCH, STACK_SEQ, STACK_DECODE_STEPS = 48, 2, 16384, 256


def stack_pattern(n_layers: int = STACK_LAYERS) -> list[int]:
    """hybrid_layer_pattern of the 48-layer stack: layer 0 global, then 5 sliding : 1 global."""
    return [0 if l % 6 == 0 else 1 for l in range(n_layers)]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, g: torch.Generator, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dtype)


def layer_inputs(w: Workload, seed: int, device="cpu", batch=None, seq=None):
    """q [B,S,Hq,dqk], k [B,S,Hkv,dqk], v [B,S,Hkv,dv], sinks fp32 [Hq] or None."""
    B = w.batch if batch is None else batch
    S = w.seq if seq is None else seq
    g = _gen(seed, device)
    q = randn((B, S, w.num_q_heads, w.qk_head_dim), g, w.dtype, device)
    k = randn((B, S, w.num_kv_heads, w.qk_head_dim), g, w.dtype, device)
    v = randn((B, S, w.num_kv_heads, w.v_head_dim), g, w.dtype, device)
    sinks = randn((w.num_q_heads,), g, torch.float32, device) if w.sinks else None
    return q, k, v, sinks


def cache_contents(w: Workload, seed: int, batch: int, cache_capacity: int, device="cpu"):
    """Cache contents k_cache [B,Hkv,cap,dqk], v_cache [B,Hkv,cap,dv] drawn N(0,1) (the cache
    holds keys that are already rotated, so any draw is a valid cache state)."""
    g = _gen(seed, device)
    k_cache = randn((batch, w.num_kv_heads, cache_capacity, w.qk_head_dim), g, w.dtype, device)
    v_cache = randn((batch, w.num_kv_heads, cache_capacity, w.v_head_dim), g, w.dtype, device)
    return k_cache, v_cache


def layer_weights(w: Workload, seed: int, hidden: int, out_dim: int, device="cpu"):
    """Projection weights of the layer, drawn N(0, 1/fan_in) (so projected activations stay about
    unit scale): w_q [hidden, Hq*dqk], w_k [hidden, Hkv*dqk], w_v [hidden, Hkv*dv],
    w_o [Hq*dv, out_dim], in the workload dtype."""
    g = _gen(seed, device)
    mk = lambda r, c: (torch.randn((r, c), generator=g, dtype=torch.float32, device=device)
                       / math.sqrt(r)).to(w.dtype)
    return (mk(hidden, w.num_q_heads * w.qk_head_dim), mk(hidden, w.num_kv_heads * w.qk_head_dim),
            mk(hidden, w.num_kv_heads * w.v_head_dim), mk(w.num_q_heads * w.v_head_dim, out_dim))


def layer_input(w: Workload, seed: int, hidden: int, device="cpu", batch=None, seq=None):
    """Layer input x [B,S,hidden] drawn N(0,1) and its sinks (fp32 [Hq] or None)."""
    B = w.batch if batch is None else batch
    S = w.seq if seq is None else seq
    g = _gen(seed, device)
    x = randn((B, S, hidden), g, w.dtype, device)
    sinks = randn((w.num_q_heads,), g, torch.float32, device) if w.sinks else None
    return x, sinks


ROUTER_TOKENS = 2 * 16384   # one router call per MoE layer of the stack's prefill batch


def router_inputs(seed: int, tokens: int, experts: int = 256, device="cpu", bias_sd: float = 0.1):
    """Gate logits [T, E] drawn N(0, 4) (fp32) and a correction bias [E] drawn N(0, bias_sd^2)."""
    g = _gen(seed, device)
    logits = torch.randn((tokens, experts), generator=g, dtype=torch.float32, device=device) * 2
    bias = torch.randn((experts,), generator=g, dtype=torch.float32, device=device) * bias_sd
    return logits, bias


# fp8 cache scales of the synthetic fp8 workloads (the stored values come out about N(0,1))
FP8_K_SCALE, FP8_V_SCALE = 1.0 / 16.0, 1.0 / 8.0


def fp8_cache_contents(w: Workload, seed: int, batch: int, cache_capacity: int, device="cpu",
                       k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE):
    """fp8 cache contents as uint8 e4m3 codes [B,Hkv,cap,dqk] / [B,Hkv,cap,dv]: N(0,1) draws
    divided by the scale, turned into codes by torch's float8_e4m3fn conversion (random codes whose
    stored values are about N(0,1); any code pattern is a valid cache state)."""
    g = _gen(seed, device)
    k = torch.randn((batch, w.num_kv_heads, cache_capacity, w.qk_head_dim), generator=g,
                    dtype=torch.float32, device=device) / k_scale
    v = torch.randn((batch, w.num_kv_heads, cache_capacity, w.v_head_dim), generator=g,
                    dtype=torch.float32, device=device) / v_scale
    code = lambda t: t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return code(k), code(v)


def decode_lengths(seed: int, batch: int = DECODE_BATCH, lo: int = DECODE_MIN_LEN,
                   hi: int = DECODE_MAX_LEN) -> torch.Tensor:
    """Tokens already cached per sequence, uniform in [lo, hi] inclusive (host int32)."""
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)


def decode_inputs(w: Workload, seed: int, batch: int, cache_capacity: int, device="cpu"):
    """One decode step: q [B,Hq,dqk], k_new/v_new [B,Hkv,d], sinks, and cache contents
    k_cache [B,Hkv,cap,dqk], v_cache [B,Hkv,cap,dv] drawn N(0,1) (the cache holds keys that are
    already rotated, so any draw is a valid cache state)."""
    g = _gen(seed, device)
    q = randn((batch, w.num_q_heads, w.qk_head_dim), g, w.dtype, device)
    k_new = randn((batch, w.num_kv_heads, w.qk_head_dim), g, w.dtype, device)
    v_new = randn((batch, w.num_kv_heads, w.v_head_dim), g, w.dtype, device)
    sinks = randn((w.num_q_heads,), g, torch.float32, device) if w.sinks else None
    k_cache = randn((batch, w.num_kv_heads, cache_capacity, w.qk_head_dim), g, w.dtype, device)
    v_cache = randn((batch, w.num_kv_heads, cache_capacity, w.v_head_dim), g, w.dtype, device)
    return q, k_new, v_new, sinks, k_cache, v_cache
