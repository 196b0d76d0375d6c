"""Per-layer dispatch of the hybrid attention stack from ``hybrid_layer_pattern``.

Pages:
  * "add Xiaomi MiMo v2 (mimo_v2_flash)" (mlxcel issue 842), "Architecture, verified against
    upstream": an explicit hybrid_layer_pattern list chooses the kind (1 = sliding window, else
    global); the window is sliding_window_size; theta is swa_rope_theta on sliding layers and
    rope_theta otherwise; the rotated width is int(partial_rotary_factor * head_dim), where the
    factor may arrive typed as an int and is parsed defensively.  "Implementation plan": sliding
    layers keep a rotating cache.
  * "Add Xiaomi MiMo-V2" (transformers PR 45144), "Additional useful info": KV-group count per
    kind, V head dim separate from the QK head dim, value scale sqrt(hidden / (heads * v_head_dim)),
    sinks on sliding layers only.

The two KV-head counts are named ``num_key_value_heads`` (global) and ``swa_num_key_value_heads``
(sliding) here; the pages state that they differ but do not name the fields.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

from .binding import BF16, LAYER_GLOBAL, LAYER_SWA, Params


def rope_dims_from_factor(partial_rotary_factor, head_dim: int) -> int:
    """int(partial_rotary_factor * head_dim), with the factor accepted as int, float or string."""
    f = float(partial_rotary_factor)
    if not (0.0 <= f <= 1.0):
        raise ValueError(f"partial_rotary_factor {partial_rotary_factor!r} outside [0, 1]")
    return int(f * head_dim)


@dataclasses.dataclass
class HybridAttentionConfig:
    hidden_size: int
    num_attention_heads: int
    num_key_value_heads: int          # global layers
    swa_num_key_value_heads: int      # sliding-window layers
    head_dim: int                     # QK head dim
    v_head_dim: int
    partial_rotary_factor: float
    rope_theta: float
    swa_rope_theta: float
    sliding_window_size: int
    hybrid_layer_pattern: Sequence[int]
    rope_dims: Optional[int] = None   # explicit override of the rotated width

    @property
    def rotated_dims(self) -> int:
        return self.rope_dims if self.rope_dims is not None else rope_dims_from_factor(
            self.partial_rotary_factor, self.head_dim)

    @property
    def v_scale(self) -> float:
        return math.sqrt(self.hidden_size / (self.num_attention_heads * self.v_head_dim))


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    index: int
    kind: int                 # LAYER_GLOBAL or LAYER_SWA
    rope_theta: float
    num_kv_heads: int
    window: int               # 0 on global layers
    has_sinks: bool           # sliding layers only
    cache: str                # "ring" (sliding) or "linear" (global)

    def params(self, cfg: HybridAttentionConfig, batch: int, dtype: int = BF16) -> Params:
        return Params(batch=batch, num_q_heads=cfg.num_attention_heads,
                      num_kv_heads=self.num_kv_heads, qk_head_dim=cfg.head_dim,
                      v_head_dim=cfg.v_head_dim, rope_dims=cfg.rotated_dims,
                      layer_kind=self.kind, window=self.window, rope_theta=self.rope_theta,
                      v_scale=cfg.v_scale, softmax_scale=0.0, dtype=dtype)


def layer_spec(cfg: HybridAttentionConfig, index: int) -> LayerSpec:
    sliding = int(cfg.hybrid_layer_pattern[index]) == 1
    if sliding:
        return LayerSpec(index, LAYER_SWA, float(cfg.swa_rope_theta), cfg.swa_num_key_value_heads,
                         int(cfg.sliding_window_size), True, "ring")
    return LayerSpec(index, LAYER_GLOBAL, float(cfg.rope_theta), cfg.num_key_value_heads, 0,
                     False, "linear")


def layer_specs(cfg: HybridAttentionConfig) -> list[LayerSpec]:
    return [layer_spec(cfg, i) for i in range(len(cfg.hybrid_layer_pattern))]
