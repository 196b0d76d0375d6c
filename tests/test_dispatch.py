"""Per-layer dispatch from hybrid_layer_pattern (host logic, CPU).

Fixtures in tests/golden/ hold what the pages (and the workload description) fix: the interleave
rule, the theta selection and the rotated-width formula.
"""
import json
import math
import os

import pytest

import global_attention_rope_amd as mimo
from global_attention_rope_amd import layers
from tests import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _full_config(pattern):
    return mimo.HybridAttentionConfig(
        hidden_size=4096, num_attention_heads=64, num_key_value_heads=4, swa_num_key_value_heads=8,
        head_dim=192, v_head_dim=128, partial_rotary_factor=1.0 / 3.0, rope_theta=5e6,
        swa_rope_theta=1e4, sliding_window_size=128, hybrid_layer_pattern=pattern)


def test_golden_dispatch_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "dispatch.json")))
    for case in fx["rope_dims"]:
        assert mimo.rope_dims_from_factor(case["partial_rotary_factor"], case["head_dim"]) == \
            case["rope_dims"], case
    pattern = synth.stack_pattern(fx["stack"]["layers"])
    specs = mimo.layer_specs(_full_config(pattern))
    ga = [s.index for s in specs if s.kind == mimo.LAYER_GLOBAL]
    assert ga == fx["stack"]["global_layers"]
    assert sum(1 for s in specs if s.kind == mimo.LAYER_SWA) == fx["stack"]["sliding_layer_count"]
    for s in specs:
        sel = fx["theta_selection"]["sliding" if s.kind == mimo.LAYER_SWA else "global"]
        assert s.rope_theta == sel["theta"]
        assert s.has_sinks == sel["sinks"]
        assert s.cache == sel["cache"]
        assert s.num_kv_heads == sel["kv_heads"]
        assert s.window == sel["window"]


def test_pattern_value_one_means_sliding_anything_else_global():
    cfg = _full_config([1, 0, 1, 1, 0])
    kinds = [s.kind for s in mimo.layer_specs(cfg)]
    assert kinds == [1, 0, 1, 1, 0]


def test_params_from_spec():
    cfg = _full_config(synth.stack_pattern())
    p0 = mimo.layer_spec(cfg, 0).params(cfg, batch=2)
    p1 = mimo.layer_spec(cfg, 1).params(cfg, batch=2)
    assert (p0.layer_kind, p0.num_kv_heads, p0.window, p0.rope_theta) == (0, 4, 0, 5e6)
    assert (p1.layer_kind, p1.num_kv_heads, p1.window, p1.rope_theta) == (1, 8, 128, 1e4)
    assert p0.rope_dims == p1.rope_dims == 64
    assert math.isclose(p0.v_scale, math.sqrt(4096 / (64 * 128)))
    assert mimo.check_params(p0) == 0 and mimo.check_params(p1) == 0


def test_partial_rotary_factor_parsed_defensively():
    assert mimo.rope_dims_from_factor(1, 192) == 192          # typed int upstream
    assert mimo.rope_dims_from_factor("0.33", 32) == 10
    assert mimo.rope_dims_from_factor(0.0, 192) == 0
    with pytest.raises(ValueError):
        mimo.rope_dims_from_factor(1.5, 192)
    cfg = _full_config([1])
    cfg.partial_rotary_factor = 0.33
    assert cfg.rotated_dims == 63                              # odd: the library rejects it
    assert mimo.check_params(mimo.layer_spec(cfg, 0).params(cfg, 1)) == mimo.MIMO_ERR_INVALID_ARG
    cfg.rope_dims = 64
    assert cfg.rotated_dims == 64


def test_v_scale_values():
    assert synth.TINY_SWA.v_scale == 1.0
    assert math.isclose(synth.SWA_PREFILL.v_scale, 0.7071067811865476)
    assert math.isclose(layers.HybridAttentionConfig(
        hidden_size=64, num_attention_heads=4, num_key_value_heads=1, swa_num_key_value_heads=1,
        head_dim=32, v_head_dim=16, partial_rotary_factor=0.33, rope_theta=1e4,
        swa_rope_theta=1e4, sliding_window_size=16, hybrid_layer_pattern=[1]).v_scale, 1.0)
