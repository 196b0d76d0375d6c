"""CPU checks of the rounding model the GPU parity tests use (tests/rounding_model.py).

  * with nothing to round (no rotation, one visible key, no sink) the model's output is the
    oracle's, rounded once to bf16 — the single rounding the model adds there;
  * on random layers of both kinds at several rotation widths, the model's error against the
    oracle stays inside the derived per-element bound everywhere, with margin;
  * the bound grows with the number of rotated (rounded) dims, and is mostly tighter than the
    fixed 1e-2 + 2e-2 |x| bound.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import OracleParams
from tests import rounding_model as rm
from tests import synth


def _case(kind, r, S=120, B=1, Hq=4, Hkv=2, seed=3):
    theta = 1e4 if kind == 1 else 5e6
    w = synth.Workload("m", batch=B, seq=S, num_q_heads=Hq, num_kv_heads=Hkv, qk_head_dim=192,
                       v_head_dim=128, rope_dims=r, rope_theta=theta, layer_kind=kind,
                       window=64 if kind else 0, sinks=kind == 1, hidden=4096,
                       dtype=torch.bfloat16)
    q, k, v, s = synth.layer_inputs(w, seed)
    f = lambda t: None if t is None else t.float().numpy()
    pos = np.stack([np.arange(S, dtype=np.int32) + 11 * b for b in range(B)])
    op = OracleParams(B, Hq, Hkv, 192, 128, r, kind, w.window, theta, w.v_scale)
    return op, f(q), f(k), f(v), pos, f(s)


def test_single_key_is_one_rounding_of_the_oracle():
    op, q, k, v, pos, _ = _case(0, 0, S=1)
    ref = oracle.prefill(op, q, k, v, pos)
    model = rm.prefill(op, q, k, v, pos)
    assert np.array_equal(model, rm.bf16(ref))


@pytest.fixture
def every_row(monkeypatch):
    """The bound on every row (by default rows seeing more than BOUND_MAX_KEYS keys get 0)."""
    monkeypatch.setattr(rm, "BOUND_MAX_KEYS", 1 << 30)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", [0, 64, 192])
def test_model_error_inside_derived_bound(kind, r, every_row):
    op, q, k, v, pos, s = _case(kind, r)
    ref = oracle.prefill(op, q, k, v, pos, s)
    model = rm.prefill(op, q, k, v, pos, s)
    bound = rm.prefill_bound(op, q, k, v, pos, s)
    err = np.abs(model - ref)
    assert np.all(err <= 0.9 * bound), float(np.max(err / bound))
    # the model is an actual perturbation, not the oracle itself
    assert rm.rel_l2(model, ref) > 5e-4


def test_default_bound_covers_only_rows_with_few_keys():
    op, q, k, v, pos, s = _case(0, 64, S=200)
    bound = rm.prefill_bound(op, q, k, v, pos, s)
    assert np.all(bound[:, :rm.BOUND_MAX_KEYS] > 0)
    assert np.all(bound[:, rm.BOUND_MAX_KEYS:] == 0)


def test_bound_grows_with_rotated_dims_and_is_mostly_tighter_than_fixed(every_row):
    meds = []
    for r in (0, 64, 192):
        op, q, k, v, pos, s = _case(0, r)
        ref = oracle.prefill(op, q, k, v, pos, s)
        bound = rm.prefill_bound(op, q, k, v, pos, s)
        meds.append(float(np.median(bound)))
        assert np.mean(bound > 1e-2 + 2e-2 * np.abs(ref)) < 0.25
    assert meds[0] < meds[1] < meds[2]


def test_extend_bound_matches_prefill_bound_on_an_empty_cache(every_row):
    op, q, k, v, pos, s = _case(1, 64, B=1)
    bp = rm.prefill_bound(op, q, k, v, pos, s)
    be = rm.extend_bound(op, q, k, v, pos[:, 0], None, None, None, None, s)
    np.testing.assert_allclose(be, bp, rtol=1e-12, atol=0)
