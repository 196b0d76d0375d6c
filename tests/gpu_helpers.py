"""Helpers for the GPU parity tests: comparisons and oracle-side views of seeded inputs.

Tolerance for bf16 inputs with fp32 accumulation (absolute 1e-2, relative 2e-2): PASS iff every
element satisfies |gpu - oracle| <= 1e-2 + 2e-2 * |oracle| (allclose form of the two bounds) and
the whole tensor satisfies ||gpu - oracle||_2 / ||oracle||_2 <= 2e-2.  The bf16 output alone is
rounded by up to 2^-8 * |x| (0.0156 at |x| = 4), so a bare max-abs bound of 1e-2 would reject
correctly rounded large outputs.  fp32 layers: absolute 2e-5, relative 1e-5, same form.
Where every rotated dim is rounded to bf16 (rotation widths up to the whole head), bf16 arithmetic
itself can exceed that fixed bound on a few elements (rows that see few keys): there a per-element
bound derived from the rounding points (tests/rounding_model.py, error_bound) applies instead, and
the L2 error is held to the rounding model's (assert_near_model).

Layer with projections: tests/test_gpu_layer.py (tolerance from the rounding model, per row).
"""
from __future__ import annotations

import numpy as np
import torch

BF16_MAX_ABS, BF16_REL_L2 = 1e-2, 2e-2
F32_MAX_ABS, F32_REL_L2 = 2e-5, 1e-5


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def errors(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d)) / nrm if nrm > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(gpu, ref, fp32=False, what="", atol=None, bound=None):
    """atol overrides the absolute term (the relative terms stay).  bound (per element, from
    tests/rounding_model.py): an element also passes within the error that bf16 rounding of the
    operands can cause there (the derived bound), where that exceeds the fixed one."""
    gpu = to_np64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    max_abs, rel = errors(gpu, ref)
    lim_abs, lim_rel = (F32_MAX_ABS, F32_REL_L2) if fp32 else (BF16_MAX_ABS, BF16_REL_L2)
    if atol is not None:
        lim_abs = atol   # (a scalar, or one value per element)
    lim_elem = lim_abs + lim_rel * np.abs(ref)
    widened = 0
    if bound is not None:
        widened = int(np.count_nonzero(bound > lim_elem))
        lim_elem = np.maximum(lim_elem, bound)
    excess = np.abs(gpu - ref) - lim_elem
    worst = int(np.argmax(excess)) if excess.size else 0
    ok_elem = excess.size == 0 or excess.flat[worst] <= 0
    assert ok_elem and rel <= lim_rel, (
        f"{what}: worst element {np.unravel_index(worst, gpu.shape)} gpu {gpu.flat[worst]:.5f} "
        f"oracle {ref.flat[worst]:.5f}; max_abs {max_abs:.3e}, rel_l2 {rel:.3e} "
        f"(limits abs {lim_abs} + rel {lim_rel})")
    lit = int(np.count_nonzero(np.abs(gpu - ref) > BF16_MAX_ABS + lim_rel * np.abs(ref)))
    extra = f" (derived bound wider on {widened} of {ref.size}; {lit} outside the fixed bound)" \
        if bound is not None else ""
    print(f"  [{what}] max_abs {max_abs:.3e} rel_l2 {rel:.3e}{extra}", flush=True)
    return max_abs, rel


# A kernel that rounds where the rounding model rounds (tests/rounding_model.py) and accumulates in
# fp32 lands a different draw of the same rounding errors: its L2 error against the oracle stays
# within this factor of the model's (plus a floor for small outputs), on every case measured.
MODEL_RATIO, MODEL_FLOOR = 1.5, 2e-4


def assert_near_model(gpu, ref, model, what=""):
    """The kernel's L2 error against the oracle is no larger than ideal bf16 arithmetic's (the
    rounding model's), up to MODEL_RATIO: a tighter check than the fixed 2e-2 bound, which a lost
    term of under 2% (a dropped sink on a 128-key window moves outputs by ~0.8%) would pass."""
    gpu = to_np64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    sel = np.isfinite(ref) & np.isfinite(model)
    _, rel_g = errors(gpu[sel], ref[sel])
    _, rel_m = errors(model[sel], ref[sel])
    lim = MODEL_RATIO * rel_m + MODEL_FLOOR
    print(f"  [{what}] rel_l2 kernel {rel_g:.3e} model {rel_m:.3e} (ratio {rel_g / max(rel_m, 1e-30):.2f})",
          flush=True)
    assert rel_g <= lim, f"{what}: rel_l2 {rel_g:.3e} above {MODEL_RATIO} x the rounding model's {rel_m:.3e}"
    return rel_g, rel_m


def _f32np(t):
    return None if t is None else t.to("cpu", torch.float32).numpy()


def workload_oparams(w, batch=None):
    """The oracle's parameter block for a synth.Workload."""
    from oracle import OracleParams
    return OracleParams(w.batch if batch is None else batch, w.num_q_heads, w.num_kv_heads,
                        w.qk_head_dim, w.v_head_dim, w.rope_dims, w.layer_kind, w.window,
                        w.rope_theta, w.v_scale)


def prefill_bound_for(w, q, k, v, sinks, positions, rows=None):
    """The derived per-element bound (tests/rounding_model.py) of a prefill of workload w on the
    given torch inputs; rows not listed are NaN."""
    from tests import rounding_model
    return rounding_model.prefill_bound(workload_oparams(w, q.shape[0]), _f32np(q), _f32np(k),
                                        _f32np(v), np.asarray(positions), _f32np(sinks), rows=rows)


def ring_positions(pos: int, window: int) -> np.ndarray:
    """Position held by each ring slot just before the token at `pos` is appended: the most
    recent position < pos congruent to the slot (negative: the slot is still empty)."""
    s = np.arange(window)
    return pos - 1 - ((pos - 1 - s) % window)
