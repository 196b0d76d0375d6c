"""GPU parity of the layer entry point (q/k/v projections, attention, output projection with the
value rescale folded in) against the oracle's fp64 layer.  Seeds: 12000 + case.

Tolerance (reading A23): the layer output has no fixed scale, and its error comes from bf16
roundings (projected q and v, the rotated key, the scaled query, softmax weights, the attention
output, the output) carried through dense products; rows that see few keys keep the largest
errors.  The rounding model (tests/rounding_model.py, layer_prefill) computes the same layer with
exactly those roundings; each element passes within 6 times the RMS of the model's own error over
its row (plus two roundings of the output, and the usual 2e-2 relative term), and the kernel's L2
error must stay within 1.5 times the model's."""
import numpy as np
import pytest
import torch

import global_attention_rope_amd as mimo
import oracle
from tests import rounding_model, synth
from tests.gpu_helpers import assert_close, assert_near_model
from tests.test_gpu_parity import _f32, _note, _oparams, _params, _wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(w, hidden, out_dim, starts, seed, rows=None, with_cache=False):
    x, s = synth.layer_input(w, seed, hidden, device=DEV)
    wq, wk, wv, wo = synth.layer_weights(w, seed + 1, hidden, out_dim, device=DEV)
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    kc = vc = None
    if with_cache:
        cap = w.window if w.layer_kind == 1 else max(starts) + w.seq
        kc = torch.zeros((w.batch, w.num_kv_heads, cap, w.qk_head_dim), dtype=w.dtype, device=DEV)
        vc = torch.zeros((w.batch, w.num_kv_heads, cap, w.v_head_dim), dtype=w.dtype, device=DEV)
    out = mimo.layer_prefill(_params(w), x, wq, wk, wv, wo, sp, sinks=s, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    pos = np.stack([np.arange(w.seq, dtype=np.int32) + st for st in starts])
    args = (_oparams(w), _f32(x), _f32(wq), _f32(wk), _f32(wv), _f32(wo), pos, _f32(s))
    ref = oracle.layer_prefill(*args, rows=rows)
    model = rounding_model.layer_prefill(*args, rows=rows)
    return out, ref, model


@pytest.mark.parametrize("case", [
    dict(kind=1, B=2, S=100, Hq=8, Hkv=2, sinks=True, starts=[0, 40], W=32, hidden=512, out=384),
    dict(kind=0, B=2, S=77, Hq=8, Hkv=2, sinks=False, starts=[0, 5], hidden=768, out=512),
    dict(kind=1, B=1, S=300, Hq=16, Hkv=2, sinks=True, starts=[0], W=128, hidden=1024, out=1024),
    # rotated widths the projection epilogue does not rotate (the prefill's key pass does), and
    # none at all; a single KV head (a key tile holding a head's start and part of nothing else)
    dict(kind=0, B=2, S=90, Hq=8, Hkv=2, sinks=False, starts=[0, 7], r=128, hidden=512, out=256),
    dict(kind=1, B=1, S=150, Hq=8, Hkv=1, sinks=True, starts=[3], W=64, r=0, hidden=640, out=136),
])
def test_layer_prefill_small(case):
    case = dict(case)
    starts, hidden, out_dim = case.pop("starts"), case.pop("hidden"), case.pop("out")
    w = _wl(**case)
    _note(f"layer {case} hidden {hidden} out {out_dim}")
    out, ref, model = _run(w, hidden, out_dim, starts, 12000 + w.seq, with_cache=True)
    assert_close(out, ref, what=f"layer {case}", atol=rounding_model.layer_row_tolerance(model, ref))
    assert_near_model(out, ref, model, what=f"layer {case}")


@pytest.mark.parametrize("kind", [0, 1])
def test_layer_prefill_full_size_sampled_rows(kind):
    """Hidden 4096 -> 64 query heads -> 4096: the sliding layer at 4096 tokens, the global one at
    8192, sampled rows (first, last, random)."""
    w = synth.SWA_PREFILL if kind == 1 else synth.GA_PREFILL
    _note(f"layer full {w.name}")
    rng = np.random.default_rng(12 + kind)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(w.seq - 8, w.seq),
                                     rng.integers(0, w.seq, 24)])).astype(np.int32)
    out, ref, model = _run(w, 4096, 4096, [0], 12100 + kind, rows=rows)
    o, r, m = out.to("cpu", torch.float64).numpy()[:, rows], ref[:, rows], model[:, rows]
    assert_close(o, r, what=f"layer {w.name}", atol=rounding_model.layer_row_tolerance(m, r))
    assert_near_model(o, r, m, what=f"layer {w.name}")
