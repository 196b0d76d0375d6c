"""GPU parity of the MoE router kernel against the router oracle.

Expert indices are compared exactly.  Both sides take every decision on the same float32 values
(the fp64 sigmoid rounded to fp32, plus the bias in fp32, and the fp32 group sums), except that
the two fp64 exponentials may differ in their last bits: a row may therefore differ only where
the scores of the exchanged experts are within 2 fp32 ulps of each other, which the test checks
(it has not happened on these inputs).  Weights: fp32 against fp64, relative 1e-6.  Seeds:
14000 + case.
"""
import numpy as np
import pytest
import torch

import global_attention_rope_amd as mimo
import oracle
from tests import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _note(msg):
    print(f"[case] {msg}", flush=True)


def _check(p, logits, bias, idx, w):
    op = oracle.RouterParams(p.num_experts, p.n_group, p.topk_group, p.top_k, p.norm_topk_prob,
                             p.routed_scaling_factor)
    x = logits.cpu().numpy()
    b = None if bias is None else bias.cpu().numpy()
    ridx, rw = oracle.router(op, x, b)
    gi, gw = idx.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    bad = np.nonzero((gi != ridx).any(axis=1))[0]
    if len(bad):
        s = torch.sigmoid(torch.from_numpy(x[bad].astype(np.float64))).float()
        c = (s + (0 if b is None else torch.from_numpy(b))).numpy()
        for r, t in enumerate(bad):
            cg, co = c[r, gi[t]], c[r, ridx[t]]
            ulp = np.spacing(np.maximum(np.abs(cg), np.abs(co)).astype(np.float32))
            assert np.all(np.abs(cg - co) <= 2 * ulp), f"token {t}: {gi[t]} vs oracle {ridx[t]}"
    ok = ~np.isin(np.arange(len(gi)), bad)
    np.testing.assert_allclose(gw[ok], rw[ok], rtol=1e-6, atol=1e-7)
    return len(bad)


CASES = [
    dict(E=256, G=8, TG=4, K=8, norm=True, scale=2.5, T=1001, bias_sd=0.1),
    dict(E=64, G=1, TG=1, K=6, norm=True, scale=1.0, T=333, bias_sd=0.0),
    dict(E=128, G=16, TG=3, K=5, norm=False, scale=1.0, T=517, bias_sd=0.3),
    dict(E=512, G=64, TG=8, K=16, norm=True, scale=1.0, T=250, bias_sd=0.1),
    dict(E=256, G=8, TG=2, K=8, norm=True, scale=1.0, T=400, bias_sd=2.0),   # many negative scores
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_router_against_oracle(ci):
    c = CASES[ci]
    _note(str(c))
    logits, bias = synth.router_inputs(14000 + ci, c["T"], c["E"], device=DEV, bias_sd=c["bias_sd"])
    if c["bias_sd"] >= 1.0:
        bias = bias - 3.0
    p = mimo.RouterParams(c["E"], c["G"], c["TG"], c["K"], c["norm"], c["scale"])
    idx, w = mimo.router_topk(p, logits, bias)
    torch.cuda.synchronize()
    assert _check(p, logits, bias, idx, w) == 0


def test_router_full_size_and_ties():
    p = mimo.RouterParams()
    T = synth.ROUTER_TOKENS
    _note(f"router T={T}")
    logits, bias = synth.router_inputs(14100, T, device=DEV)
    idx, w = mimo.router_topk(p, logits, bias)
    torch.cuda.synchronize()
    assert _check(p, logits, bias, idx, w) == 0
    # all scores equal: the lowest indices of the first groups, weights 1/k
    z = torch.zeros((8, 256), dtype=torch.float32, device=DEV)
    idx, w = mimo.router_topk(p, z, None)
    torch.cuda.synchronize()
    assert (idx.cpu() == torch.arange(8, dtype=torch.int32)).all()
    assert torch.allclose(w.cpu(), torch.full((8, 8), 1.0 / 8))
