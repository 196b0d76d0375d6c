"""The allocation-free decode entry point (mimo_attn_decode_noalloc) against mimo_attn_decode.

Both run the same kernels; the allocation-free one keeps its split partials in the library's own
per-device scratch array instead of a caller workspace.  Two calls in a row, the second with a
smaller input (fewer sequences, shorter caches, the other layer kind), each against the workspace
entry point on copies of the same caches: outputs bit for bit, caches (the appended token) bit for
bit.  The first call's grid leaves partials in the array; the second must not be affected by
them.  Global-layer cases are split (several partial records per head), so the array is used.
"""
import pytest
import torch

import global_attention_rope_amd as mimo
from tests import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(kind, B, max_len, seed):
    heads = synth.GA_HEADS if kind == 0 else synth.SWA_HEADS
    w = synth.Workload("noalloc", B, 1, dtype=torch.bfloat16, **heads)
    positions = synth.decode_lengths(seed, batch=B, lo=max(1, max_len // 4), hi=max_len)
    cap = w.window if kind == 1 else int(positions.max()) + 1
    q, kn, vn, s, kc, vc = synth.decode_inputs(w, seed, B, cap, device=DEV)
    p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, 192, 128, w.rope_dims, w.layer_kind,
                    w.window, w.rope_theta, w.v_scale)
    pos = positions.to(DEV)
    return p, q, kn, vn, s, kc, vc, pos, int(positions.max())


def _run_both(kind, B, max_len, seed):
    p, q, kn, vn, s, kc, vc, pos, maxp = _case(kind, B, max_len, seed)
    if kind == 0:
        assert mimo.decode_workspace_size(p, maxp) > 0, "the case must use split partials"
    kc2, vc2 = kc.clone(), vc.clone()
    ref = mimo.decode(p, q, kn, vn, pos, maxp, kc, vc, sinks=s)
    out = torch.full_like(ref, 7.0)
    mimo.decode_noalloc(p, q, kn, vn, pos, maxp, kc2, vc2, sinks=s, out=out)
    torch.cuda.synchronize()
    print(f"[noalloc] kind={kind} B={B} max_len={maxp}", flush=True)
    assert torch.equal(out, ref), "outputs differ from the workspace entry point"
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc), "caches differ after the append"


def test_noalloc_decode_matches_workspace_decode_two_calls():
    _run_both(kind=0, B=16, max_len=20000, seed=31)   # ~ 2.5 MB of partials
    _run_both(kind=0, B=3, max_len=3000, seed=32)     # smaller: fewer sequences and splits
    _run_both(kind=1, B=2, max_len=500, seed=33)      # one split, no partials


def test_noalloc_decode_under_graph_replay():
    """Captured once, replayed twice with the positions advanced between replays: each replay
    equals an eager workspace decode of the same step."""
    p, q, kn, vn, s, kc, vc, pos, maxp = _case(0, 4, 6000, 34)
    cap = kc.shape[2]
    maxp2 = maxp + 2
    kc = torch.cat([kc, kc[:, :, :3]], dim=2).contiguous()
    vc = torch.cat([vc, vc[:, :, :3]], dim=2).contiguous()
    kc_ref, vc_ref = kc.clone(), vc.clone()
    out = torch.empty((4, p.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    ppos = pos.clone()
    g = torch.cuda.CUDAGraph()
    mimo.decode_noalloc(p, q, kn, vn, ppos, maxp2, kc.clone(), vc.clone(), sinks=s, out=out)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mimo.decode_noalloc(p, q, kn, vn, ppos, maxp2, kc, vc, sinks=s, out=out)
    for step in range(2):
        ppos.copy_(pos + step)
        g.replay()
        ref = mimo.decode(p, q, kn, vn, pos + step, maxp2, kc_ref, vc_ref, sinks=s)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {step}"
    assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref)
    del cap
