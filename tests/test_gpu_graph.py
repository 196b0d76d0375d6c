"""Decode and extend under HIP graph capture.

A serving loop captures one decode step (the layers' decode calls plus the position advance) and
replays it; the entry points allocate nothing, set no memory and never synchronise, so they can be
captured.  Each replay must reproduce the eager calls on the same state bit for bit (the kernels
are deterministic), with unrelated eager work and synchronisations between the replays, and leave
the caches exactly as the eager calls leave them.
"""
from __future__ import annotations

import pytest
import torch

import global_attention_rope_amd as mimo
from tests import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _layer(kind, B, P0, R, seed, fp8=False):
    heads = synth.SWA_HEADS if kind == 1 else synth.GA_HEADS
    w = synth.Workload("graph", B, 1, dtype=torch.bfloat16, **heads)
    cap = w.window if kind == 1 else P0 + R
    q, kn, vn, s, kc, vc = synth.decode_inputs(w, seed, B, cap, device=DEV)
    p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, w.qk_head_dim, w.v_head_dim, w.rope_dims,
                    w.layer_kind, w.window, w.rope_theta, w.v_scale)
    if fp8:
        kc, vc = synth.fp8_cache_contents(w, seed + 7, B, cap, device=DEV)
        p.cache_dtype = mimo.CACHE_FP8_E4M3
        p.k_cache_scale, p.v_cache_scale = synth.FP8_K_SCALE, synth.FP8_V_SCALE
    ws = torch.empty(mimo.decode_workspace_size(p, P0 + R - 1) + 256, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, w.num_q_heads, w.v_head_dim), dtype=torch.bfloat16, device=DEV)
    return dict(p=p, q=q, kn=kn, vn=vn, s=s, kc=kc, vc=vc, ws=ws, out=out)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_graph_replays_match_eager(fp8):
    B, P0, R = 2, 3000, 4
    layers = [_layer(0, B, P0, R, 9100, fp8), _layer(1, B, P0, R, 9101, fp8)]
    maxp = P0 + R - 1
    print(f"[case] graph decode B={B} positions {P0}..{maxp}, global + sliding layer, fp8 {fp8}",
          flush=True)

    def step(pos, caches, outs):
        for l, (kc, vc), out in zip(layers, caches, outs):
            mimo.decode(l["p"], l["q"], l["kn"], l["vn"], pos, maxp, kc, vc, sinks=l["s"], out=out,
                        workspace=l["ws"])
        pos.add_(1)

    # eager reference on copies of the caches
    caches_e = [(l["kc"].clone(), l["vc"].clone()) for l in layers]
    outs_e = [torch.empty_like(l["out"]) for l in layers]
    pos_e = torch.full((B,), P0, dtype=torch.int32, device=DEV)
    ref = []
    for _ in range(R):
        step(pos_e, caches_e, outs_e)
        ref.append([o.clone() for o in outs_e])
    torch.cuda.synchronize()

    # captured step on the original caches
    caches = [(l["kc"], l["vc"]) for l in layers]
    outs = [l["out"] for l in layers]
    pos = torch.full((B,), P0, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pos, caches, outs)
    torch.cuda.synchronize()
    assert int(pos[0]) == P0, "capture must not execute the step"
    for t in range(R):
        g.replay()
        torch.cuda.synchronize()
        for li, (o, r) in enumerate(zip(outs, ref[t])):
            assert torch.equal(o, r), f"replay {t} layer {li} differs from the eager call"
        junk = torch.randn(4096, device=DEV)   # unrelated eager work between replays
        assert torch.isfinite(junk.sum())
        torch.cuda.synchronize()
    assert torch.equal(pos, pos_e)
    for (kc, vc), (kce, vce) in zip(caches, caches_e):
        assert torch.equal(kc, kce) and torch.equal(vc, vce)


@pytest.mark.parametrize("S,fp8", [(4, False), (40, False), (4, True), (40, True)])
def test_extend_graph_replays_match_eager(S, fp8):
    """A captured extend step (global and sliding layer; 4 tokens run the multi-token tile
    kernel, 40 the prefill kernel; bf16 or fp8 caches) replayed on the same caches: every replay
    equals the eager call on a copy of the state."""
    B, P0, R = 2, 500, 3
    print(f"[case] graph extend S={S} fp8={fp8}", flush=True)
    layers = []
    for kind, seed in ((0, 9200), (1, 9201)):
        heads = synth.SWA_HEADS if kind == 1 else synth.GA_HEADS
        w = synth.Workload("graph_ext", B, S, dtype=torch.bfloat16, **heads)
        cap = w.window if kind == 1 else P0 + R * S
        q, k, v, s = synth.layer_inputs(w, seed, device=DEV)
        if fp8:
            kc, vc = synth.fp8_cache_contents(w, seed + 1, B, cap, device=DEV)
        else:
            kc, vc = synth.cache_contents(w, seed + 1, B, cap, device=DEV)
        p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, w.qk_head_dim, w.v_head_dim,
                        w.rope_dims, w.layer_kind, w.window, w.rope_theta, w.v_scale)
        if fp8:
            p.cache_dtype = mimo.CACHE_FP8_E4M3
            p.k_cache_scale, p.v_cache_scale = synth.FP8_K_SCALE, synth.FP8_V_SCALE
        maxs = P0 + (R - 1) * S
        ws = torch.empty(mimo.extend_workspace_size(p, S, maxs) + 256, dtype=torch.uint8, device=DEV)
        out = torch.empty((B, S, w.num_q_heads, w.v_head_dim), dtype=torch.bfloat16, device=DEV)
        layers.append(dict(p=p, q=q, k=k, v=v, s=s, kc=kc, vc=vc, ws=ws, out=out, maxs=maxs))

    def step(pos, caches, outs):
        for l, (kc, vc), out in zip(layers, caches, outs):
            mimo.extend(l["p"], l["q"], l["k"], l["v"], pos, l["maxs"], kc, vc, sinks=l["s"],
                        out=out, workspace=l["ws"])
        pos.add_(S)

    caches_e = [(l["kc"].clone(), l["vc"].clone()) for l in layers]
    outs_e = [torch.empty_like(l["out"]) for l in layers]
    pos_e = torch.full((B,), P0, dtype=torch.int32, device=DEV)
    ref = []
    for _ in range(R):
        step(pos_e, caches_e, outs_e)
        ref.append([o.clone() for o in outs_e])
    torch.cuda.synchronize()
    caches = [(l["kc"], l["vc"]) for l in layers]
    outs = [l["out"] for l in layers]
    pos = torch.full((B,), P0, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pos, caches, outs)
    torch.cuda.synchronize()
    assert int(pos[0]) == P0, "capture must not execute the step"
    for t in range(R):
        g.replay()
        torch.cuda.synchronize()
        for li, (o, r) in enumerate(zip(outs, ref[t])):
            assert torch.equal(o, r), f"replay {t} layer {li} differs from the eager call"
        junk = torch.randn(4096, device=DEV)
        assert torch.isfinite(junk.sum())
        torch.cuda.synchronize()
    for (kc, vc), (kce, vce) in zip(caches, caches_e):
        assert torch.equal(kc, kce) and torch.equal(vc, vce)
