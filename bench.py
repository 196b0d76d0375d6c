"""Benchmark of the hybrid attention hot path on one MI355X.

One step = one pass of the whole path over one batch of the 48-layer attention-only stack:
hybrid_layer_pattern = layer 0 global then 5 sliding : 1 global; batch 2; prefill of 16384 tokens
per layer (each layer writes its KV cache: linear for global layers, 128-slot ring for sliding
ones), then 256 single-token decode steps through all 48 layers.  Head shapes: 64 query heads,
QK head dim 192 (64 rotated), V head dim 128; global layers 4 KV heads, theta 5e6, no sink;
sliding layers 8 KV heads, theta 1e4, window 128, per-head sinks.  Inputs are seeded N(0,1) bf16,
generated on the device before timing; every layer has its own inputs (seed 4000 + layer).

Output: one JSON line.  `value` is the step's algorithmic TFLOP/s (prefill + decode flops, masked
pairs not counted, over the measured step time); the per-phase numbers (prefill TFLOP/s, decode
KV GB/s, each kind separately, with roofline fractions) are in `phases`; `roofline` covers the
dominant kernel (global-layer prefill) and `cpu_baseline` the fp64 oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N] [--no-cpu-baseline]
                      [--eager-decode]

The decode phase replays one HIP graph per step (the 48 decode calls and the position increment,
captured once before timing); --eager-decode launches them from Python instead.

Single-layer workloads for profiling (not the bench line): --workload swa_prefill (batch 1, 4096
tokens, sliding), ga_prefill (batch 1, 8192 tokens, global), decode (batch 64, cached lengths
uniform in [1024, 32768] for the global layer, full 128-slot rings for the sliding one; with bf16
and with fp8 e4m3 caches), copy
(a 2 GiB device-to-device copy: the known-size reference for HBM byte counters and the
achievable HBM rate), gemm (8192^3 bf16 matrix product: the achievable matrix-core rate),
extend (new tokens against a cache: a 2048-token chunk after 30000 cached positions, global and
sliding, batch 1; and 4 tokens per sequence after the decode workload's cached lengths, batch 64,
the shape of multi-token verification; the global ones again over fp8 caches), layer (the layer entry point: hidden 4096 -> q/k/v
projections -> attention -> output projection back to 4096, on the sliding 4096-token and the
global 8192-token prefill shapes; the projections run on this library's bf16 MFMA kernel), router (the MoE router
kernel: 32768 tokens, 256 experts in 8 groups, 4 groups kept, top 8).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
DQK, DV = 192, 128

# HBM bytes per global-layer prefill call, counted by rocprofv3 (FETCH_SIZE and WRITE_SIZE, each
# scaled by what the counter reads for a copy of known size); valid only for the kernel sources it
# was taken on, which the summary records as a SHA-256.
TRAFFIC_PROFILE = os.path.join("profiles", "ga_prefill_b2_s16384_hbm_counters.md")
TRAFFIC_SOURCES = ["global_attention_rope_amd/csrc/prefill_bf16.hip",
                   "global_attention_rope_amd/csrc/rope_kv.hip",
                   "global_attention_rope_amd/csrc/device_common.h",
                   "global_attention_rope_amd/csrc/kernels.h"]


def counted_traffic():
    """Bytes per call from the committed counter summary, or None when the kernels changed since."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, TRAFFIC_PROFILE)).read()
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    except OSError:
        return None
    m_b = re.search(r"traffic_bytes_per_call:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    if not m_b or not m_h or m_h.group(1) != h.hexdigest():
        return None
    return float(m_b.group(1))


def pairs_visible(S: int, kind: int, W: int) -> int:
    """Number of (query, key) pairs the mask admits in a prefill of S tokens."""
    if kind == 0:
        return S * (S + 1) // 2
    full = max(0, S - W)
    head = min(S, W)
    return head * (head + 1) // 2 + full * W


def prefill_counts(B, S, Hq, Hkv, kind, W):
    flops = B * Hq * pairs_visible(S, kind, W) * 2 * (DQK + DV)
    io = B * S * (Hq * DQK + Hkv * (DQK + DV) + Hq * DV) * 2       # q, k, v read; out written
    cached = min(S, W) if kind == 1 else S
    io += B * cached * Hkv * (DQK + DV) * 2                          # rotated K and V stored
    return flops, io


def decode_counts(B, Hq, Hkv, kind, W, positions, cache_bytes=2):
    """flops and bytes of one decode step: every visible cached slot read once, q/k/v_new read,
    out and the appended slot written (cache_bytes per cache element: 2 bf16, 1 fp8)."""
    flops = bytes_ = 0
    for p in positions:
        cached = min(W - 1, p) if kind == 1 else p
        flops += Hq * (cached + 1) * 2 * (DQK + DV)
        bytes_ += Hkv * cached * (DQK + DV) * cache_bytes
    B = len(positions)
    bytes_ += B * (Hq * DQK + Hkv * (DQK + DV) + Hq * DV) * 2 + B * Hkv * (DQK + DV) * cache_bytes
    return flops, bytes_


def extend_counts(Hq, Hkv, kind, W, starts, S, cache_bytes=2):
    """flops and bytes of one extend call: visible (query, key) pairs; q, k, v read, out written,
    the cached positions any new token sees read once, the new tokens stored (ring: the last W),
    cache elements of cache_bytes bytes (1 for fp8 codes)."""
    flops = bytes_ = 0
    for st in starts:
        if kind == 0:
            pairs = S * st + S * (S + 1) // 2          # row i sees st + i + 1 keys
            cached, stored = st, S
        else:
            pairs = sum(min(W, st + i + 1) for i in range(S))
            cached, stored = min(W - 1, st), min(S, W)
        flops += Hq * pairs * 2 * (DQK + DV)
        bytes_ += (S * (Hq * DQK + Hkv * (DQK + DV) + Hq * DV) * 2
                   + Hkv * (cached + stored) * (DQK + DV) * cache_bytes)
    return flops, bytes_


def cpu_baseline(stack_cfg, seed_base):
    """The fp64 oracle on a bounded sample of the same workload (about 15 s of host work): sequence
    0 of layer 0 (global) over its first 6144 tokens, of layer 1 (sliding) over its first 4096
    tokens, and one global decode step at position 6144 against the oracle's own rotated keys."""
    import numpy as np
    import torch

    import oracle
    from tests import synth

    ga, swa = synth.GA_PREFILL, synth.SWA_PREFILL
    S_ga, S_swa = 6144, 4096
    f = lambda t: t.to(torch.float32).numpy()
    q, k, v, _ = synth.layer_inputs(ga, seed_base + 0, batch=1, seq=S_ga + 1)
    q2, k2, v2, s2 = synth.layer_inputs(swa, seed_base + 1, batch=1, seq=S_swa)
    op_ga = oracle.OracleParams(1, 64, 4, DQK, DV, 64, 0, 0, 5e6, ga.v_scale)
    op_swa = oracle.OracleParams(1, 64, 8, DQK, DV, 64, 1, 128, 1e4, swa.v_scale)
    pos_ga = np.arange(S_ga, dtype=np.int32)[None]
    pos_swa = np.arange(S_swa, dtype=np.int32)[None]
    qa, ka, va = f(q[:, :S_ga]), f(k[:, :S_ga]), f(v[:, :S_ga])
    qs, ks, vs, ss = f(q2), f(k2), f(v2), f(s2)
    t0 = time.perf_counter()
    _, krot = oracle.prefill(op_ga, qa, ka, va, pos_ga, None, want_k_rot=True)
    oracle.prefill(op_swa, qs, ks, vs, pos_swa, ss)
    kc = np.ascontiguousarray(krot.transpose(0, 2, 1, 3)).astype(np.float32)
    vc = np.ascontiguousarray(va.transpose(0, 2, 1, 3))
    oracle.decode(op_ga, f(q[:, S_ga]), f(k[:, S_ga]), f(v[:, S_ga]), np.array([S_ga], np.int32),
                  kc, vc, pos_ga, np.array([S_ga], np.int32), None)
    dt = time.perf_counter() - t0
    flops = (prefill_counts(1, S_ga, 64, 4, 0, 0)[0] + prefill_counts(1, S_swa, 64, 8, 1, 128)[0]
             + decode_counts(1, 64, 4, 0, 128, [S_ga])[0])
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu, "kind": "oracle",
            "sample": (f"fp64 oracle, sequence 0 only: layer 0 (global) prefill of the first {S_ga} "
                       f"tokens, layer 1 (sliding) prefill of the first {S_swa} tokens, one global "
                       f"decode step at position {S_ga}; {flops:.3e} algorithmic flop in "
                       f"{dt:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-decode", action="store_true",
                    help="launch every decode call from Python instead of replaying a HIP graph")
    ap.add_argument("--workload", default="stack",
                    choices=["stack", "swa_prefill", "ga_prefill", "decode", "extend", "layer",
                             "router", "copy", "gemm", "decode_latency", "ceilings"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hybrid attention hot path runs on a single device "
              "here (multi-GPU sharding is described, not built); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import global_attention_rope_amd as mimo
    from tests import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mimo.lib()  # fails loudly when the HIP library is missing
    if args.workload != "stack":
        single_layer(args, dev)
        return

    L, B, S, T = synth.STACK_LAYERS, synth.STACK_BATCH, synth.STACK_SEQ, args.decode_steps
    pattern = synth.stack_pattern(L)
    cfg = mimo.HybridAttentionConfig(
        hidden_size=4096, num_attention_heads=64, num_key_value_heads=4,
        swa_num_key_value_heads=8, head_dim=DQK, v_head_dim=DV, partial_rotary_factor=1.0 / 3.0,
        rope_theta=5e6, swa_rope_theta=1e4, sliding_window_size=128, hybrid_layer_pattern=pattern,
        rope_dims=64)
    specs = mimo.layer_specs(cfg)
    Hq = cfg.num_attention_heads
    seed_base = 4000

    # ---- inputs and state, all resident before timing
    layers = []
    for sp in specs:
        w = synth.SWA_PREFILL if sp.kind == mimo.LAYER_SWA else synth.GA_PREFILL
        q, k, v, s = synth.layer_inputs(w, seed_base + sp.index, device=dev, batch=B, seq=S)
        cap = sp.window if sp.kind == mimo.LAYER_SWA else S + T
        kc = torch.zeros((B, sp.num_kv_heads, cap, DQK), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros((B, sp.num_kv_heads, cap, DV), dtype=torch.bfloat16, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(seed_base + 100 + sp.index)
        # the decoding token's q/k/v buffers of this layer (a serving engine's projection outputs:
        # fixed addresses, rewritten every step; the values do not change the work)
        dq = torch.randn((B, Hq, DQK), generator=g, device=dev).to(torch.bfloat16)
        dk = torch.randn((B, sp.num_kv_heads, DQK), generator=g, device=dev).to(torch.bfloat16)
        dv = torch.randn((B, sp.num_kv_heads, DV), generator=g, device=dev).to(torch.bfloat16)
        layers.append(dict(spec=sp, p=sp.params(cfg, B), q=q, k=k, v=v,
                           sinks=s if sp.has_sinks else None, kc=kc, vc=vc, dq=dq, dk=dk, dv=dv))
    start_pos = torch.zeros(B, dtype=torch.int32, device=dev)
    dec_pos = torch.full((B,), S, dtype=torch.int32, device=dev)   # position of the decoding token
    out_pf = torch.empty((B, S, Hq, DV), dtype=torch.bfloat16, device=dev)
    out_dec = torch.empty((B, Hq, DV), dtype=torch.bfloat16, device=dev)
    ws_pf = torch.empty(max(mimo.prefill_workspace_size(l["p"], S) for l in layers) + 256,
                        dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(mimo.decode_workspace_size(l["p"], S + T - 1) for l in layers) + 256,
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    ga_events = []

    def decode_step():
        """One decode step through the 48 layers, then the position advances."""
        for l in layers:
            mimo.decode(l["p"], l["dq"], l["dk"], l["dv"], dec_pos, S + T - 1, l["kc"], l["vc"],
                        sinks=l["sinks"], out=out_dec, workspace=ws_dec)
        dec_pos.add_(1)

    graph = None
    if not args.eager_decode:
        # decode is launch-bound at batch 2 (48 small layers per step): the step is captured once
        # as a HIP graph and replayed; positions live in device memory, so one graph serves every
        # step.  Warm up eagerly first (kernel code objects load on first launch).
        dec_pos.fill_(S)
        decode_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_step()
        torch.cuda.synchronize()

    def step(record):
        for l in layers:
            is_ga = l["spec"].kind == mimo.LAYER_GLOBAL
            if record and is_ga:
                e0 = ev()
                e0.record()
            mimo.prefill(l["p"], l["q"], l["k"], l["v"], start_pos, sinks=l["sinks"], out=out_pf,
                         k_cache=l["kc"], v_cache=l["vc"], workspace=ws_pf)
            if record and is_ga:
                e1 = ev()
                e1.record()
                ga_events.append((e0, e1))
        mid = ev()
        mid.record()
        dec_pos.fill_(S)
        for t in range(T):
            if graph is not None:
                graph.replay()
            else:
                decode_step()
        return mid

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    starts, mids, ends = [], [], []
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        e0 = ev()
        e0.record()
        mids.append(step(True))
        e1 = ev()
        e1.record()
        starts.append(e0)
        ends.append(e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall

    step_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    prefill_ms = sum(a.elapsed_time(b) for a, b in zip(starts, mids)) / args.steps
    decode_ms = sum(a.elapsed_time(b) for a, b in zip(mids, ends)) / args.steps
    ga_ms = sum(a.elapsed_time(b) for a, b in ga_events) / len(ga_events)

    # ---- algorithmic work of one step
    n_ga = sum(1 for sp in specs if sp.kind == mimo.LAYER_GLOBAL)
    n_swa = L - n_ga
    f_ga, b_ga = prefill_counts(B, S, Hq, 4, 0, 0)
    f_swa, b_swa = prefill_counts(B, S, Hq, 8, 1, 128)
    pf_flops = n_ga * f_ga + n_swa * f_swa
    dec_f = dec_b = dec_b_ga = dec_b_swa = 0
    for t in range(T):
        fg, bg = decode_counts(B, Hq, 4, 0, 128, [S + t] * B)
        fs, bs = decode_counts(B, Hq, 8, 1, 128, [S + t] * B)
        dec_f += n_ga * fg + n_swa * fs
        dec_b_ga += n_ga * bg
        dec_b_swa += n_swa * bs
    dec_b = dec_b_ga + dec_b_swa
    step_flops = pf_flops + dec_f
    value = step_flops / (step_ms * 1e-3) / 1e12
    ga_tflops = f_ga / (ga_ms * 1e-3) / 1e12
    swa_prefill_ms = (prefill_ms - n_ga * ga_ms) / n_swa
    swa_gbps = b_swa / (swa_prefill_ms * 1e-3) / 1e9
    dec_gbps = dec_b / (decode_ms * 1e-3) / 1e9

    result = {
        "metric": "attention prefill TFLOP/s and decode KV GB/s (SWA and GA) + % of roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hybrid_stack_48L_b2_s16384_prefill_256_decode",
                   "layers": L, "global_layers": n_ga, "sliding_layers": n_swa, "batch": B,
                   "prefill_tokens": S, "decode_steps": T, "num_q_heads": Hq,
                   "kv_heads_global": 4, "kv_heads_sliding": 8, "qk_head_dim": DQK,
                   "v_head_dim": DV, "rope_dims": 64, "window": 128,
                   "theta_global": 5e6, "theta_sliding": 1e4},
        "phases": {
            "prefill": {"ms": round(prefill_ms, 3),
                        "tflops": round(pf_flops / (prefill_ms * 1e-3) / 1e12, 2),
                        "global_layer_ms": round(ga_ms, 4),
                        "global_layer_tflops": round(ga_tflops, 2),
                        "global_frac_mfma_peak": round(ga_tflops / PEAK_BF16_TFLOPS, 4),
                        "sliding_layer_ms_avg": round(swa_prefill_ms, 4),
                        "sliding_layer_GBps": round(swa_gbps, 1),
                        "sliding_frac_hbm_peak": round(swa_gbps / PEAK_HBM_GBPS, 4)},
            "decode": {"ms": round(decode_ms, 3), "steps": T,
                       "launch": "eager" if graph is None else "hip_graph_per_step",
                       "GBps": round(dec_gbps, 1),
                       "frac_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
                       "kv_bytes_global": dec_b_ga, "kv_bytes_sliding": dec_b_swa},
        },
        "roofline": {"bound": "mfma", "achieved": round(ga_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ga_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic(),
                     "traffic_source": TRAFFIC_PROFILE,
                     "kernel": "global-layer prefill (key rotation pass + attention kernel), "
                               f"B{B} S{S}, {f_ga:.4e} flop per call"},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, seed_base)
    print(json.dumps(result), flush=True)


def decode_latency(args, dev):
    """Per-call time of the stack's decode calls (batch 2) against the latency floor, each set of
    calls captured in one HIP graph and replayed: 40 calls that only launch (empty kernel, 16
    workgroups), 40 one-tile dependent reads (16 workgroups, 80 KiB each, a fresh 1.3 MB region per
    call: the bytes of one sliding layer's ring), the 40 sliding-layer decodes and the 8
    global-layer decodes of one decode step (positions 16384); then one decode call of each kind
    at the decode workload's batch of 64.  'cold': a 512 MiB scratch buffer is written before
    every replay, outside the timed region, so every ring comes from memory (the write-back of
    that buffer's dirty lines can still overlap the replay); 'hot': replayed back to back."""
    import ctypes

    import torch

    import global_attention_rope_amd as mimo
    from global_attention_rope_amd import build as hb
    from tests import synth

    probe = ctypes.CDLL(hb.PROBE_LIB)
    vp = ctypes.c_void_p
    probe.mimo_probe_empty.argtypes = [vp, ctypes.c_int32, vp]
    probe.mimo_probe_tile_read.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, vp]
    B, S, NSW, NGA, G = 2, synth.STACK_SEQ, 40, 8, 16
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    region = G * 80 * 1024
    src = torch.ones(NSW * region // 4, dtype=torch.int32, device=dev)
    dst = torch.empty(NSW * G * 256, dtype=torch.int32, device=dev)
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def probes_empty():
        for l in range(NSW):
            assert probe.mimo_probe_empty(vp(dst.data_ptr() + l * G * 1024), G, cur()) == 0

    def probes_read():
        for l in range(NSW):
            assert probe.mimo_probe_tile_read(vp(src.data_ptr() + l * region),
                                              vp(dst.data_ptr() + l * G * 1024), G, 80, cur()) == 0

    def mk_layers(heads, n, seed):
        w = synth.Workload("dec", B, 1, dtype=torch.bfloat16, **heads)
        cap = w.window if w.layer_kind == 1 else S + 1
        out = []
        for i in range(n):
            q, kn, vn, sk, kc, vc = synth.decode_inputs(w, seed + i, B, cap, device=dev)
            p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims, w.layer_kind,
                            w.window, w.rope_theta, w.v_scale)
            ws = torch.empty(mimo.decode_workspace_size(p, S) + 256, dtype=torch.uint8, device=dev)
            o = torch.empty((B, w.num_q_heads, DV), dtype=torch.bfloat16, device=dev)
            out.append((p, q, kn, vn, sk, kc, vc, ws, o))
        return out

    pos = torch.full((B,), S, dtype=torch.int32, device=dev)
    sw = mk_layers(synth.SWA_HEADS, NSW, 15000)
    ga = mk_layers(synth.GA_HEADS, NGA, 15100)

    def decodes(ls):
        def run():
            for (p, q, kn, vn, sk, kc, vc, ws, o) in ls:
                mimo.decode(p, q, kn, vn, pos, S, kc, vc, sinks=sk, out=o, workspace=ws)
        return run

    # the decode workload's batch of 64 (cached lengths uniform in [1024, 32768]; full 128-slot
    # rings), one layer of each kind per replay
    lengths = synth.decode_lengths(3).tolist()
    B64 = len(lengths)
    pos64 = torch.tensor(lengths, dtype=torch.int32, device=dev)

    def mk_b64(heads, seed):
        w = synth.Workload("dec64", B64, 1, dtype=torch.bfloat16, **heads)
        cap = w.window if w.layer_kind == 1 else max(lengths) + 1
        q, kn, vn, sk, kc, vc = synth.decode_inputs(w, seed, B64, cap, device=dev)
        p = mimo.Params(B64, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims, w.layer_kind,
                        w.window, w.rope_theta, w.v_scale)
        ws = torch.empty(mimo.decode_workspace_size(p, max(lengths)) + 256, dtype=torch.uint8,
                         device=dev)
        o = torch.empty((B64, w.num_q_heads, DV), dtype=torch.bfloat16, device=dev)
        return lambda: mimo.decode(p, q, kn, vn, pos64, max(lengths), kc, vc, sinks=sk, out=o,
                                   workspace=ws)

    cases = [("empty_kernel", probes_empty, NSW), ("tile_read_80KiB", probes_read, NSW),
             ("sliding_decode", decodes(sw), NSW), ("global_decode", decodes(ga), NGA),
             ("sliding_decode_b64", mk_b64(synth.SWA_HEADS, 15200), 1),
             ("global_decode_b64", mk_b64(synth.GA_HEADS, 15300), 1)]
    res = {}
    for name, fn, n in cases:
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        for mode in ("cold", "hot"):
            ts = []
            for _ in range(max(args.steps, 5)):
                if mode == "cold":
                    flush.fill_(1)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / n)
            ts.sort()
            res[f"{name}_{mode}_us_per_call"] = round(ts[len(ts) // 2], 3)
    return res


def single_layer(args, dev):
    """Time one layer configuration on its own (profiling aid); prints one JSON line."""
    import torch

    import global_attention_rope_amd as mimo
    from tests import synth

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {"workload": args.workload, "steps": args.steps}
    if args.workload == "decode_latency":
        res.update(decode_latency(args, dev))
    elif args.workload == "gemm":
        # achievable dense bf16 matrix-core rate on this part (hipBLASLt through torch), the
        # practical ceiling next to the nominal peak
        n = 8192
        x = torch.randn((n, n), device=dev).to(torch.bfloat16)
        y = torch.randn((n, n), device=dev).to(torch.bfloat16)
        ms = timed(lambda: torch.mm(x, y), args.steps)
        res.update(ms=ms, tflops=2 * n ** 3 / ms / 1e9)
    elif args.workload == "ceilings":
        # attainable read bandwidth and dense bf16 matrix rate of this part, measured by the probe
        # library's stream-read and MFMA-loop kernels (the practical ceilings beside the nominal
        # 8 TB/s and 2.5 PFLOP/s)
        import ctypes

        from global_attention_rope_amd import build as hb
        probe = ctypes.CDLL(hb.PROBE_LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        probe.mimo_probe_stream_read.argtypes = [vp, i64, i32, vp, i32, vp]
        probe.mimo_probe_mfma.argtypes = [vp, i32, i32, vp]
        cur = lambda: vp(torch.cuda.current_stream().cuda_stream)
        nbytes, G = 2 << 30, 2048
        src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        dst = torch.empty(G * 512, dtype=torch.int32, device=dev)
        for flags, name in ((0, "stream_read"), (1, "stream_read_nontemporal"),
                            (2, "stream_read_slices"), (3, "stream_read_slices_nontemporal")):
            fn = lambda: probe.mimo_probe_stream_read(vp(src.data_ptr()), nbytes, flags,
                                                      vp(dst.data_ptr()), G, cur())
            assert fn() == 0
            ms = timed(fn, args.steps)
            res[name] = dict(ms=ms, bytes=nbytes, GBps=nbytes / ms / 1e6,
                             frac_hbm=nbytes / ms / 1e6 / PEAK_HBM_GBPS)
        iters = 20000
        for groups, name in ((256, "mfma_loop_2_waves_per_simd"), (512, "mfma_loop_4_waves_per_simd")):
            fn = lambda: probe.mimo_probe_mfma(vp(dst.data_ptr()), groups, iters, cur())
            assert fn() == 0
            ms = timed(fn, args.steps)
            f = groups * 8 * iters * 4 * 32768
            res[name] = dict(ms=ms, flop=f, tflops=f / ms / 1e9,
                             frac_mfma=f / ms / 1e9 / PEAK_BF16_TFLOPS)
    elif args.workload == "copy":
        nbytes = 2 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = timed(lambda: dst.copy_(src), args.steps)
        res.update(ms=ms, bytes_read=nbytes, bytes_written=nbytes, GBps=2 * nbytes / ms / 1e6)
    elif args.workload in ("swa_prefill", "ga_prefill"):
        w = synth.SWA_PREFILL if args.workload == "swa_prefill" else synth.GA_PREFILL
        q, k, v, s = synth.layer_inputs(w, 1000 if w.layer_kind else 2000, device=dev)
        p = mimo.Params(w.batch, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims,
                        w.layer_kind, w.window, w.rope_theta, w.v_scale)
        sp = torch.zeros(w.batch, dtype=torch.int32, device=dev)
        out = torch.empty((w.batch, w.seq, w.num_q_heads, DV), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mimo.prefill_workspace_size(p, w.seq) + 256, dtype=torch.uint8, device=dev)
        ms = timed(lambda: mimo.prefill(p, q, k, v, sp, sinks=s, out=out, workspace=ws), args.steps)
        f, b = prefill_counts(w.batch, w.seq, w.num_q_heads, w.num_kv_heads, w.layer_kind,
                              w.window)
        b -= w.batch * (min(w.seq, w.window) if w.layer_kind else w.seq) * w.num_kv_heads * (DQK + DV) * 2
        res.update(ms=ms, tflops=f / ms / 1e9, GBps=b / ms / 1e6, flop=f, bytes=b,
                   frac_mfma=f / ms / 1e9 / PEAK_BF16_TFLOPS, frac_hbm=b / ms / 1e6 / PEAK_HBM_GBPS)
    elif args.workload == "router":
        p = mimo.RouterParams()
        T = synth.ROUTER_TOKENS
        logits, bias = synth.router_inputs(14100, T, p.num_experts, device=dev)
        idx = torch.empty((T, p.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, p.top_k), dtype=torch.float32, device=dev)
        ms = timed(lambda: mimo.router_topk(p, logits, bias, idx, wts), args.steps)
        b = T * p.num_experts * 4 + p.num_experts * 4 + T * p.top_k * 8
        res.update(ms=ms, tokens=T, experts=p.num_experts, bytes=b, GBps=b / ms / 1e6,
                   frac_hbm=b / ms / 1e6 / PEAK_HBM_GBPS)
    elif args.workload == "layer":
        hidden = 4096
        for name, w in (("sliding", synth.SWA_PREFILL), ("global", synth.GA_PREFILL)):
            x, s = synth.layer_input(w, 13000 + w.layer_kind, hidden, device=dev)
            wq, wk, wv, wo = synth.layer_weights(w, 13100 + w.layer_kind, hidden, hidden, device=dev)
            p = mimo.Params(w.batch, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims,
                            w.layer_kind, w.window, w.rope_theta, w.v_scale)
            sp = torch.zeros(w.batch, dtype=torch.int32, device=dev)
            out = torch.empty((w.batch, w.seq, hidden), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mimo.layer_workspace_size(p, hidden, w.seq) + 256, dtype=torch.uint8,
                             device=dev)
            ms = timed(lambda: mimo.layer_prefill(p, x, wq, wk, wv, wo, sp, sinks=s, out=out,
                                                  workspace=ws), args.steps)
            T = w.batch * w.seq
            f_attn, _ = prefill_counts(w.batch, w.seq, w.num_q_heads, w.num_kv_heads, w.layer_kind,
                                       w.window)
            f_proj = 2 * T * hidden * (w.num_q_heads * DQK + w.num_kv_heads * (DQK + DV))
            f_out = 2 * T * w.num_q_heads * DV * hidden
            f = f_attn + f_proj + f_out
            res[name] = dict(ms=ms, tflops=f / ms / 1e9, flop=f, flop_projections=f_proj + f_out,
                             flop_attention=f_attn, frac_mfma=f / ms / 1e9 / PEAK_BF16_TFLOPS)
    elif args.workload == "extend":
        lengths = synth.decode_lengths(3).tolist()
        cases = [("global_chunk", synth.GA_HEADS, [30000], 2048, False),
                 ("sliding_chunk", synth.SWA_HEADS, [30000], 2048, False),
                 ("global_verify4", synth.GA_HEADS, lengths, 4, False),
                 ("sliding_verify4", synth.SWA_HEADS, lengths, 4, False),
                 ("global_chunk_fp8", synth.GA_HEADS, [30000], 2048, True),
                 ("global_verify4_fp8", synth.GA_HEADS, lengths, 4, True)]
        for name, heads, starts, S, fp8 in cases:
            B = len(starts)
            w = synth.Workload(name, B, S, dtype=torch.bfloat16, **heads)
            swa = w.layer_kind == 1
            cap = w.window if swa else max(starts) + S
            q, k, v, s = synth.layer_inputs(w, 8000 + w.layer_kind, device=dev)
            if fp8:
                kc, vc = synth.fp8_cache_contents(w, 8100 + w.layer_kind, B, cap, device=dev)
            else:
                kc, vc = synth.cache_contents(w, 8100 + w.layer_kind, B, cap, device=dev)
            p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims, w.layer_kind,
                            w.window, w.rope_theta, w.v_scale)
            if fp8:
                p.cache_dtype = mimo.CACHE_FP8_E4M3
                p.k_cache_scale, p.v_cache_scale = synth.FP8_K_SCALE, synth.FP8_V_SCALE
            sp = torch.tensor(starts, dtype=torch.int32, device=dev)
            out = torch.empty((B, S, w.num_q_heads, DV), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mimo.extend_workspace_size(p, S, max(starts)) + 256, dtype=torch.uint8,
                             device=dev)
            # the same call repeated: the new tokens' slots are rewritten with the same values
            ms = timed(lambda: mimo.extend(p, q, k, v, sp, max(starts), kc, vc, sinks=s, out=out,
                                           workspace=ws), args.steps)
            f, b = extend_counts(w.num_q_heads, w.num_kv_heads, w.layer_kind, w.window, starts, S,
                                 1 if fp8 else 2)
            res[name] = dict(ms=ms, tflops=f / ms / 1e9, GBps=b / ms / 1e6, flop=f, bytes=b,
                             frac_mfma=f / ms / 1e9 / PEAK_BF16_TFLOPS,
                             frac_hbm=b / ms / 1e6 / PEAK_HBM_GBPS)
    else:
        lengths = synth.decode_lengths(3).tolist()
        B = len(lengths)
        for name, heads, fp8 in (("global", synth.GA_HEADS, False),
                                 ("sliding", synth.SWA_HEADS, False),
                                 ("global_fp8", synth.GA_HEADS, True),
                                 ("sliding_fp8", synth.SWA_HEADS, True)):
            w = synth.Workload(name, B, 1, dtype=torch.bfloat16, **heads)
            swa = w.layer_kind == 1
            cap = w.window if swa else max(lengths) + 1
            if fp8:
                q, kn, vn, s, _, _ = synth.decode_inputs(w, 7000 + w.layer_kind, B, 1, device=dev)
                kc, vc = synth.fp8_cache_contents(w, 7100 + w.layer_kind, B, cap, device=dev)
            else:
                q, kn, vn, s, kc, vc = synth.decode_inputs(w, 7000 + w.layer_kind, B, cap,
                                                           device=dev)
            p = mimo.Params(B, w.num_q_heads, w.num_kv_heads, DQK, DV, w.rope_dims, w.layer_kind,
                            w.window, w.rope_theta, w.v_scale)
            if fp8:
                p.cache_dtype = mimo.CACHE_FP8_E4M3
                p.k_cache_scale, p.v_cache_scale = synth.FP8_K_SCALE, synth.FP8_V_SCALE
            pos = torch.tensor(lengths, dtype=torch.int32, device=dev)
            out = torch.empty((B, w.num_q_heads, DV), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mimo.decode_workspace_size(p, max(lengths)) + 256, dtype=torch.uint8,
                             device=dev)
            # the same step repeated: the appended slot is rewritten with the same values
            ms = timed(lambda: mimo.decode(p, q, kn, vn, pos, max(lengths), kc, vc, sinks=s,
                                           out=out, workspace=ws), args.steps)
            f, b = decode_counts(B, w.num_q_heads, w.num_kv_heads, w.layer_kind, w.window, lengths,
                                 cache_bytes=1 if fp8 else 2)
            res[name] = dict(ms=ms, GBps=b / ms / 1e6, bytes=b, tflops=f / ms / 1e9,
                             frac_hbm=b / ms / 1e6 / PEAK_HBM_GBPS)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
