"""Accuracy and oracle time per workload: the HIP library against the fp64 oracle on each of the
five workloads at full size, with the host oracle timed on the same inputs.

Run on a GPU machine from the repository root:  python -m tests.accuracy_table [out.md]
Prints one line per workload and writes a markdown table (and a JSON copy beside it).

Columns: max |gpu - oracle|; relative L2 error; elements above the literal 1e-2 absolute bound
and above the allclose form 1e-2 + 2e-2 |oracle|; the rounding model's relative L2 error (ideal
bf16 arithmetic, tests/rounding_model.py) where it is computed; the oracle's wall time on the
host's OpenMP threads and its fp64 rate; the GPU time of one call (HIP events, warm).
The stack row is measured on sampled rows and sequences; its oracle time for the whole stack is
extrapolated from the measured per-row cost and labelled so.
"""
from __future__ import annotations

import json
import os
import platform
import sys
import time

import numpy as np
import torch

import global_attention_rope_amd as mimo
import oracle
from oracle import OracleParams
from tests import rounding_model, synth

DEV = "cuda:0"
DQK, DV = 192, 128


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _f32(t):
    return None if t is None else t.to("cpu", torch.float32).numpy()


def _params(w, B=None):
    return mimo.Params(batch=w.batch if B is None else B, num_q_heads=w.num_q_heads,
                       num_kv_heads=w.num_kv_heads, qk_head_dim=w.qk_head_dim,
                       v_head_dim=w.v_head_dim, rope_dims=w.rope_dims, layer_kind=w.layer_kind,
                       window=w.window, rope_theta=w.rope_theta, v_scale=w.v_scale,
                       dtype=mimo.BF16 if w.dtype == torch.bfloat16 else mimo.F32)


def _oparams(w, B=None):
    return OracleParams(w.batch if B is None else B, w.num_q_heads, w.num_kv_heads,
                        w.qk_head_dim, w.v_head_dim, w.rope_dims, w.layer_kind, w.window,
                        w.rope_theta, w.v_scale)


def _gpu_ms(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _errs(gpu, ref, model=None):
    g = gpu.to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) else gpu
    sel = np.isfinite(ref)
    d = np.abs(g[sel] - ref[sel])
    r = {"max_abs": float(d.max()), "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref[sel])),
         "n": int(d.size), "above_1e-2": int(np.count_nonzero(d > 1e-2)),
         "above_allclose": int(np.count_nonzero(d > 1e-2 + 2e-2 * np.abs(ref[sel])))}
    if model is not None:
        r["model_rel_l2"] = rounding_model.rel_l2(model[sel], ref[sel])
    return r


def _prefill_flops(B, S, Hq, kind, W):
    if kind == 0:
        pairs = S * (S + 1) // 2
    else:
        pairs = sum(min(i + 1, W) for i in range(S))
    return B * Hq * pairs * 2 * (DQK + DV)


def row_prefill(name, w, seed, rows=None, model_rows=None):
    """model_rows: rows the rounding model computes (all of the oracle's when None)."""
    q, k, v, s = synth.layer_inputs(w, seed, device=DEV)
    sp = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    p = _params(w)
    out = mimo.prefill(p, q, k, v, sp, sinks=s)
    torch.cuda.synchronize()
    ms = _gpu_ms(lambda: mimo.prefill(p, q, k, v, sp, sinks=s))
    out = out.to("cpu", torch.float64).numpy()
    pos = np.stack([np.arange(w.seq, dtype=np.int32)] * w.batch)
    fq, fk, fv, fs = _f32(q), _f32(k), _f32(v), _f32(s)
    t0 = time.perf_counter()
    ref = oracle.prefill(_oparams(w), fq, fk, fv, pos, fs, rows=rows)
    dt = time.perf_counter() - t0
    model = None
    if w.dtype == torch.bfloat16:
        mrows = rows if model_rows is None else model_rows
        model = rounding_model.prefill(_oparams(w), fq, fk, fv, pos, fs, rows=mrows)
        if model_rows is not None:   # the model's rows only, for its column
            r = _errs(out[:, mrows], ref[:, mrows], model[:, mrows])
            model = np.full(ref.shape, np.nan)
            mr = r["model_rel_l2"]
    flops = _prefill_flops(w.batch, w.seq, w.num_q_heads, w.layer_kind, w.window)
    if rows is not None:
        flops = flops * len(rows) / w.seq   # (approximate: rows are sampled uniformly)
    e = _errs(out, ref, None if model_rows is not None else model)
    if model_rows is not None:
        e["model_rel_l2"] = mr
    return dict(workload=name, **e, oracle_s=dt, oracle_gflops=flops / dt / 1e9, gpu_ms=ms,
                oracle_rows="all" if rows is None else f"{len(rows)} sampled rows")


def row_decode(name, kind, seed):
    Hkv = 4 if kind == 0 else 8
    heads = synth.GA_HEADS if kind == 0 else synth.SWA_HEADS
    B = synth.DECODE_BATCH
    w = synth.Workload(name, B, 1, dtype=torch.bfloat16, **heads)
    positions = synth.decode_lengths(3 + kind).tolist()
    cap = w.window if kind == 1 else max(positions) + 1
    q, kn, vn, s, kc, vc = synth.decode_inputs(w, seed, B, cap, device=DEV)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    p = _params(w, B)
    # the oracle reads the cache as it was before the step appended to it
    if kind == 1:
        kc0, vc0 = _f32(kc), _f32(vc)
    out = mimo.decode(p, q, kn, vn, pos_t, max(positions), kc, vc, sinks=s)
    torch.cuda.synchronize()
    ms = _gpu_ms(lambda: mimo.decode(p, q, kn, vn, pos_t, max(positions), kc, vc, sinks=s))
    ref = np.zeros((B, w.num_q_heads, DV))
    model = np.zeros_like(ref)
    dt = 0.0
    flops = 0
    for b, P in enumerate(positions):
        if kind == 1:
            held = np.arange(P - (w.window - 1), P)
            slots = held % w.window
            kcb, vcb = kc0[b:b + 1][:, :, slots], vc0[b:b + 1][:, :, slots]
            kpos = held[None].astype(np.int32)
        else:
            # (slots 0..P-1 are untouched by the step, which wrote slot P)
            kcb = _f32(kc[b:b + 1, :, :P])
            vcb = _f32(vc[b:b + 1, :, :P])
            kpos = np.arange(P, dtype=np.int32)[None]
        args = (_oparams(w, 1), _f32(q[b:b + 1]), _f32(kn[b:b + 1]), _f32(vn[b:b + 1]),
                np.array([P], np.int32), kcb, vcb, kpos, np.array([kpos.shape[1]], np.int32),
                _f32(s))
        t0 = time.perf_counter()
        ref[b:b + 1] = oracle.decode(*args)
        dt += time.perf_counter() - t0
        model[b:b + 1] = rounding_model.decode(*args)
        flops += w.num_q_heads * (kpos.shape[1] + 1) * 2 * (DQK + DV)
    return dict(workload=name, **_errs(out, ref, model), oracle_s=dt,
                oracle_gflops=flops / dt / 1e9, gpu_ms=ms, oracle_rows="all 64 sequences")


def row_stack(seed_base=4000):
    """Layers 0 (global) and 1 (sliding) of the stack at full size on sampled rows, then the
    oracle's per-row cost extrapolated to the 48-layer prefill (8 global + 40 sliding layers)."""
    B, S = synth.STACK_BATCH, synth.STACK_SEQ
    out_rows, res = {}, []
    total_est = 0.0
    for layer, heads, nl in ((0, synth.GA_HEADS, 8), (1, synth.SWA_HEADS, 40)):
        w = synth.Workload("stack", B, S, dtype=torch.bfloat16, **heads)
        rng = np.random.default_rng(layer)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(S - 16, S),
                                         rng.integers(0, S, 32)])).astype(np.int32)
        r = row_prefill(f"stack layer {layer}", w, seed_base + layer, rows=rows)
        res.append(r)
        # per-row cost grows with the keys a row sees: scale by the visible pairs
        seen = (rows + 1).sum() if heads is synth.GA_HEADS else np.minimum(rows + 1, 128).sum()
        allp = S * (S + 1) // 2 if heads is synth.GA_HEADS else sum(min(i + 1, 128) for i in range(S))
        total_est += nl * r["oracle_s"] / B * B * allp / seen
    keys = ("max_abs", "rel_l2", "model_rel_l2")
    agg = {k: max(r[k] for r in res) for k in keys}
    agg.update(n=sum(r["n"] for r in res), above_1e_2=sum(r["above_1e-2"] for r in res),
               above_allclose=sum(r["above_allclose"] for r in res))
    return dict(workload="48-layer stack (layers 0 and 1, sampled rows)", max_abs=agg["max_abs"],
                rel_l2=agg["rel_l2"], model_rel_l2=agg["model_rel_l2"], n=agg["n"],
                **{"above_1e-2": agg["above_1e_2"], "above_allclose": agg["above_allclose"]},
                oracle_s=total_est, oracle_gflops=9.481e13 / total_est / 1e9,
                gpu_ms=float("nan"),
                oracle_rows="extrapolated to the whole 48-layer prefill from 2 x 64 sampled rows")


def main():
    out_md = sys.argv[1] if len(sys.argv) > 1 else "gpurun_out/accuracy.md"
    cores = oracle.num_threads()
    cpu = _cpu_model()
    rows = []

    def emit(r):
        rows.append(r)
        print(json.dumps(r), flush=True)

    emit(row_prefill("tiny sliding layer, fp32 (B1 S64)", synth.TINY_SWA, 0))
    emit(row_prefill("sliding prefill B1 S4096", synth.SWA_PREFILL, 1000))
    rng = np.random.default_rng(2)
    mrows = np.unique(np.concatenate([np.arange(64), np.arange(8192 - 64, 8192),
                                      rng.integers(0, 8192, 384)])).astype(np.int32)
    emit(row_prefill("global prefill B1 S8192", synth.GA_PREFILL, 2000, model_rows=mrows))
    emit(row_decode("decode B64, global layer", 0, 7000))
    emit(row_decode("decode B64, sliding layer", 1, 8000))
    emit(row_stack())
    os.makedirs(os.path.dirname(out_md) or ".", exist_ok=True)
    with open(out_md, "w") as f:
        f.write(f"Oracle host: {cpu}, {cores} OpenMP threads.\n\n")
        f.write("| workload | max abs | rel L2 | model rel L2 | > 1e-2 abs | outside allclose | "
                "elements | oracle s | oracle GFLOP/s (fp64) | oracle rows | GPU ms |\n")
        f.write("|---|---:|---:|---:|---:|---:|---:|---:|---:|---|---:|\n")
        for r in rows:
            f.write(f"| {r['workload']} | {r['max_abs']:.3e} | {r['rel_l2']:.3e} | "
                    f"{r.get('model_rel_l2', float('nan')):.3e} | {r['above_1e-2']} | "
                    f"{r['above_allclose']} | {r['n']} | {r['oracle_s']:.2f} | "
                    f"{r['oracle_gflops']:.1f} | {r['oracle_rows']} | {r['gpu_ms']:.3f} |\n")
    with open(os.path.splitext(out_md)[0] + ".json", "w") as f:
        json.dump(dict(cpu_model=cpu, cores=cores, rows=rows), f, indent=1)
    print(f"wrote {out_md}", flush=True)


if __name__ == "__main__":
    main()
