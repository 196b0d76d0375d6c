"""GPU parity of extend (chunked prefill): new tokens against a cache of earlier ones.

Two kinds of check, both against the fp64 oracle:
  * a synthetic cache (N(0,1) rotated keys and values, laid out as the linear cache or the ring
    holds them) with several start offsets per batch: the outputs against the oracle's extend,
    which takes the same cache as a position-keyed list, and the caches afterwards (new rotated
    keys and values in their slots, every other slot untouched);
  * a full-size prompt cut into chunks (prefill, then extends of the cache the previous chunks
    left) against the oracle's prefill of the whole prompt.
Seeds: 5000 + case.
"""
import numpy as np
import pytest
import torch

import global_attention_rope_amd as mimo
import oracle
from tests import rounding_model, synth
from tests.gpu_helpers import assert_close, prefill_bound_for, ring_positions, to_np64
from tests.test_gpu_parity import _f32, _note, _oparams, _params, _wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_cache(w, kc, vc, starts):
    """The cache as the oracle takes it: per sequence the entries that hold a position before
    its start, first, with their positions and count."""
    kc_h, vc_h = kc.to("cpu", torch.float32).numpy(), vc.to("cpu", torch.float32).numpy()
    B, cap = kc.shape[0], kc.shape[2]
    L = max(1, cap)
    okc = np.zeros((B, w.num_kv_heads, L, w.qk_head_dim), np.float32)
    ovc = np.zeros((B, w.num_kv_heads, L, w.v_head_dim), np.float32)
    kpos = np.full((B, L), -1, np.int32)
    count = np.zeros(B, np.int32)
    for b, st in enumerate(starts):
        if w.layer_kind == 1:
            pos = ring_positions(st, w.window)
        else:
            pos = np.where(np.arange(cap) < st, np.arange(cap), -1)
        slots = np.nonzero(pos >= 0)[0]
        n = len(slots)
        okc[b, :, :n] = kc_h[b][:, slots]
        ovc[b, :, :n] = vc_h[b][:, slots]
        kpos[b, :n] = pos[slots]
        count[b] = n
    return okc, ovc, kpos, count


def _stored_slots(w, st, S):
    """Cache slot of each new token that the extend stores (token index -> slot)."""
    if w.layer_kind == 1:
        return {i: (st + i) % w.window for i in range(max(0, S - w.window), S)}
    return {i: st + i for i in range(S)}


CASES = [
    dict(kind=1, B=3, S=100, Hq=16, Hkv=2, sinks=True, starts=[0, 50, 1000]),   # S < W
    dict(kind=1, B=2, S=300, Hq=8, Hkv=2, sinks=True, starts=[5, 4000]),        # S > W, start < W
    dict(kind=1, B=1, S=1, Hq=8, Hkv=1, sinks=False, starts=[333], W=200),      # one token
    dict(kind=1, B=2, S=77, Hq=8, Hkv=8, sinks=True, starts=[0, 9], W=1),
    dict(kind=1, B=1, S=130, Hq=8, Hkv=2, sinks=True, starts=[64], W=4096),     # ring not full
    dict(kind=0, B=3, S=129, Hq=16, Hkv=1, sinks=False, starts=[0, 37, 700]),
    dict(kind=0, B=2, S=1, Hq=8, Hkv=2, sinks=True, starts=[5, 1234]),
    dict(kind=0, B=1, S=300, Hq=8, Hkv=2, sinks=False, starts=[64]),            # tile-aligned
    # up to 16 new tokens: the multi-token tile kernel ((head, token) query columns)
    dict(kind=1, B=3, S=4, Hq=16, Hkv=2, sinks=True, starts=[0, 2, 1000]),       # start < W
    dict(kind=1, B=2, S=16, Hq=8, Hkv=1, sinks=True, starts=[126, 131], W=128),
    dict(kind=1, B=2, S=7, Hq=8, Hkv=8, sinks=False, starts=[0, 9], W=1),
    dict(kind=1, B=2, S=3, Hq=8, Hkv=2, sinks=True, starts=[0, 500]),          # 16 columns, 1 split
    dict(kind=0, B=3, S=2, Hq=16, Hkv=1, sinks=False, starts=[0, 255, 4097]),
    dict(kind=0, B=2, S=16, Hq=8, Hkv=2, sinks=True, starts=[1, 700]),
    dict(kind=0, B=1, S=5, Hq=64, Hkv=4, sinks=False, starts=[20000]),           # split partials
    # 118 splits: the combine reads past its first prefetch block of 96 (with a sink)
    dict(kind=0, B=1, S=4, Hq=64, Hkv=4, sinks=True, starts=[30000]),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_extend_against_synthetic_cache(ci):
    run_extend_case(CASES[ci], 5000 + ci)


def run_extend_case(case, seed, q_scale=1.0):
    """One extend call on a synthetic cache: outputs and caches afterwards against the oracle."""
    case = dict(case)
    starts = case.pop("starts")
    w = _wl(**case)
    S = w.seq
    _note(f"extend {case} starts {starts}")
    q, k, v, s = synth.layer_inputs(w, seed, device=DEV)
    if q_scale != 1.0:
        q = q * q_scale  # a power of two: exact in bf16
    cap = w.window if w.layer_kind == 1 else max(starts) + S + 5
    kc, vc = synth.cache_contents(w, seed + 100, w.batch, cap, device=DEV)
    kc0, vc0 = to_np64(kc), to_np64(vc)
    okc, ovc, kpos, count = _oracle_cache(w, kc, vc, starts)
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = mimo.extend(_params(w), q, k, v, sp, max(starts), kc, vc, sinks=s)
    torch.cuda.synchronize()
    ref, krot = oracle.extend(_oparams(w), _f32(q), _f32(k), _f32(v), np.array(starts, np.int32),
                              okc, ovc, kpos, count, _f32(s), want_k_rot=True)
    bound = rounding_model.extend_bound(_oparams(w), _f32(q), _f32(k), _f32(v), starts, okc, ovc,
                                        kpos, count, _f32(s))
    assert_close(out, ref, what=f"extend out {case}", bound=bound)

    # caches: the new tokens in their slots, every other slot as it was
    kc1, vc1, v_h = to_np64(kc), to_np64(vc), to_np64(v)
    for b, st in enumerate(starts):
        slots = _stored_slots(w, st, S)
        kept = np.setdiff1d(np.arange(cap), list(slots.values()))
        assert np.array_equal(kc1[b][:, kept], kc0[b][:, kept]), f"seq {b}: foreign K slot changed"
        assert np.array_equal(vc1[b][:, kept], vc0[b][:, kept]), f"seq {b}: foreign V slot changed"
        tok = np.array(sorted(slots)), np.array([slots[i] for i in sorted(slots)])
        assert np.array_equal(vc1[b][:, tok[1]], v_h[b, tok[0]].transpose(1, 0, 2))
        assert_close(kc1[b][:, tok[1]], krot[b, tok[0]].transpose(1, 0, 2), what=f"seq {b} K")


@pytest.mark.parametrize("kind,S", [(0, 40), (1, 40), (0, 3), (1, 3)])
def test_extend_skips_sequences_past_max_start(kind, S):
    w = _wl(kind=kind, B=2, S=S, Hq=8, Hkv=2, sinks=kind == 1)
    starts, max_start = [10, 500], 100
    _note(f"extend skip kind={kind} S={S}")
    q, k, v, s = synth.layer_inputs(w, 5200 + kind, device=DEV)
    cap = w.window if kind == 1 else max_start + w.seq
    kc, vc = synth.cache_contents(w, 5300 + kind, w.batch, cap, device=DEV)
    kc0, vc0 = kc.clone(), vc.clone()
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = torch.full((2, w.seq, w.num_q_heads, w.v_head_dim), 3.0, dtype=w.dtype, device=DEV)
    mimo.extend(_params(w), q, k, v, sp, max_start, kc, vc, sinks=s, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[1]) == 0, "skipped sequence must get a zero output"
    assert torch.equal(kc[1], kc0[1]) and torch.equal(vc[1], vc0[1]), "skipped sequence stored"
    okc, ovc, kpos, count = _oracle_cache(w, kc0[:1], vc0[:1], starts[:1])
    ref = oracle.extend(_oparams(w, batch=1), _f32(q[:1]), _f32(k[:1]), _f32(v[:1]),
                        np.array(starts[:1], np.int32), okc, ovc, kpos, count, _f32(s))
    bound = rounding_model.extend_bound(_oparams(w, batch=1), _f32(q[:1]), _f32(k[:1]),
                                        _f32(v[:1]), starts[:1], okc, ovc, kpos, count, _f32(s))
    assert_close(out[:1], ref, what="accepted sequence", bound=bound)


def _chunked(w, q, k, v, s, chunks, cap):
    """Prefill of the first chunk, then extends; returns the concatenated output and caches."""
    B = w.batch
    kc = torch.zeros((B, w.num_kv_heads, cap, w.qk_head_dim), dtype=w.dtype, device=DEV)
    vc = torch.zeros((B, w.num_kv_heads, cap, w.v_head_dim), dtype=w.dtype, device=DEV)
    p = _params(w)
    outs, at = [], 0
    for n, c in enumerate(chunks):
        sl = slice(at, at + c)
        sp = torch.full((B,), at, dtype=torch.int32, device=DEV)
        qc, kk, vv = q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous()
        if n == 0:
            outs.append(mimo.prefill(p, qc, kk, vv, sp, sinks=s, k_cache=kc, v_cache=vc))
        else:
            outs.append(mimo.extend(p, qc, kk, vv, sp, at, kc, vc, sinks=s))
        at += c
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), kc, vc


def test_chunked_prefill_sliding_full_size():
    w = synth.SWA_PREFILL
    chunks = [1000, 1048, 37, 2011]
    _note(f"{w.name} chunks {chunks}")
    q, k, v, s = synth.layer_inputs(w, 5400, device=DEV)
    out, kc, vc = _chunked(w, q, k, v, s, chunks, w.window)
    pos = np.arange(w.seq, dtype=np.int32)[None]
    ref, krot = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s), want_k_rot=True)
    assert_close(out, ref, what=f"{w.name} chunked", bound=prefill_bound_for(w, q, k, v, s, pos))
    # the ring holds the prompt's last window tokens, as a single prefill leaves it
    last = np.arange(w.seq - w.window, w.seq)
    assert np.array_equal(to_np64(vc)[0][:, last % w.window], to_np64(v)[0, last].transpose(1, 0, 2))
    assert_close(to_np64(kc)[0][:, last % w.window], krot[0, last].transpose(1, 0, 2), what="ring K")


def test_chunked_prefill_global_full_size_sampled_rows():
    w = synth.GA_PREFILL
    chunks = [2053, 4096, 2043]
    _note(f"{w.name} chunks {chunks}")
    q, k, v, s = synth.layer_inputs(w, 5500, device=DEV)
    out, kc, vc = _chunked(w, q, k, v, s, chunks, w.seq)
    rng = np.random.default_rng(5)
    bounds = np.cumsum([0] + chunks)
    rows = np.unique(np.concatenate([bounds[:-1], bounds[1:] - 1, bounds[1:-1] - 2, bounds[1:-1] + 1,
                                     rng.integers(0, w.seq, 96)])).astype(np.int32)
    pos = np.arange(w.seq, dtype=np.int32)[None]
    ref = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s), rows=rows)
    bound = prefill_bound_for(w, q, k, v, s, pos, rows=rows)
    assert_close(out[:, rows], ref[:, rows], what=f"{w.name} chunked", bound=bound[:, rows])


def test_extend_global_long_cache_sampled_rows():
    """A 2048-token chunk after 30000 cached positions (decode-length context), 64 query heads."""
    w = _wl(kind=0, B=1, S=2048, Hq=64, Hkv=4, sinks=False)
    start = 30000
    _note(f"extend long cache start {start} S {w.seq}")
    q, k, v, s = synth.layer_inputs(w, 5600, device=DEV)
    kc, vc = synth.cache_contents(w, 5601, 1, start + w.seq, device=DEV)
    okc, ovc, kpos, count = _oracle_cache(w, kc, vc, [start])
    sp = torch.tensor([start], dtype=torch.int32, device=DEV)
    out = mimo.extend(_params(w), q, k, v, sp, start, kc, vc)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 1000, 2046, 2047], np.int32)
    ref = oracle.extend(_oparams(w), _f32(q), _f32(k), _f32(v), np.array([start], np.int32), okc,
                        ovc, kpos, count, None, rows=rows)
    assert_close(out[:, rows], ref[:, rows], what="long cache")


def test_extend_four_tokens_mixed_lengths_all_sequences():
    """Four new tokens per sequence over 64 global-layer caches of mixed lengths (300..18000, some
    at a split boundary): the key rows are cut into splits whose partials the combine merges, and
    short sequences' later splits are empty.  The oracle checks every sequence."""
    w = _wl(kind=0, B=64, S=4, Hq=16, Hkv=4, sinks=False)
    rng = np.random.default_rng(12)
    starts = [300, 18000, 9020, 9021, 9019] + rng.integers(300, 18001, size=59).tolist()
    B = len(starts)
    cap = max(starts) + w.seq
    _note(f"extend 4 tokens many splits B={B}")
    q, k, v, _ = synth.layer_inputs(w, 5900, device=DEV)
    kc, vc = synth.cache_contents(w, 5901, B, cap, device=DEV)
    pre = (kc.clone(), vc.clone())
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = mimo.extend(_params(w), q, k, v, sp, max(starts), kc, vc)
    torch.cuda.synchronize()
    for b in range(B):
        okc, ovc, kpos, count = _oracle_cache(w, pre[0][b:b + 1], pre[1][b:b + 1], [starts[b]])
        ref = oracle.extend(_oparams(w, batch=1), _f32(q[b:b + 1]), _f32(k[b:b + 1]), _f32(v[b:b + 1]),
                            np.array([starts[b]], np.int32), okc, ovc, kpos, count, None)
        assert_close(out[b:b + 1], ref, what=f"seq {b} start {starts[b]}")


@pytest.mark.parametrize("kind", [0, 1])
def test_extend_four_tokens_batch64_full_size(kind):
    """Four new tokens per sequence after the decode workload's cached lengths (batch 64, uniform
    in [1024, 32768]): sampled sequences (global) or all of them (sliding) against the oracle."""
    Hkv = 4 if kind == 0 else 8
    w = _wl(kind=kind, B=synth.DECODE_BATCH, S=4, Hq=64, Hkv=Hkv, sinks=kind == 1)
    starts = synth.decode_lengths(3 + kind).tolist()
    B = len(starts)
    cap = w.window if kind == 1 else max(starts) + w.seq
    _note(f"extend 4 tokens B={B} kind={kind}")
    q, k, v, s = synth.layer_inputs(w, 5700 + kind, device=DEV)
    kc, vc = synth.cache_contents(w, 5800 + kind, B, cap, device=DEV)
    sample = list(range(B)) if kind == 1 else sorted({int(np.argmin(starts)), int(np.argmax(starts)), 5, 17, 42})
    pre = {b: (kc[b:b + 1].clone(), vc[b:b + 1].clone()) for b in sample}
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = mimo.extend(_params(w), q, k, v, sp, max(starts), kc, vc, sinks=s)
    torch.cuda.synchronize()
    for b in sample:
        okc, ovc, kpos, count = _oracle_cache(w, pre[b][0], pre[b][1], [starts[b]])
        ref = oracle.extend(_oparams(w, batch=1), _f32(q[b:b + 1]), _f32(k[b:b + 1]), _f32(v[b:b + 1]),
                            np.array([starts[b]], np.int32), okc, ovc, kpos, count, _f32(s))
        assert_close(out[b:b + 1], ref, what=f"seq {b} start {starts[b]}")
