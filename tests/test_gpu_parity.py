"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by element.

Small cases span several tiles with ragged tails and the band edges; full-size workloads are
compared whole where the oracle finishes in seconds, else on sampled rows.  Seeds: 1000 * case +
layer.  Tolerances in tests/gpu_helpers.py.
"""
import numpy as np
import pytest
import torch

import global_attention_rope_amd as mimo
import oracle
from oracle import OracleParams
from tests import synth
from tests import rounding_model
from tests.gpu_helpers import (assert_close, assert_near_model, prefill_bound_for, ring_positions,
                               to_np64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _note(msg):
    print(f"[case] {msg}", flush=True)


def _wl(kind, B, S, Hq, Hkv, sinks, W=128, theta=None, r=64, dtype=torch.bfloat16, dqk=192,
        dv=128, hidden=4096):
    return synth.Workload("case", batch=B, seq=S, num_q_heads=Hq, num_kv_heads=Hkv, qk_head_dim=dqk,
                          v_head_dim=dv, rope_dims=r,
                          rope_theta=theta if theta else (1e4 if kind == 1 else 5e6),
                          layer_kind=kind, window=W if kind == 1 else 0, sinks=sinks,
                          hidden=hidden, dtype=dtype)


def _params(w, batch=None):
    return mimo.Params(batch=w.batch if batch is None else batch, num_q_heads=w.num_q_heads,
                       num_kv_heads=w.num_kv_heads, qk_head_dim=w.qk_head_dim,
                       v_head_dim=w.v_head_dim, rope_dims=w.rope_dims, layer_kind=w.layer_kind,
                       window=w.window, rope_theta=w.rope_theta, v_scale=w.v_scale,
                       dtype=mimo.BF16 if w.dtype == torch.bfloat16 else mimo.F32)


def _oparams(w, batch=None):
    return OracleParams(batch=w.batch if batch is None else batch, num_q_heads=w.num_q_heads,
                        num_kv_heads=w.num_kv_heads, qk_head_dim=w.qk_head_dim,
                        v_head_dim=w.v_head_dim, rope_dims=w.rope_dims, layer_kind=w.layer_kind,
                        window=w.window, rope_theta=w.rope_theta, v_scale=w.v_scale)


def _f32(t):
    return None if t is None else t.to("cpu", torch.float32).numpy()


def _run_prefill(w, seed, starts, rows=None, with_cache=False, cap=None, q_scale=1.0):
    q, k, v, s = synth.layer_inputs(w, seed, device=DEV)
    if q_scale != 1.0:
        q = q * q_scale  # a power of two: exact in bf16
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    kc = vc = None
    if with_cache:
        cap = cap if cap else (w.window if w.layer_kind == 1 else max(starts) + w.seq + 7)
        kc = torch.full((w.batch, w.num_kv_heads, cap, w.qk_head_dim), 7.0, dtype=w.dtype, device=DEV)
        vc = torch.full((w.batch, w.num_kv_heads, cap, w.v_head_dim), 7.0, dtype=w.dtype, device=DEV)
    out = mimo.prefill(_params(w), q, k, v, sp, sinks=s, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    pos = np.stack([np.arange(w.seq, dtype=np.int32) + st for st in starts])
    ref = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s), rows=rows,
                         want_k_rot=with_cache)
    return (q, k, v, s, out, ref, kc, vc, pos)


# ----------------------------------------------------------------------------- prefill


def test_tiny_swa_fp32_full():
    w = synth.TINY_SWA
    _note(w.name)
    *_, out, ref, _, _, _ = _run_prefill(w, seed=0, starts=[0])
    assert_close(out, ref, fp32=True, what=w.name)


@pytest.mark.parametrize("case", [
    dict(kind=1, B=2, S=300, Hq=16, Hkv=2, sinks=True, starts=[0, 1000]),
    dict(kind=1, B=1, S=77, Hq=8, Hkv=8, sinks=True, starts=[5], W=1),
    dict(kind=1, B=1, S=260, Hq=8, Hkv=1, sinks=False, starts=[0], W=200),
    dict(kind=1, B=2, S=130, Hq=8, Hkv=2, sinks=True, starts=[3, 0], W=4096),
    dict(kind=1, B=1, S=190, Hq=8, Hkv=4, sinks=True, starts=[0], W=65, r=0),
    dict(kind=0, B=2, S=333, Hq=16, Hkv=1, sinks=False, starts=[0, 20000]),
    dict(kind=0, B=1, S=129, Hq=8, Hkv=2, sinks=True, starts=[7]),
    dict(kind=0, B=1, S=1, Hq=4, Hkv=4, sinks=False, starts=[0]),
    # every dim rotated (each rotated dim adds a bf16 rounding of an operand)
    dict(kind=0, B=1, S=257, Hq=8, Hkv=2, sinks=False, starts=[0], r=192),
    # sliding layers whose GQA group is a multiple of 4 run the grouped kernel, which builds a
    # cos/sin table of the rows' positions: at the widest rotation (every dim, its rows packed)
    # and with no rotation at all
    dict(kind=1, B=1, S=200, Hq=8, Hkv=2, sinks=True, starts=[3], r=192),
    dict(kind=1, B=2, S=150, Hq=8, Hkv=2, sinks=True, starts=[0, 300], r=0),
])
def test_prefill_bf16_small(case):
    case = dict(case)
    starts = case.pop("starts")
    w = _wl(**case)
    _note(str(case))
    q, k, v, s, out, ref, _, _, pos = _run_prefill(w, seed=1000 + w.seq, starts=starts)
    bound = rounding_model.prefill_bound(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_close(out, ref, what=str(case), bound=bound)
    model = rounding_model.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_near_model(out, ref, model, what=str(case))


def test_prefill_swa_full_size_all_rows():
    w = synth.SWA_PREFILL
    _note(w.name)
    q, k, v, s, out, ref, _, _, pos = _run_prefill(w, seed=1000, starts=[0])
    assert_close(out, ref, what=w.name, bound=prefill_bound_for(w, q, k, v, s, pos))
    model = rounding_model.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_near_model(out, ref, model, what=w.name)


def test_prefill_global_full_size_sampled_rows():
    w = synth.GA_PREFILL
    _note(w.name)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.seq - 64, w.seq),
                                     rng.integers(0, w.seq, 128)])).astype(np.int32)
    q, k, v, s, out, ref, _, _, pos = _run_prefill(w, seed=2000, starts=[0], rows=rows)
    bound = prefill_bound_for(w, q, k, v, s, pos, rows=rows)
    assert_close(out[:, rows], ref[:, rows], what=w.name, bound=bound[:, rows])
    model = rounding_model.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s), rows=rows)
    assert_near_model(to_np64(out)[:, rows], ref[:, rows], model[:, rows], what=w.name)


@pytest.mark.parametrize("kind", [0, 1])
def test_prefill_writes_caches(kind):
    w = _wl(kind=kind, B=2, S=200, Hq=8, Hkv=2, sinks=kind == 1, W=128)
    starts = [0, 50]
    _note(f"cache kind={kind}")
    q, k, v, s, out, (ref, krot), kc, vc, pos = _run_prefill(w, seed=3000 + kind, starts=starts,
                                                             with_cache=True)
    assert_close(out, ref, what="out", bound=prefill_bound_for(w, q, k, v, s, pos))
    kc_h, vc_h = to_np64(kc), to_np64(vc)
    v_h = to_np64(v)
    cap = kc.shape[2]
    for b in range(w.batch):
        written = set()
        for i in range(w.seq):
            p = int(pos[b, i])
            if kind == 1 and i < w.seq - w.window:
                continue
            slot = p % w.window if kind == 1 else p
            written.add(slot)
            # rotated key: bf16 rounding of the exact rotation
            exp = krot[b, i]
            np.testing.assert_allclose(kc_h[b, :, slot], exp, rtol=2 ** -8, atol=1e-6)
            # value: copied bit for bit
            assert np.array_equal(vc_h[b, :, slot], v_h[b, i])
        untouched = [sl for sl in range(cap) if sl not in written]
        assert all((kc_h[b, :, sl] == 7.0).all() and (vc_h[b, :, sl] == 7.0).all() for sl in untouched)


@pytest.mark.parametrize("kind,Hq,Hkv", [(0, 16, 2), (1, 8, 8), (1, 16, 2)])
def test_prefill_late_keys_outgrow_the_reference(kind, Hq, Hkv, monkeypatch):
    """Keys past the first 64-key tile scaled by 16 (exact in bf16): a row's later scores exceed
    its first tile's maximum by tens of binary orders, so the reference each row took on its first
    keys must move mid-row (the global kernel and the sliding one for GQA groups that are not a
    multiple of 4 find this from the weights' sums and compute the tile's scores again; the
    16-row sliding kernel from its row maxima).  Scores this large and this peaked turn the bf16
    rounding of the operands into output errors of ~0.2 (ideal bf16 arithmetic, the rounding
    model, lands on the same values), past the fixed 1e-2 bound: every row gets the derived bound."""
    monkeypatch.setattr(rounding_model, "BOUND_MAX_KEYS", 512)
    w = _wl(kind=kind, B=1, S=300, Hq=Hq, Hkv=Hkv, sinks=kind == 1, W=200)
    _note(f"late keys x16 kind={kind} Hq={Hq} Hkv={Hkv}")
    q, k, v, s = synth.layer_inputs(w, 4100 + kind, device=DEV)
    k = k.clone()
    k[:, 64:] *= 16.0
    sp = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mimo.prefill(_params(w), q, k, v, sp, sinks=s)
    torch.cuda.synchronize()
    pos = np.arange(w.seq, dtype=np.int32)[None]
    ref = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert np.isfinite(to_np64(out)).all()
    assert_close(out, ref, what="late keys", bound=prefill_bound_for(w, q, k, v, s, pos))
    model = rounding_model.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_near_model(out, ref, model, what="late keys")


def test_prefill_deterministic():
    w = _wl(kind=0, B=1, S=500, Hq=16, Hkv=1, sinks=False)
    q, k, v, s = synth.layer_inputs(w, 4000, device=DEV)
    sp = torch.zeros(1, dtype=torch.int32, device=DEV)
    a = mimo.prefill(_params(w), q, k, v, sp, sinks=s)
    b = mimo.prefill(_params(w), q, k, v, sp, sinks=s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_empty_and_invalid_arguments():
    w = _wl(kind=1, B=1, S=0, Hq=8, Hkv=1, sinks=True)
    q, k, v, s = synth.layer_inputs(w, 1, device=DEV)
    sp = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mimo.prefill(_params(w), q, k, v, sp, sinks=s)
    assert out.shape[1] == 0
    bad = _params(w)
    bad.rope_dims = 63
    w2 = _wl(kind=1, B=1, S=16, Hq=8, Hkv=1, sinks=True)
    q, k, v, s = synth.layer_inputs(w2, 1, device=DEV)
    sentinel = torch.full((1, 16, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mimo.MimoAttnError) as ei:
        mimo.prefill(bad, q, k, v, sp, sinks=s, out=sentinel)
    assert ei.value.code == mimo.MIMO_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (sentinel == 3.0).all()  # nothing written on error


# ----------------------------------------------------------------------------- decode


def _decode_case(w, positions, seed, cap=None, q_scale=1.0, max_position=None, with_model=False):
    """Random cache state + one decode step on the GPU, and the oracle on the same state (rows of
    sequences past max_position, which the GPU leaves at zero, are not meaningful in ref).
    with_model: return (out, ref, rounding model's output) instead."""
    B = len(positions)
    swa = w.layer_kind == 1
    maxp = max(positions) if max_position is None else max_position
    cap = w.window if swa else (cap if cap else maxp + 1)
    q, kn, vn, s, kc, vc = synth.decode_inputs(w, seed, B, cap, device=DEV)
    if q_scale != 1.0:
        q = q * q_scale  # a power of two: exact in bf16
    kc0, vc0 = _f32(kc), _f32(vc)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    out = mimo.decode(_params(w, B), q, kn, vn, pos_t, maxp, kc, vc, sinks=s)
    torch.cuda.synchronize()
    opos = [p if p <= maxp else 0 for p in positions]
    if swa:
        # occupied ring slots only (a slot still empty holds no token), packed first
        kc_o = np.zeros_like(kc0)
        vc_o = np.zeros_like(vc0)
        kpos = np.zeros((B, w.window), np.int32)
        cnt = np.zeros(B, np.int32)
        for b, p in enumerate(opos):
            held = ring_positions(p, w.window)
            slots = np.nonzero(held >= 0)[0]
            n = len(slots)
            kc_o[b, :, :n] = kc0[b, :, slots].transpose(1, 0, 2)
            vc_o[b, :, :n] = vc0[b, :, slots].transpose(1, 0, 2)
            kpos[b, :n] = held[slots]
            cnt[b] = n
        kc_m, vc_m = kc_o, vc_o
    else:
        kpos = np.tile(np.arange(cap, dtype=np.int32), (B, 1))
        cnt = np.array(opos, np.int32)
        kc_m, vc_m = kc0, vc0
    ref, krot = oracle.decode(_oparams(w, B), _f32(q), _f32(kn), _f32(vn), np.array(opos),
                              kc_m, vc_m, kpos, cnt, _f32(s), want_k_rot=True)
    if with_model:
        model = rounding_model.decode(_oparams(w, B), _f32(q), _f32(kn), _f32(vn),
                                      np.array(opos), kc_m, vc_m, kpos, cnt, _f32(s))
        return out, ref, model
    return out, ref, krot, kc, vc, kc0, vc0, vn


@pytest.mark.parametrize("case", [
    dict(kind=0, Hq=16, Hkv=1, sinks=False, positions=[0, 1, 255, 256, 257, 1000, 4097]),
    dict(kind=0, Hq=8, Hkv=2, sinks=True, positions=[31, 32, 33]),
    dict(kind=1, Hq=8, Hkv=1, sinks=True, positions=[0, 5, 126, 127, 128, 129, 300, 5000]),
    dict(kind=1, Hq=16, Hkv=2, sinks=False, positions=[1, 200]),
    # rings wider than one 32-slot tile per wave (the slot loop with refills): 200 and 1024 slots
    dict(kind=1, Hq=8, Hkv=2, sinks=True, W=200, positions=[0, 150, 199, 200, 201, 1000]),
    dict(kind=1, Hq=16, Hkv=1, sinks=False, W=1024, positions=[5, 1023, 1024, 3000]),
])
def test_decode_bf16_small(case):
    case = dict(case)
    positions = case.pop("positions")
    w = _wl(B=len(positions), S=1, **case)
    _note(str(case) + str(positions))
    out, ref, krot, kc, vc, kc0, vc0, vn = _decode_case(w, positions, seed=5000 + len(positions))
    assert_close(out, ref, what=str(case))
    # the new token was appended (rotated key, raw value) and nothing else changed
    kc_h, vc_h = _f32(kc), _f32(vc)
    vn_h = _f32(vn)
    for b, p in enumerate(positions):
        slot = p % w.window if w.layer_kind == 1 else p
        np.testing.assert_allclose(kc_h[b, :, slot], krot[b], rtol=2 ** -8, atol=1e-6)
        assert np.array_equal(vc_h[b, :, slot], vn_h[b])
        kc_h[b, :, slot] = kc0[b, :, slot]
        vc_h[b, :, slot] = vc0[b, :, slot]
    assert np.array_equal(kc_h, kc0) and np.array_equal(vc_h, vc0)


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_skips_positions_past_max_position(kind):
    """A sequence whose position exceeds max_position gets a zero output and appends nothing;
    the others are unaffected (global: split-K over 1001 slots; sliding: one ring pass)."""
    positions = [100, 700, 5000]
    w = _wl(kind=kind, B=len(positions), S=1, Hq=8, Hkv=2, sinks=kind == 1)
    _note(f"decode past max_position kind={kind}")
    out, ref, _, kc, vc, kc0, vc0, _ = _decode_case(w, positions, seed=9600 + kind,
                                                    max_position=1000)
    assert torch.count_nonzero(out[2]) == 0, "a sequence past max_position must get zeros"
    assert np.array_equal(_f32(kc)[2], kc0[2]) and np.array_equal(_f32(vc)[2], vc0[2]), \
        "a sequence past max_position must not append"
    assert_close(out[:2], ref[:2], what=f"accepted sequences kind={kind}")


def test_decode_fp32_tiny():
    w = synth.Workload("tiny_dec", batch=3, seq=1, num_q_heads=4, num_kv_heads=1, qk_head_dim=32,
                       v_head_dim=16, rope_dims=10, rope_theta=1e4, layer_kind=1, window=16,
                       sinks=True, hidden=64, dtype=torch.float32)
    out, ref, *_ = _decode_case(w, [3, 15, 40], seed=6000)
    assert_close(out, ref, fp32=True, what="fp32 decode")


def test_decode_full_size_global_sampled_sequences():
    """64 sequences with cached lengths uniform in [1024, 32768], linear caches; the oracle checks
    a sample of sequences (shortest, longest and random ones)."""
    w = _wl(kind=0, B=synth.DECODE_BATCH, S=1, Hq=64, Hkv=4, sinks=False)
    lengths = synth.decode_lengths(3)
    positions = lengths.tolist()
    B, cap = len(positions), max(positions) + 1
    _note(f"decode GA full B={B} cap={cap}")
    q, kn, vn, s, kc, vc = synth.decode_inputs(w, 7000, B, cap, device=DEV)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    out = mimo.decode(_params(w, B), q, kn, vn, pos_t, max(positions), kc, vc, sinks=s)
    torch.cuda.synchronize()
    order = np.argsort(positions)
    sample = sorted({int(order[0]), int(order[-1]), 5, 17, 42})
    for b in sample:
        L = positions[b]
        kcb = kc[b:b + 1, :, :L].to("cpu", torch.float32).numpy()
        vcb = vc[b:b + 1, :, :L].to("cpu", torch.float32).numpy()
        ref = oracle.decode(_oparams(w, 1), _f32(q[b:b + 1]), _f32(kn[b:b + 1]), _f32(vn[b:b + 1]),
                            np.array([L]), kcb, vcb, np.arange(L, dtype=np.int32)[None],
                            np.array([L]), None)
        assert_close(out[b:b + 1], ref, what=f"seq {b} len {L}")


def test_decode_many_splits_mixed_lengths_all_sequences():
    """A decode grid over lengths from 255 to 8500 (16 sequences x 2 KV heads x 9 splits of 1024
    slots, one round of workgroups): short sequences' splits past their positions are empty, and
    the split boundaries fall inside tiles.  The oracle checks every sequence."""
    w = _wl(kind=0, B=16, S=1, Hq=16, Hkv=2, sinks=False)
    rng = np.random.default_rng(11)
    positions = [300, 8500, 255, 256, 257, 1023] + rng.integers(300, 8501, size=10).tolist()
    _note(f"decode GA many splits B=16 max {max(positions)}")
    out, ref, *_ = _decode_case(w, positions, seed=7100)
    assert_close(out, ref, what="decode, many splits")


def test_decode_full_round_grid_without_splits():
    """512 (sequence, KV head) pairs over short caches: one split each, so the grid is exactly one
    round of resident workgroups (two per CU), with a sink on a global layer and no combine.  The
    oracle checks every sequence."""
    w = _wl(kind=0, B=64, S=1, Hq=16, Hkv=8, sinks=True)
    rng = np.random.default_rng(23)
    positions = [0, 1, 31, 32, 100, 127] + rng.integers(0, 128, size=58).tolist()
    assert mimo.decode_workspace_size(_params(w, 64), max(positions)) == 0   # one split
    _note("decode GA one-round grid, B=64 Hkv=8, no splits")
    out, ref, *_ = _decode_case(w, positions, seed=7120)
    assert_close(out, ref, what="decode, full-round grid without splits")


# A decode whose grid takes more than one round of resident workgroups goes out in blocks of 4
# splits per (sequence, KV head) pair.  64 sequences x 4 KV heads over lengths up to 20000 make
# 10 splits of 2048 slots (bf16 and fp8 caches alike; tests/test_abi_cpu.py pins this geometry
# through the workspace size), so the blocks round 10 up to 12 and the last block's two padded
# splits start past every sequence's key range.
BLOCKED_MAX_POSITION = 20000


def blocked_positions(seed):
    rng = np.random.default_rng(seed)
    return [BLOCKED_MAX_POSITION, 300, 2047, 2048, 2049, 6143, 16385] + \
        rng.integers(300, BLOCKED_MAX_POSITION + 1, size=57).tolist()


def test_decode_blocked_grid_padded_block_all_sequences():
    w = _wl(kind=0, B=64, S=1, Hq=16, Hkv=4, sinks=False)
    positions = blocked_positions(17)
    assert mimo.decode_workspace_size(_params(w, 64), max(positions)) == 64 * 16 * 10 * 130 * 4
    _note(f"decode GA blocked grid B=64 max {max(positions)}")
    out, ref, *_ = _decode_case(w, positions, seed=7150)
    assert_close(out, ref, what="decode, blocked grid with a padded block")


def test_decode_full_size_swa_all_sequences():
    w = _wl(kind=1, B=synth.DECODE_BATCH, S=1, Hq=64, Hkv=8, sinks=True)
    positions = synth.decode_lengths(4).tolist()
    _note("decode SWA full")
    out, ref, *_ = _decode_case(w, positions, seed=8000)
    assert_close(out, ref, what="swa decode full")


@pytest.mark.parametrize("kind", [0, 1])
def test_prefill_then_decode_matches_longer_prefill(kind):
    """prefill(S) writing the cache, then one decode step == row S of prefill(S + 1)."""
    S = 300
    w = _wl(kind=kind, B=2, S=S + 1, Hq=16, Hkv=2, sinks=kind == 1)
    q, k, v, s = synth.layer_inputs(w, 9000 + kind, device=DEV)
    starts = [0, 11]
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    cap = w.window if kind == 1 else S + 20
    kc = torch.zeros((2, w.num_kv_heads, cap, 192), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((2, w.num_kv_heads, cap, 128), dtype=torch.bfloat16, device=DEV)
    wS = _wl(kind=kind, B=2, S=S, Hq=16, Hkv=2, sinks=kind == 1)
    pre = None
    if kind == 0:
        # a global layer's decode attends to every earlier position, and the linear cache of
        # sequence 1 must hold its positions 0..10 for the identity: a prefill of 11 tokens of its
        # own writes them first (the ring of a sliding layer only holds the last window)
        wp = _wl(kind=0, B=1, S=starts[1], Hq=16, Hkv=2, sinks=False)
        pre = synth.layer_inputs(wp, 9100, device=DEV)
        mimo.prefill(_params(wp), *pre[:3], torch.zeros(1, dtype=torch.int32, device=DEV),
                     k_cache=kc[1:2], v_cache=vc[1:2])
    mimo.prefill(_params(wS), q[:, :S].contiguous(), k[:, :S].contiguous(), v[:, :S].contiguous(),
                 sp, sinks=s, k_cache=kc, v_cache=vc)
    pos = torch.tensor([S + st for st in starts], dtype=torch.int32, device=DEV)
    dec = mimo.decode(_params(wS), q[:, S].contiguous(), k[:, S].contiguous(), v[:, S].contiguous(),
                      pos, max(starts) + S, kc, vc, sinks=s)
    full = mimo.prefill(_params(w), q, k, v, sp, sinks=s)
    torch.cuda.synchronize()
    posn = np.stack([np.arange(S + 1, dtype=np.int32) + st for st in starts])
    ref = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), posn, _f32(s),
                         rows=np.array([S], np.int32))
    assert_close(full[:, S], ref[:, S], what="longer prefill")
    ref_dec = ref[:, S]
    if kind == 0:
        # sequence 1's decode == the last row of one prefill over all its positions 0..S + 11
        n = starts[1] + S + 1
        w1 = _wl(kind=0, B=1, S=n, Hq=16, Hkv=2, sinks=False)
        cat = [np.concatenate([_f32(a), _f32(b[1:2])], axis=1) for a, b in zip(pre[:3], (q, k, v))]
        ref1 = oracle.prefill(_oparams(w1), *cat, np.arange(n, dtype=np.int32)[None],
                              rows=np.array([n - 1], np.int32))
        ref_dec = np.concatenate([ref_dec[:1], ref1[:, n - 1]], axis=0)
    assert_close(dec, ref_dec, what="decode after prefill")


def _stack_config():
    """The 48-layer stack's configuration as a model config carries it (hybrid_layer_pattern and
    the per-kind fields), from which the dispatcher derives every layer's parameters."""
    return mimo.HybridAttentionConfig(
        hidden_size=4096, num_attention_heads=64, num_key_value_heads=4, swa_num_key_value_heads=8,
        head_dim=192, v_head_dim=128, partial_rotary_factor=1.0 / 3.0, rope_theta=5e6,
        swa_rope_theta=1e4, sliding_window_size=128, hybrid_layer_pattern=synth.stack_pattern(),
        rope_dims=64)


def _golden_layer(index):
    """What the pages fix for stack layer `index` (tests/golden/dispatch.json, each fact cited
    there): its kind, theta, KV heads, window, sinks and cache kind."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dispatch.json")))
    kind = "global" if index in fx["stack"]["global_layers"] else "sliding"
    return kind, fx["theta_selection"][kind]


@pytest.mark.parametrize("layer", [0, 1, 5, 6])
def test_stack_layer_full_size_prefill_then_decode_sampled(layer):
    """A layer of the 48-layer stack at full size (batch 2, 16384 tokens), configured by the
    per-layer dispatch (layer_specs of the stack's hybrid_layer_pattern config): prefill writes the
    cache, then two decode steps.  The oracle gets the layer the pages define for that index
    (kind, theta, KV heads, window, sinks from the golden dispatch facts), so a wrong kind, theta,
    KV-head count, window or sink choice of the dispatcher fails here.  Sampled prefill rows and
    every decode output are checked (the oracle's decode cache is its own rotated keys)."""
    cfg = _stack_config()
    spec = mimo.layer_specs(cfg)[layer]
    B, S, T = synth.STACK_BATCH, synth.STACK_SEQ, 2
    p = spec.params(cfg, B)
    kind_name, fact = _golden_layer(layer)
    okind = 1 if kind_name == "sliding" else 0
    op = OracleParams(batch=B, num_q_heads=64, num_kv_heads=fact["kv_heads"], qk_head_dim=192,
                      v_head_dim=128, rope_dims=64, layer_kind=okind, window=fact["window"],
                      rope_theta=fact["theta"], v_scale=float(np.sqrt(4096 / (64 * 128))))
    _note(f"stack layer {layer}: dispatch kind {spec.kind} theta {spec.rope_theta} "
          f"kv {spec.num_kv_heads} window {spec.window} sinks {spec.has_sinks}")
    # inputs drawn with the pages' shapes for the index (KV heads from the golden facts)
    w = synth.Workload("stack", B, S + T, num_q_heads=64, num_kv_heads=fact["kv_heads"],
                       qk_head_dim=192, v_head_dim=128, rope_dims=64, rope_theta=fact["theta"],
                       layer_kind=okind, window=fact["window"], sinks=True, hidden=4096,
                       dtype=torch.bfloat16)
    q, k, v, s_all = synth.layer_inputs(w, 4000 + layer, device=DEV)
    s_gpu = s_all if spec.has_sinks else None
    s_ref = s_all if fact["sinks"] else None
    sp = torch.zeros(B, dtype=torch.int32, device=DEV)
    cap = spec.window if spec.cache == "ring" else S + T
    kc = torch.zeros((B, spec.num_kv_heads, cap, 192), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((B, spec.num_kv_heads, cap, 128), dtype=torch.bfloat16, device=DEV)
    out = mimo.prefill(p, q[:, :S].contiguous(), k[:, :S].contiguous(), v[:, :S].contiguous(), sp,
                       sinks=s_gpu, k_cache=kc, v_cache=vc)
    decs = []
    for t in range(T):
        pos = torch.full((B,), S + t, dtype=torch.int32, device=DEV)
        decs.append(mimo.decode(p, q[:, S + t].contiguous(), k[:, S + t].contiguous(),
                                v[:, S + t].contiguous(), pos, S + T - 1, kc, vc, sinks=s_gpu))
    torch.cuda.synchronize()
    rng = np.random.default_rng(layer)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(S - 8, S),
                                     rng.integers(0, S, 16)])).astype(np.int32)
    rows_all = np.concatenate([rows, np.arange(S, S + T, dtype=np.int32)])
    posn = np.stack([np.arange(S + T, dtype=np.int32)] * B)
    ref = oracle.prefill(op, _f32(q), _f32(k), _f32(v), posn, _f32(s_ref), rows=rows_all)
    bound = rounding_model.prefill_bound(op, _f32(q), _f32(k), _f32(v), posn, _f32(s_ref),
                                         rows=rows)
    assert_close(out[:, rows], ref[:, rows], what=f"stack layer {layer} prefill rows",
                 bound=bound[:, rows])
    model = rounding_model.prefill(op, _f32(q), _f32(k), _f32(v), posn, _f32(s_ref), rows=rows_all)
    assert_near_model(to_np64(out)[:, rows], ref[:, rows], model[:, rows],
                      what=f"stack layer {layer} prefill rows")
    for t in range(T):
        assert_close(decs[t], ref[:, S + t], what=f"stack layer {layer} decode step {t}")
