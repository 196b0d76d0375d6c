"""GPU parity of the fp8 (e4m3) KV cache: decode and extend over coded caches, prefill writing them.

Against the fp64 oracle: decode outputs over the same coded cache (the oracle decodes the codes
itself); the appended token's codes (values: the same fp32 product on both sides, so bit for bit;
keys: the kernel rotates in fp32 with its own sin/cos, so a key element may take the neighbouring
code where the exact product lies within rounding of a midpoint — every key code must be one of
the two codes around the oracle's product, and almost all equal to the oracle's); prefill's coded
caches likewise.  Seeds: 11000 + case.
"""
import numpy as np
import pytest
import torch

import global_attention_rope_amd as mimo
import oracle
from tests import synth
from tests import rounding_model
from tests.gpu_helpers import assert_close, prefill_bound_for, ring_positions
from tests.test_gpu_parity import _f32, _note, _oparams, _params, _wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KS, VS = synth.FP8_K_SCALE, synth.FP8_V_SCALE


def _p8(w, B=None):
    p = _params(w, B)
    p.cache_dtype, p.k_cache_scale, p.v_cache_scale = mimo.CACHE_FP8_E4M3, KS, VS
    return p


def _np8(t):
    return t.to("cpu").numpy()


def _oracle_cache8(w, kc8, vc8, positions):
    """The coded cache as the oracle takes it: per sequence the slots that hold a position
    before the new token, first, with their positions."""
    B, cap = kc8.shape[0], kc8.shape[2]
    okc = np.zeros_like(kc8)
    ovc = np.zeros_like(vc8)
    kpos = np.zeros((B, cap), np.int32)
    cnt = np.zeros(B, np.int32)
    for b, p in enumerate(positions):
        held = ring_positions(p, w.window) if w.layer_kind == 1 else np.where(
            np.arange(cap) < p, np.arange(cap), -1)
        slots = np.nonzero(held >= 0)[0]
        n = len(slots)
        okc[b, :, :n] = kc8[b][:, slots]
        ovc[b, :, :n] = vc8[b][:, slots]
        kpos[b, :n] = held[slots]
        cnt[b] = n
    return okc, ovc, kpos, cnt


def _check_key_codes(gpu_codes, exact_rot, what):
    """Every key code is one of the two codes around fp32(exact) * (1 / scale); nearly all equal
    the nearest one."""
    inv = np.float32(1) / np.float32(KS)
    y = exact_rot.astype(np.float32) * inv
    ref = oracle.e4m3_encode(exact_rot.astype(np.float32), inv)
    gv = oracle.e4m3_decode(gpu_codes)
    rv = oracle.e4m3_decode(ref)
    a = np.abs(y.astype(np.float64))
    quantum = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(gv - y) <= quantum * (1 + 1e-9)), f"{what}: a key code is not a neighbour"
    frac = float(np.mean(gpu_codes == ref))
    assert frac >= 0.995, f"{what}: only {frac:.4f} of the key codes are the nearest"
    return frac


def _decode8_case(w, positions, seed, q_scale=1.0):
    B = len(positions)
    swa = w.layer_kind == 1
    cap = w.window if swa else max(positions) + 1
    q, kn, vn, s, _, _ = synth.decode_inputs(w, seed, B, 1, device=DEV)
    if q_scale != 1.0:
        q = q * q_scale  # a power of two: exact in bf16
    kc8, vc8 = synth.fp8_cache_contents(w, seed + 1, B, cap, device=DEV)
    kc0, vc0 = _np8(kc8), _np8(vc8)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    out = mimo.decode(_p8(w, B), q, kn, vn, pos_t, max(positions), kc8, vc8, sinks=s)
    torch.cuda.synchronize()
    okc, ovc, kpos, cnt = _oracle_cache8(w, kc0, vc0, positions)
    ref, krot, kcode, vcode = oracle.decode_fp8(_oparams(w, B), _f32(q), _f32(kn), _f32(vn),
                                                np.array(positions, np.int32), okc, ovc, kpos, cnt,
                                                KS, VS, _f32(s))
    return out, ref, krot, kcode, vcode, kc8, vc8, kc0, vc0


@pytest.mark.parametrize("case", [
    dict(kind=0, Hq=16, Hkv=1, sinks=False, positions=[0, 1, 255, 256, 257, 1000, 4097]),
    dict(kind=0, Hq=8, Hkv=2, sinks=True, positions=[31, 32, 33]),
    dict(kind=1, Hq=8, Hkv=1, sinks=True, positions=[0, 5, 126, 127, 128, 129, 300, 5000]),
    dict(kind=1, Hq=16, Hkv=2, sinks=False, positions=[1, 200]),
    # rings wider than one 32-slot tile per wave (the slot loop with refills): 200 and 1024 slots
    dict(kind=1, Hq=8, Hkv=2, sinks=True, W=200, positions=[0, 150, 199, 200, 201, 1000]),
    dict(kind=1, Hq=16, Hkv=1, sinks=False, W=1024, positions=[5, 1023, 1024, 3000]),
])
def test_decode_fp8_small(case):
    case = dict(case)
    positions = case.pop("positions")
    w = _wl(B=len(positions), S=1, **case)
    _note(f"fp8 decode {case} {positions}")
    out, ref, krot, kcode, vcode, kc8, vc8, kc0, vc0 = _decode8_case(w, positions,
                                                                     11000 + len(positions))
    assert_close(out, ref, what=f"fp8 decode {case}")
    kc1, vc1 = _np8(kc8), _np8(vc8)
    for b, p in enumerate(positions):
        slot = p % w.window if w.layer_kind == 1 else p
        assert np.array_equal(vc1[b, :, slot], vcode[b]), f"seq {b}: value codes"
        _check_key_codes(kc1[b, :, slot], krot[b], f"seq {b}")
        kc1[b, :, slot] = kc0[b, :, slot]
        vc1[b, :, slot] = vc0[b, :, slot]
    assert np.array_equal(kc1, kc0) and np.array_equal(vc1, vc0), "a foreign slot changed"


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_fp8_full_size(kind):
    """Batch 64, cached lengths uniform in [1024, 32768]: every sequence (sliding) or a sample of
    them (global) against the oracle."""
    Hkv = 4 if kind == 0 else 8
    w = _wl(kind=kind, B=synth.DECODE_BATCH, S=1, Hq=64, Hkv=Hkv, sinks=kind == 1)
    positions = synth.decode_lengths(3 + kind).tolist()
    B = len(positions)
    cap = w.window if kind == 1 else max(positions) + 1
    _note(f"fp8 decode full kind={kind} B={B} cap={cap}")
    q, kn, vn, s, _, _ = synth.decode_inputs(w, 11100 + kind, B, 1, device=DEV)
    kc8, vc8 = synth.fp8_cache_contents(w, 11200 + kind, B, cap, device=DEV)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    # (the oracle reads the cache as it was before the step appended to it)
    kc0, vc0 = (_np8(kc8), _np8(vc8)) if kind == 1 else (None, None)
    sample = sorted({int(np.argmin(positions)), int(np.argmax(positions)), 5, 17, 42})
    pre = {b: (_np8(kc8[b:b + 1, :, :positions[b]]), _np8(vc8[b:b + 1, :, :positions[b]]))
           for b in sample} if kind == 0 else None
    out = mimo.decode(_p8(w, B), q, kn, vn, pos_t, max(positions), kc8, vc8, sinks=s)
    torch.cuda.synchronize()
    if kind == 1:
        okc, ovc, kpos, cnt = _oracle_cache8(w, kc0, vc0, positions)
        ref, *_ = oracle.decode_fp8(_oparams(w, B), _f32(q), _f32(kn), _f32(vn),
                                    np.array(positions, np.int32), okc, ovc, kpos, cnt, KS, VS,
                                    _f32(s))
        assert_close(out, ref, what="fp8 sliding decode full")
        return
    for b in sample:
        L = positions[b]
        kcb, vcb = pre[b]
        ref, *_ = oracle.decode_fp8(_oparams(w, 1), _f32(q[b:b + 1]), _f32(kn[b:b + 1]),
                                    _f32(vn[b:b + 1]), np.array([L], np.int32), kcb, vcb,
                                    np.arange(L, dtype=np.int32)[None], np.array([L], np.int32),
                                    KS, VS, None)
        assert_close(out[b:b + 1], ref, what=f"fp8 global seq {b} len {L}")


def test_decode_fp8_blocked_grid_padded_block_all_sequences():
    """fp8 caches through the blocked dispatch with a padded last block: 64 sequences x 4 KV heads
    x 10 splits of 2048 slots (blocks of 4 round 10 up to 12): every sequence against the oracle."""
    from tests.test_gpu_parity import blocked_positions
    w = _wl(kind=0, B=64, S=1, Hq=16, Hkv=4, sinks=False)
    positions = blocked_positions(19)
    B, cap = len(positions), max(positions) + 1
    assert mimo.decode_workspace_size(_p8(w, B), max(positions)) == B * 16 * 10 * 130 * 4
    _note(f"fp8 decode blocked grid B={B} cap={cap}")
    q, kn, vn, _, _, _ = synth.decode_inputs(w, 11160, B, 1, device=DEV)
    kc8, vc8 = synth.fp8_cache_contents(w, 11260, B, cap, device=DEV)
    pre = {b: (_np8(kc8[b:b + 1, :, :positions[b]]), _np8(vc8[b:b + 1, :, :positions[b]]))
           for b in range(B)}
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    out = mimo.decode(_p8(w, B), q, kn, vn, pos_t, max(positions), kc8, vc8)
    torch.cuda.synchronize()
    for b in range(B):
        L = positions[b]
        kcb, vcb = pre[b]
        ref, *_ = oracle.decode_fp8(_oparams(w, 1), _f32(q[b:b + 1]), _f32(kn[b:b + 1]),
                                    _f32(vn[b:b + 1]), np.array([L], np.int32), kcb, vcb,
                                    np.arange(L, dtype=np.int32)[None], np.array([L], np.int32),
                                    KS, VS, None)
        assert_close(out[b:b + 1], ref, what=f"fp8 global seq {b} len {L}")


def test_decode_fp8_many_splits_mixed_lengths_all_sequences():
    """A global-layer decode over fp8 caches, lengths from 300 to 17000 (16 sequences x 2 KV heads
    x 9 splits of 2048 slots, one round of workgroups): every sequence against the oracle."""
    w = _wl(kind=0, B=16, S=1, Hq=16, Hkv=2, sinks=False)
    rng = np.random.default_rng(13)
    positions = [300, 17000, 511, 512, 513, 2047] + rng.integers(300, 17001, size=10).tolist()
    B = len(positions)
    cap = max(positions) + 1
    _note(f"fp8 decode many splits B={B} cap={cap}")
    q, kn, vn, _, _, _ = synth.decode_inputs(w, 11150, B, 1, device=DEV)
    kc8, vc8 = synth.fp8_cache_contents(w, 11250, B, cap, device=DEV)
    pre = {b: (_np8(kc8[b:b + 1, :, :positions[b]]), _np8(vc8[b:b + 1, :, :positions[b]]))
           for b in range(B)}
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    out = mimo.decode(_p8(w, B), q, kn, vn, pos_t, max(positions), kc8, vc8)
    torch.cuda.synchronize()
    for b in range(B):
        L = positions[b]
        kcb, vcb = pre[b]
        ref, *_ = oracle.decode_fp8(_oparams(w, 1), _f32(q[b:b + 1]), _f32(kn[b:b + 1]),
                                    _f32(vn[b:b + 1]), np.array([L], np.int32), kcb, vcb,
                                    np.arange(L, dtype=np.int32)[None], np.array([L], np.int32),
                                    KS, VS, None)
        assert_close(out[b:b + 1], ref, what=f"fp8 global seq {b} len {L}")


@pytest.mark.parametrize("kind", [0, 1])
def test_prefill_writes_fp8_caches_and_decode_continues(kind):
    """Prefill storing coded caches (value codes bit for bit, key codes neighbour-valid), its
    output unchanged, then decode steps over the coded cache against the oracle's own chain."""
    run_prefill_fp8_chain(kind, seed=11300 + kind)


def run_prefill_fp8_chain(kind, seed, r=64, theta=None, q_scale=1.0):
    """One prefill writing fp8 caches and one decode step over them, both against the oracle."""
    S = 300
    w = _wl(kind=kind, B=2, S=S, Hq=16, Hkv=2, sinks=kind == 1, r=r, theta=theta)
    _note(f"fp8 prefill cache kind={kind} r={r}")
    q, k, v, s = synth.layer_inputs(w, seed, device=DEV)
    if q_scale != 1.0:
        q = q * q_scale  # a power of two: exact in bf16
    starts = [0, 11]
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    cap = w.window if kind == 1 else S + max(starts) + 8
    kc8 = torch.zeros((2, w.num_kv_heads, cap, 192), dtype=torch.uint8, device=DEV)
    vc8 = torch.zeros((2, w.num_kv_heads, cap, 128), dtype=torch.uint8, device=DEV)
    out = mimo.prefill(_p8(w), q, k, v, sp, sinks=s, k_cache=kc8, v_cache=vc8)
    torch.cuda.synchronize()
    pos = np.stack([np.arange(S, dtype=np.int32) + st for st in starts])
    ref, krot = oracle.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s), want_k_rot=True)
    assert_close(out, ref, what="prefill output with an fp8 cache",
                 bound=prefill_bound_for(w, q, k, v, s, pos))
    kc1, vc1 = _np8(kc8), _np8(vc8)
    vin = _f32(v)
    stored = {}
    for b, st in enumerate(starts):
        toks = range(max(0, S - w.window), S) if kind == 1 else range(S)
        slots = np.array([(st + i) % w.window if kind == 1 else st + i for i in toks])
        tk = np.array(list(toks))
        assert np.array_equal(vc1[b][:, slots], oracle.e4m3_encode(vin[b, tk], np.float32(1) / np.float32(VS)).transpose(1, 0, 2))
        _check_key_codes(kc1[b][:, slots], krot[b, tk].transpose(1, 0, 2), f"prefill seq {b}")
        stored[b] = (slots, st + tk)
    # decode one more token over the coded cache; the oracle's chain uses its own codes
    qd, kd, vd, _, _, _ = synth.decode_inputs(w, seed + 100, 2, 1, device=DEV)
    if q_scale != 1.0:
        qd = qd * q_scale
    dpos = [S + st for st in starts]
    dec = mimo.decode(_p8(w), qd, kd, vd, torch.tensor(dpos, dtype=torch.int32, device=DEV),
                      max(dpos), kc8, vc8, sinks=s)
    torch.cuda.synchronize()
    inv_k = np.float32(1) / np.float32(KS)
    # a linear cache also holds the positions before the prompt's start, which this test never
    # wrote: their slots keep the zero codes they were allocated with (keys and values 0.0), and
    # the decode attends to them like any earlier position
    lead = {b: (starts[b] if kind == 0 else 0) for b in stored}
    L = max(len(stored[b][0]) + lead[b] for b in stored)
    okc = np.zeros((2, w.num_kv_heads, L, 192), np.uint8)
    ovc = np.zeros((2, w.num_kv_heads, L, 128), np.uint8)
    kpos = np.zeros((2, L), np.int32)
    cnt = np.zeros(2, np.int32)
    for b, (slots, poss) in stored.items():
        n, z = len(slots), lead[b]
        tk = poss - starts[b]
        kpos[b, :z] = np.arange(z)
        okc[b, :, z:z + n] = oracle.e4m3_encode(krot[b, tk].astype(np.float32), inv_k).transpose(1, 0, 2)
        ovc[b, :, z:z + n] = oracle.e4m3_encode(vin[b, tk], np.float32(1) / np.float32(VS)).transpose(1, 0, 2)
        kpos[b, z:z + n] = poss
        cnt[b] = z + n
    dref, *_ = oracle.decode_fp8(_oparams(w), _f32(qd), _f32(kd), _f32(vd), np.array(dpos, np.int32),
                                 okc, ovc, kpos, cnt, KS, VS, _f32(s))
    assert_close(dec, dref, what="decode after an fp8 prefill")


# ----------------------------------------------------------------------------- extend
# Extend over fp8 caches: the cached positions are attended through their codes, the new tokens at
# full precision (as prefill does), and the new tokens are stored as codes.  The oracle takes the
# cache as the values its codes stand for (exact: e4m3 values times power-of-two scales).

EXT_CASES = [
    dict(kind=0, B=2, S=40, Hq=8, Hkv=2, sinks=False, starts=[0, 700]),        # prefill kernel
    dict(kind=0, B=3, S=4, Hq=16, Hkv=1, sinks=True, starts=[1, 255, 4097]),   # tile kernel
    # the tile kernel's other workgroup sizes (16 heads x 16 / 8 token columns: 8 / 4 waves, whose
    # threads split a tile's 1280 code units unevenly / evenly; 4 columns: one wave)
    dict(kind=0, B=2, S=12, Hq=32, Hkv=2, sinks=False, starts=[3, 2500]),
    dict(kind=0, B=2, S=7, Hq=32, Hkv=2, sinks=True, starts=[0, 1300]),
    dict(kind=0, B=2, S=1, Hq=8, Hkv=2, sinks=False, starts=[64, 333]),
    dict(kind=0, B=2, S=2, Hq=8, Hkv=2, sinks=True, starts=[100, 3000]),       # 8 columns, 12 splits
    dict(kind=1, B=2, S=300, Hq=8, Hkv=2, sinks=True, starts=[5, 4000]),       # ring, S > W
    dict(kind=1, B=3, S=4, Hq=16, Hkv=2, sinks=True, starts=[0, 2, 1000]),     # ring, tile kernel
]


@pytest.mark.parametrize("ci", range(len(EXT_CASES)))
def test_extend_fp8_caches(ci):
    from tests.test_gpu_extend import _oracle_cache, _stored_slots
    case = dict(EXT_CASES[ci])
    starts = case.pop("starts")
    w = _wl(**case)
    S, B = w.seq, w.batch
    _note(f"fp8 extend {case} starts {starts}")
    q, k, v, s = synth.layer_inputs(w, 11500 + ci, device=DEV)
    cap = w.window if w.layer_kind == 1 else max(starts) + S + 5
    kc8, vc8 = synth.fp8_cache_contents(w, 11600 + ci, B, cap, device=DEV)
    kc0, vc0 = _np8(kc8), _np8(vc8)
    kf = torch.from_numpy(oracle.e4m3_decode(kc0) * KS)
    vf = torch.from_numpy(oracle.e4m3_decode(vc0) * VS)
    okc, ovc, kpos, count = _oracle_cache(w, kf, vf, starts)
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = mimo.extend(_p8(w), q, k, v, sp, max(starts), kc8, vc8, sinks=s)
    torch.cuda.synchronize()
    ref, krot = oracle.extend(_oparams(w), _f32(q), _f32(k), _f32(v), np.array(starts, np.int32),
                              okc, ovc, kpos, count, _f32(s), want_k_rot=True)
    bound = rounding_model.extend_bound(_oparams(w), _f32(q), _f32(k), _f32(v), starts, okc, ovc,
                                        kpos, count, _f32(s))
    assert_close(out, ref, what=f"fp8 extend {case}", bound=bound)
    # caches: the new tokens' codes in their slots, every other slot as it was
    kc1, vc1 = _np8(kc8), _np8(vc8)
    vin = _f32(v)
    inv_v = np.float32(1) / np.float32(VS)
    for b, st in enumerate(starts):
        slots = _stored_slots(w, st, S)
        kept = np.setdiff1d(np.arange(cap), list(slots.values()))
        assert np.array_equal(kc1[b][:, kept], kc0[b][:, kept]), f"seq {b}: foreign K slot changed"
        assert np.array_equal(vc1[b][:, kept], vc0[b][:, kept]), f"seq {b}: foreign V slot changed"
        tok = np.array(sorted(slots))
        sl = np.array([slots[i] for i in tok])
        assert np.array_equal(vc1[b][:, sl], oracle.e4m3_encode(vin[b, tok], inv_v).transpose(1, 0, 2))
        _check_key_codes(kc1[b][:, sl], krot[b, tok].transpose(1, 0, 2), f"extend seq {b}")
