"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties the oracle to the mathematics the pages fix, through a route that does not retype
the oracle's formulas:
  * the rotation is compared with the matrix exponential of its generator (scipy ``expm``), with
    frequencies built as a geometric sequence by repeated multiplication;
  * whole-layer outputs are compared with torch's fp64 ``scaled_dot_product_attention`` given
    explicitly repeated KV heads, an additive mask and the sink as an extra zero-value key;
  * closed forms (zero query, first row, sink as a pure denominator term), limits (sink -> -inf,
    sink -> +inf), invariances (window >= seq is global attention; rope_dims = 0 ignores theta
    and positions; a common position shift changes nothing) and decode/prefill agreement.

Pages: "Add Xiaomi MiMo-V2" (transformers PR 45144), "Additional useful info" (dual theta,
per-kind KV groups, decoupled V dim, value rescale, SWA-only sink, partial RoPE); "feat(models):
add Xiaomi MiMo v2" (mlxcel issue 842), "Architecture, verified against upstream" (rope dims,
theta selection, window) and "Implementation plan" (rotating cache).
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import OracleParams
from tests import synth

TOL = 1e-11


def _params(w: synth.Workload, batch=None, **kw) -> OracleParams:
    d = dict(batch=w.batch if batch is None else batch, num_q_heads=w.num_q_heads,
             num_kv_heads=w.num_kv_heads, qk_head_dim=w.qk_head_dim, v_head_dim=w.v_head_dim,
             rope_dims=w.rope_dims, layer_kind=w.layer_kind, window=w.window,
             rope_theta=w.rope_theta, v_scale=w.v_scale)
    d.update(kw)
    return OracleParams(**d)


def _small(kind=1, Hq=4, Hkv=2, dqk=16, dv=8, r=6, theta=1.0e4, W=5, sinks=True, hidden=None):
    return synth.Workload("pin", batch=2, seq=12, num_q_heads=Hq, num_kv_heads=Hkv,
                          qk_head_dim=dqk, v_head_dim=dv, rope_dims=r, rope_theta=theta,
                          layer_kind=kind, window=W, sinks=sinks,
                          hidden=hidden if hidden else Hq * dv * 2, dtype=torch.float32)


def _np(t):
    return None if t is None else t.to(torch.float32).numpy()


def _frequencies(r, theta):
    # geometric sequence omega_0 = 1, ratio theta^(-2/r), built by repeated multiplication
    ratio = theta ** (-2.0 / r) if r else 1.0
    om, cur = [], 1.0
    for _ in range(r // 2):
        om.append(cur)
        cur *= ratio
    return np.array(om)


def _rotation_matrix(dim, r, theta, pos):
    """exp(pos * G), G the generator turning pair (d, d + r/2) at rate omega_d."""
    G = np.zeros((dim, dim))
    om = _frequencies(r, theta)
    h = r // 2
    for d in range(h):
        G[d + h, d] = om[d]
        G[d, d + h] = -om[d]
    return scipy.linalg.expm(pos * G)


def _positions(B, S, starts):
    return np.stack([np.arange(S, dtype=np.int32) + s for s in starts])


# ----------------------------------------------------------------------------- rotation


@pytest.mark.parametrize("dim,r,theta", [(32, 10, 1e4), (16, 6, 1e4), (24, 24, 5e6), (8, 0, 1e4)])
def test_rotation_is_matrix_exponential_of_generator(dim, r, theta):
    rng = np.random.default_rng(1)
    pos = np.array([0, 1, 7, 130, 4099], dtype=np.int32)
    x = rng.standard_normal((len(pos), dim))
    y = oracle.rotate(x.astype(np.float32), r, theta, pos)
    for i, p in enumerate(pos):
        R = _rotation_matrix(dim, r, theta, float(p))
        ref = R @ x[i].astype(np.float32).astype(np.float64)
        np.testing.assert_allclose(y[i], ref, rtol=0, atol=1e-9 * max(1.0, p / 100))


def test_rotation_preserves_pair_norms_and_passes_tail_unchanged():
    rng = np.random.default_rng(2)
    dim, r = 192, 64
    x = rng.standard_normal((50, dim)).astype(np.float32).astype(np.float64)
    pos = rng.integers(0, 40000, 50).astype(np.int32)
    y = oracle.rotate(x, r, 5e6, pos)
    h = r // 2
    n_in = x[:, :h] ** 2 + x[:, h:r] ** 2
    n_out = y[:, :h] ** 2 + y[:, h:r] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13, atol=1e-13)
    assert np.array_equal(y[:, r:], x[:, r:])  # dims >= r untouched, bit for bit


def test_frequencies_follow_geometric_sequence():
    for r, theta in [(10, 1e4), (64, 1e4), (64, 5e6)]:
        np.testing.assert_allclose(oracle.omega(r, theta), _frequencies(r, theta), rtol=1e-13)


# ----------------------------------------------------------------------------- scores


def test_scores_brute_force_against_explicit_rotation_matrices():
    w = _small(Hq=4, Hkv=2, dqk=16, r=6)
    q, k, v, s = synth.layer_inputs(w, seed=11)
    B, S = w.batch, w.seq
    pos = _positions(B, S, [0, 37])
    P = _params(w)
    tau = 1.0 / math.sqrt(w.qk_head_dim)
    qn, kn = _np(q).astype(np.float64), _np(k).astype(np.float64)
    for b in range(B):
        Rs = [_rotation_matrix(w.qk_head_dim, w.rope_dims, w.rope_theta, float(p)) for p in pos[b]]
        for h in range(w.num_q_heads):
            g = h // (w.num_q_heads // w.num_kv_heads)
            z = oracle.scores(P, _np(q), _np(k), pos, b, h)
            ref = np.array([[tau * (Rs[i] @ qn[b, i, h]) @ (Rs[j] @ kn[b, j, g]) for j in range(S)]
                            for i in range(S)])
            np.testing.assert_allclose(z, ref, rtol=0, atol=1e-11)


def test_scores_depend_only_on_relative_position():
    w = _small(r=16, dqk=16)
    q, k, _, _ = synth.layer_inputs(w, seed=12)
    P = _params(w)
    z0 = oracle.scores(P, _np(q), _np(k), _positions(2, w.seq, [0, 0]), 0, 1)
    z1 = oracle.scores(P, _np(q), _np(k), _positions(2, w.seq, [9000, 0]), 0, 1)
    np.testing.assert_allclose(z1, z0, rtol=0, atol=1e-9)


# ----------------------------------------------------------------------------- library routine


def _sdpa_reference(w, q, k, v, sinks, pos, v_scale):
    """torch fp64 SDPA on rotated q/k (rotation via expm), repeated KV heads, additive mask and
    the sink as one extra key whose score is the sink logit and whose value is zero."""
    B, S, Hq, dqk = q.shape
    Hkv = k.shape[2]
    qn = q.to(torch.float64).numpy()
    kn = k.to(torch.float64).numpy()
    qr = np.empty_like(qn)
    kr = np.empty_like(kn)
    for b in range(B):
        for i in range(S):
            R = _rotation_matrix(dqk, w.rope_dims, w.rope_theta, float(pos[b, i]))
            qr[b, i] = qn[b, i] @ R.T
            kr[b, i] = kn[b, i] @ R.T
    Q = torch.from_numpy(qr).permute(0, 2, 1, 3)  # B,Hq,S,d
    K = torch.from_numpy(kr).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    V = v.to(torch.float64).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.full((B, 1, S, S + 1), float("-inf"), dtype=torch.float64)
    for b in range(B):
        for i in range(S):
            for j in range(S):
                dlt = int(pos[b, i]) - int(pos[b, j])
                ok = dlt >= 0 and (w.layer_kind == 0 or dlt < w.window)
                if ok:
                    mask[b, 0, i, j] = 0.0
    mask = mask.expand(B, Hq, S, S + 1).clone()
    # extra key: zero vector with additive bias = sink * sqrt(dqk) / sqrt(dqk) -> sink logit
    Kx = torch.cat([K, torch.zeros(B, Hq, 1, dqk, dtype=torch.float64)], dim=2)
    Vx = torch.cat([V, torch.zeros(B, Hq, 1, V.shape[-1], dtype=torch.float64)], dim=2)
    if sinks is not None:
        mask[..., S] = sinks.to(torch.float64).view(1, Hq, 1)
    out = torch.nn.functional.scaled_dot_product_attention(Q, Kx, Vx, attn_mask=mask)
    return (v_scale * out).permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("cfg", [
    dict(kind=1, Hq=4, Hkv=1, dqk=32, dv=16, r=10, theta=1e4, W=4, sinks=True),
    dict(kind=1, Hq=4, Hkv=2, dqk=16, dv=8, r=6, theta=1e4, W=5, sinks=True, hidden=96),
    dict(kind=0, Hq=6, Hkv=2, dqk=16, dv=12, r=8, theta=5e6, W=0, sinks=False, hidden=50),
    dict(kind=0, Hq=2, Hkv=2, dqk=8, dv=8, r=0, theta=1e4, W=0, sinks=True),
    dict(kind=1, Hq=3, Hkv=3, dqk=8, dv=4, r=8, theta=10.0, W=1, sinks=True),
])
def test_prefill_matches_torch_sdpa(cfg):
    w = _small(**cfg)
    q, k, v, s = synth.layer_inputs(w, seed=21)
    pos = _positions(w.batch, w.seq, [0, 5])
    out = oracle.prefill(_params(w), _np(q), _np(k), _np(v), pos, _np(s))
    ref = _sdpa_reference(w, q, k, v, s, pos, w.v_scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- invariants


def test_window_at_least_seq_reduces_to_global_causal():
    w = _small(kind=1, W=12, sinks=False)
    q, k, v, _ = synth.layer_inputs(w, seed=31)
    pos = _positions(w.batch, w.seq, [0, 3])
    swa = oracle.prefill(_params(w), _np(q), _np(k), _np(v), pos, None)
    swa_big = oracle.prefill(_params(w, window=1000), _np(q), _np(k), _np(v), pos, None)
    ga = oracle.prefill(_params(w, layer_kind=0, window=0), _np(q), _np(k), _np(v), pos, None)
    np.testing.assert_allclose(swa, ga, rtol=0, atol=TOL)
    np.testing.assert_allclose(swa_big, ga, rtol=0, atol=TOL)
    short = oracle.prefill(_params(w, window=11), _np(q), _np(k), _np(v), pos, None)
    assert np.abs(short - ga).max() > 1e-6  # the last row loses key 0 when W = S - 1


def test_sink_scales_rows_by_denominator_ratio_and_limits():
    w = _small(kind=1, W=4)
    q, k, v, s = synth.layer_inputs(w, seed=41)
    pos = _positions(w.batch, w.seq, [0, 0])
    P = _params(w)
    base = oracle.prefill(P, _np(q), _np(k), _np(v), pos, None)
    neg_inf = oracle.prefill(P, _np(q), _np(k), _np(v), pos,
                             np.full(w.num_q_heads, -np.inf, np.float32))
    np.testing.assert_array_equal(neg_inf, base)
    with_sink = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s))
    # closed form: out_sink = out_plain * D / (D + exp(s_h)), D = sum of exp(scores) in window
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            z = oracle.scores(P, _np(q), _np(k), pos, b, h)
            for i in range(w.seq):
                js = [j for j in range(w.seq) if 0 <= i - j < w.window]
                D = sum(math.exp(z[i, j]) for j in js)
                ratio = D / (D + math.exp(float(s[h])))
                np.testing.assert_allclose(with_sink[b, i, h], base[b, i, h] * ratio,
                                           rtol=1e-12, atol=1e-14)
    huge = oracle.prefill(P, _np(q), _np(k), _np(v), pos, np.full(w.num_q_heads, 80, np.float32))
    assert np.abs(huge).max() < 1e-25
    mags = [np.abs(oracle.prefill(P, _np(q), _np(k), _np(v), pos,
                                  np.full(w.num_q_heads, sv, np.float32))).sum()
            for sv in (-2.0, 0.0, 2.0, 4.0)]
    assert all(a > b for a, b in zip(mags, mags[1:]))


def test_rope_dims_zero_ignores_theta_and_positions():
    w = _small(r=0)
    q, k, v, s = synth.layer_inputs(w, seed=51)
    a = oracle.prefill(_params(w, rope_theta=1e4), _np(q), _np(k), _np(v),
                       _positions(2, w.seq, [0, 0]), _np(s))
    b_ = oracle.prefill(_params(w, rope_theta=5e6), _np(q), _np(k), _np(v),
                        _positions(2, w.seq, [777, 31]), _np(s))
    np.testing.assert_array_equal(a, b_)


def test_common_position_shift_leaves_output_unchanged_and_theta_matters():
    w = _small(r=16, dqk=16, kind=1, W=6)
    q, k, v, s = synth.layer_inputs(w, seed=61)
    P = _params(w)
    a = oracle.prefill(P, _np(q), _np(k), _np(v), _positions(2, w.seq, [0, 0]), _np(s))
    b_ = oracle.prefill(P, _np(q), _np(k), _np(v), _positions(2, w.seq, [12345, 300]), _np(s))
    np.testing.assert_allclose(b_, a, rtol=0, atol=1e-9)
    c = oracle.prefill(_params(w, rope_theta=5e6), _np(q), _np(k), _np(v),
                       _positions(2, w.seq, [0, 0]), _np(s))
    assert np.abs(c - a).max() > 1e-3


def test_zero_query_gives_window_average_with_sink_term():
    for kind, W in [(1, 5), (0, 0)]:
        w = _small(kind=kind, W=W)
        _, k, v, s = synth.layer_inputs(w, seed=71)
        q = torch.zeros((w.batch, w.seq, w.num_q_heads, w.qk_head_dim))
        pos = _positions(w.batch, w.seq, [0, 9])
        out = oracle.prefill(_params(w), _np(q), _np(k), _np(v), pos, _np(s))
        vn = _np(v).astype(np.float64)
        grp = w.num_q_heads // w.num_kv_heads
        for b in range(w.batch):
            for i in range(w.seq):
                lo = max(0, i - W + 1) if kind == 1 else 0
                n = i - lo + 1
                for h in range(w.num_q_heads):
                    ref = w.v_scale * vn[b, lo:i + 1, h // grp].sum(0) / (n + math.exp(float(s[h])))
                    np.testing.assert_allclose(out[b, i, h], ref, rtol=1e-12, atol=1e-14)


def test_first_row_closed_form():
    w = _small(kind=1, W=3)
    q, k, v, s = synth.layer_inputs(w, seed=81)
    pos = _positions(w.batch, w.seq, [0, 4])
    P = _params(w)
    out = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s))
    plain = oracle.prefill(P, _np(q), _np(k), _np(v), pos, None)
    vn = _np(v).astype(np.float64)
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            z00 = oracle.scores(P, _np(q), _np(k), pos, b, h)[0, 0]
            ref = w.v_scale * vn[b, 0, h // grp] / (1.0 + math.exp(float(s[h]) - z00))
            np.testing.assert_allclose(out[b, 0, h], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(plain[b, 0, h], w.v_scale * vn[b, 0, h // grp], rtol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_and_output_linear_in_v_scale():
    w = _small(Hq=6, Hkv=2, kind=1, W=4)
    q, k, v, s = synth.layer_inputs(w, seed=91)
    pos = _positions(w.batch, w.seq, [0, 2])
    gqa = oracle.prefill(_params(w), _np(q), _np(k), _np(v), pos, _np(s))
    kr = k.repeat_interleave(3, dim=2)
    vr = v.repeat_interleave(3, dim=2)
    mha = oracle.prefill(_params(w, num_kv_heads=6), _np(q), _np(kr), _np(vr), pos, _np(s))
    np.testing.assert_array_equal(gqa, mha)
    scaled = oracle.prefill(_params(w, v_scale=w.v_scale * 3.0), _np(q), _np(k), _np(v), pos,
                            _np(s))
    np.testing.assert_allclose(scaled, 3.0 * gqa, rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------- decode


@pytest.mark.parametrize("kind,W", [(0, 0), (1, 5), (1, 40)])
def test_decode_after_prefill_equals_longer_prefill(kind, W):
    w = _small(kind=kind, W=W, Hq=4, Hkv=2, dqk=16, dv=8, r=6)
    S = w.seq
    q, k, v, s = synth.layer_inputs(w, seed=101, seq=S + 1)
    pos = _positions(w.batch, S + 1, [0, 0])
    P = _params(w)
    full = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s))
    _, krot = oracle.prefill(P, _np(q[:, :S]), _np(k[:, :S]), _np(v[:, :S]), pos[:, :S], _np(s),
                             want_k_rot=True)
    kc = np.ascontiguousarray(krot.transpose(0, 2, 1, 3)).astype(np.float32)  # B,Hkv,S,d
    vc = np.ascontiguousarray(_np(v[:, :S]).transpose(0, 2, 1, 3))
    kpos = pos[:, :S].copy()
    cnt = np.full(w.batch, S, np.int32)
    # float32 cache of fp64 rotated keys: compare within the float rounding of the keys
    dec = oracle.decode(P, _np(q[:, S]), _np(k[:, S]), _np(v[:, S]), pos[:, S], kc, vc, kpos,
                        cnt, _np(s))
    np.testing.assert_allclose(dec, full[:, S], rtol=0, atol=1e-5)
    # the ring holds only the last W-1 past keys in arbitrary slot order: same answer
    if kind == 1:
        keep = min(W - 1, S)
        order = np.random.default_rng(3).permutation(keep)
        sl = slice(S - keep, S)
        kc_r = np.ascontiguousarray(kc[:, :, sl][:, :, order])
        vc_r = np.ascontiguousarray(vc[:, :, sl][:, :, order])
        kpos_r = np.ascontiguousarray(kpos[:, sl][:, order])
        dec_r = oracle.decode(P, _np(q[:, S]), _np(k[:, S]), _np(v[:, S]), pos[:, S], kc_r, vc_r,
                              kpos_r, np.full(w.batch, keep, np.int32), _np(s))
        np.testing.assert_allclose(dec_r, dec, rtol=0, atol=1e-13)


def test_decode_with_empty_cache_returns_scaled_new_value():
    w = _small(kind=0, W=0, sinks=False)
    q, k, v, _ = synth.layer_inputs(w, seed=111, seq=1)
    P = _params(w)
    pos = np.array([0, 17], np.int32)
    out, krot = oracle.decode(P, _np(q[:, 0]), _np(k[:, 0]), _np(v[:, 0]), pos, want_k_rot=True)
    grp = w.num_q_heads // w.num_kv_heads
    vn = _np(v[:, 0]).astype(np.float64)
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(out[:, h], w.v_scale * vn[:, h // grp], rtol=1e-15)
    ref = oracle.rotate(_np(k[:, 0]), w.rope_dims, w.rope_theta,
                        np.repeat(pos[:, None], w.num_kv_heads, 1))
    np.testing.assert_array_equal(krot, ref)


# ----------------------------------------------------------------------------- extend


def _cache_of(krot, v, upto, starts):
    """position -> (rotated key, value) map of the first `upto` tokens of each sequence."""
    kc = np.ascontiguousarray(krot[:, :upto].transpose(0, 2, 1, 3)).astype(np.float32)
    vc = np.ascontiguousarray(_np(v[:, :upto]).transpose(0, 2, 1, 3))
    kpos = np.stack([np.arange(upto, dtype=np.int32) + s0 for s0 in starts])
    return kc, vc, kpos, np.full(len(starts), upto, np.int32)


@pytest.mark.parametrize("kind,W", [(0, 0), (1, 5), (1, 40)])
@pytest.mark.parametrize("split", [1, 4, 11])
def test_extend_equals_the_unsplit_prefill(kind, W, split):
    """Prefill the first `split` tokens, extend with the rest: the rows of the extension equal
    those rows of one prefill over the whole sequence (the prefill itself is pinned by SDPA)."""
    w = _small(kind=kind, W=W)
    T = w.seq
    starts = [0, 5]
    q, k, v, s = synth.layer_inputs(w, seed=131, seq=T)
    pos = _positions(w.batch, T, starts)
    P = _params(w)
    full, krot = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s), want_k_rot=True)
    kc, vc, kpos, cnt = _cache_of(krot, v, split, starts)
    ext, krot_new = oracle.extend(P, _np(q[:, split:]), _np(k[:, split:]), _np(v[:, split:]),
                                  np.array(starts) + split, kc, vc, kpos, cnt, _np(s),
                                  want_k_rot=True)
    # float32 cache of fp64 rotated keys: equal within the float rounding of the cached keys
    np.testing.assert_allclose(ext, full[:, split:], rtol=0, atol=1e-5)
    np.testing.assert_array_equal(krot_new, krot[:, split:])
    if kind == 1:
        # a ring keeps only the last W positions, in any slot order: same answer
        keep = min(W, split)
        order = np.random.default_rng(5).permutation(keep)
        sl = slice(split - keep, split)
        ext_r = oracle.extend(P, _np(q[:, split:]), _np(k[:, split:]), _np(v[:, split:]),
                              np.array(starts) + split,
                              np.ascontiguousarray(kc[:, :, sl][:, :, order]),
                              np.ascontiguousarray(vc[:, :, sl][:, :, order]),
                              np.ascontiguousarray(kpos[:, sl][:, order]),
                              np.full(w.batch, keep, np.int32), _np(s))
        np.testing.assert_allclose(ext_r, ext, rtol=0, atol=1e-13)


def test_extend_with_empty_cache_is_prefill_and_one_token_is_decode():
    w = _small(kind=1, W=5)
    q, k, v, s = synth.layer_inputs(w, seed=141)
    starts = np.array([3, 9], np.int32)
    P = _params(w)
    pf = oracle.prefill(P, _np(q), _np(k), _np(v), _positions(w.batch, w.seq, starts), _np(s))
    ex = oracle.extend(P, _np(q), _np(k), _np(v), starts, sinks=_np(s))
    np.testing.assert_array_equal(ex, pf)
    # one new token against a cache: the decode definition
    kc = np.random.default_rng(7).standard_normal((w.batch, w.num_kv_heads, 6, w.qk_head_dim))
    vc = np.random.default_rng(8).standard_normal((w.batch, w.num_kv_heads, 6, w.v_head_dim))
    kpos = np.stack([np.arange(6, dtype=np.int32) + 4, np.arange(6, dtype=np.int32) + 1])
    cnt = np.array([6, 6], np.int32)
    st = np.array([10, 7], np.int32)
    ex1 = oracle.extend(P, _np(q[:, :1]), _np(k[:, :1]), _np(v[:, :1]), st, kc, vc, kpos, cnt,
                        _np(s))
    dec = oracle.decode(P, _np(q[:, 0]), _np(k[:, 0]), _np(v[:, 0]), st, kc, vc, kpos, cnt,
                        _np(s))
    np.testing.assert_allclose(ex1[:, 0], dec, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- fp8 KV cache
# The codes and values are pinned against torch's float8_e4m3fn conversions (a different route
# than the oracle's bit-level definition); the attention over an fp8 cache against the float
# decode on the stored values.


def _e4m3_torch_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_torch_codes(y):
    """torch's nearest-even e4m3 codes of fp32 values, clamped to +-448 first (torch itself turns
    values that round past 448 into NaN)."""
    t = torch.from_numpy(np.asarray(y, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_probe_values():
    vals = _e4m3_torch_values()[:127].astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(17)
    rnd = np.concatenate([rng.standard_normal(4000) * sc for sc in (1e-3, 0.05, 1, 30, 300)])
    big = np.array([448, 449, 463.9, 464, 464.1, 479, 480, 1e6, np.inf], np.float32)
    x = np.concatenate([vals, mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf)), rnd.astype(np.float32), big])
    return np.concatenate([x, -x]).astype(np.float32)


def test_e4m3_values_match_torch():
    mine, ref = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)), _e4m3_torch_values()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.nonzero(np.isnan(ref))[0], [0x7F, 0xFF])
    # a scale multiplies every stored value
    np.testing.assert_array_equal(oracle.e4m3_decode(np.arange(127, dtype=np.uint8), 0.375),
                                  ref[:127] * 0.375)


@pytest.mark.parametrize("inv_scale", [1.0, 0.125, 1.0 / 0.37, 3.0])
def test_e4m3_codes_match_torch_nearest_even(inv_scale):
    x = _e4m3_probe_values()
    y = x * np.float32(inv_scale)          # the fp32 product the code is taken of
    assert np.array_equal(oracle.e4m3_encode(x, np.float32(inv_scale)), _e4m3_torch_codes(y))


def test_e4m3_round_trip_error_bound_and_saturation():
    x = _e4m3_probe_values()
    x = x[np.isfinite(x)]
    back = oracle.e4m3_decode(oracle.e4m3_encode(x))
    a = np.abs(x.astype(np.float64))
    inside = a <= 448
    # half a quantum: 2^-4 of the magnitude for normals (3 mantissa bits), 2^-10 for subnormals
    bound = np.maximum(a * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(back - x)[inside] <= bound[inside] * (1 + 1e-12))
    assert np.all(np.abs(back[~inside]) == 448) and np.all(np.sign(back[~inside]) == np.sign(x[~inside]))
    # the grid itself is a fixed point, zero keeps its sign
    grid = _e4m3_torch_values()[:127]
    assert np.array_equal(oracle.e4m3_decode(oracle.e4m3_encode(grid)), grid)
    assert oracle.e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80


def _fp8_cache_case(kind, r, seed, L=7, W=5):
    w = _small(kind=kind, W=W if kind == 1 else 0, Hq=4, Hkv=2, dqk=16, dv=8, r=r)
    B = w.batch
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, w.num_q_heads, w.qk_head_dim), generator=g)
    kn = torch.randn((B, w.num_kv_heads, w.qk_head_dim), generator=g).to(torch.bfloat16).float()
    vn = torch.randn((B, w.num_kv_heads, w.v_head_dim), generator=g).to(torch.bfloat16).float()
    s = torch.randn((w.num_q_heads,), generator=g) if w.sinks else None
    kc8 = (torch.randn((B, w.num_kv_heads, L, w.qk_head_dim), generator=g) * 4).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    vc8 = (torch.randn((B, w.num_kv_heads, L, w.v_head_dim), generator=g) * 4).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    pos = np.array([L, L + 3], np.int32)
    kpos = np.stack([np.arange(L, dtype=np.int32) + (p - L) for p in pos])   # positions p-L..p-1
    kpos = np.ascontiguousarray(kpos[:, np.random.default_rng(seed).permutation(L)])
    return w, q.numpy(), kn.numpy(), vn.numpy(), None if s is None else s.numpy(), kc8, vc8, pos, kpos


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_fp8_equals_float_decode_on_stored_values(kind):
    """No rotation (r = 0) and power-of-two scales: every stored value is exact in fp32, so the
    fp8 decode must equal the float decode given the stored values for the cache and for the new
    token (quantized by torch's conversion)."""
    w, q, kn, vn, s, kc8, vc8, pos, kpos = _fp8_cache_case(kind, r=0, seed=61)
    ks, vs = 0.125, 2.0
    P = _params(w)
    cnt = np.full(w.batch, kc8.shape[2], np.int32)
    out, _, kcode, vcode = oracle.decode_fp8(P, q, kn, vn, pos, kc8, vc8, kpos, cnt, ks, vs, s)
    tv = _e4m3_torch_values()
    kst = tv[_e4m3_torch_codes(kn * np.float32(1 / ks))] * ks
    vst = tv[_e4m3_torch_codes(vn * np.float32(1 / vs))] * vs
    assert np.array_equal(kcode, _e4m3_torch_codes(kn * np.float32(1 / ks)))
    assert np.array_equal(vcode, _e4m3_torch_codes(vn * np.float32(1 / vs)))
    ref = oracle.decode(P, q, kst, vst, pos, (tv[kc8] * ks).astype(np.float32),
                        (tv[vc8] * vs).astype(np.float32), kpos, cnt, s)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    # the new token really is the quantized one: the exact one gives another answer
    exact = oracle.decode(P, q, kn, vn, pos, (tv[kc8] * ks).astype(np.float32),
                          (tv[vc8] * vs).astype(np.float32), kpos, cnt, s)
    assert np.abs(exact - out).max() > 1e-4


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_fp8_quantizes_the_rotated_key(kind):
    """With rotation the new key is rotated first, then rounded to fp32, scaled and coded."""
    w, q, kn, vn, s, kc8, vc8, pos, kpos = _fp8_cache_case(kind, r=6, seed=62)
    ks, vs = 0.37, 1.7
    P = _params(w)
    cnt = np.full(w.batch, kc8.shape[2], np.int32)
    _, krot, kcode, vcode = oracle.decode_fp8(P, q, kn, vn, pos, kc8, vc8, kpos, cnt, ks, vs, s)
    _, krot_ref = oracle.decode(P, q, kn, vn, pos, want_k_rot=True)
    np.testing.assert_array_equal(krot, krot_ref)
    inv_k, inv_v = np.float32(1) / np.float32(ks), np.float32(1) / np.float32(vs)
    assert np.array_equal(kcode, _e4m3_torch_codes(krot.astype(np.float32) * inv_k))
    assert np.array_equal(vcode, _e4m3_torch_codes(vn * inv_v))


# ----------------------------------------------------------------------------- layer with projections


def test_prefill_f64_equals_float_prefill_on_float_inputs():
    w = _small(kind=1, W=5)
    q, k, v, s = synth.layer_inputs(w, seed=71)
    pos = _positions(w.batch, w.seq, [0, 3])
    P = _params(w)
    a = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s))
    b = oracle.prefill_f64(P, _np(q).astype(np.float64), _np(k).astype(np.float64),
                           _np(v).astype(np.float64), pos, _np(s))
    assert np.array_equal(a, b)


def _selection_weights(Hq, Hkv, dqk, dv):
    """Weights that copy consecutive slices of x into q, k and v, and the identity for Wo."""
    nq, nk, nv = Hq * dqk, Hkv * dqk, Hkv * dv
    H = nq + nk + nv
    eye = np.eye(H)
    return H, eye[:, :nq], eye[:, nq:nq + nk], eye[:, nq + nk:], np.eye(Hq * dv)


@pytest.mark.parametrize("kind", [0, 1])
def test_layer_with_selection_weights_is_the_attention(kind):
    """x = [q | k | v] per token, projections that select those slices and Wo = I: the layer is
    the (pinned) attention on q, k, v, heads contiguous in the columns."""
    w = _small(kind=kind, W=5 if kind else 0, Hq=4, Hkv=2, dqk=16, dv=8, r=6)
    H, wq, wk, wv, wo = _selection_weights(4, 2, 16, 8)
    q, k, v, s = synth.layer_inputs(w, seed=72)
    B, S = w.batch, w.seq
    x = np.concatenate([_np(q).reshape(B, S, -1), _np(k).reshape(B, S, -1),
                        _np(v).reshape(B, S, -1)], axis=2)
    pos = _positions(B, S, [0, 6])
    P = _params(w)
    got = oracle.layer_prefill(P, x, wq, wk, wv, wo, pos, _np(s))
    ref = oracle.prefill(P, _np(q), _np(k), _np(v), pos, _np(s)).reshape(B, S, -1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)
    # sampled rows: the same rows, the others NaN
    rows = np.array([0, 5, S - 1], np.int32)
    part = oracle.layer_prefill(P, x, wq, wk, wv, wo, pos, _np(s), rows=rows)
    np.testing.assert_allclose(part[:, rows], ref[:, rows], rtol=0, atol=1e-13)
    assert np.isnan(np.delete(part, rows, axis=1)).all()


def test_layer_is_linear_in_the_output_and_value_projections():
    w = _small(kind=1, W=4, Hq=4, Hkv=2, dqk=16, dv=8, r=6)
    B, S, H = w.batch, w.seq, 24
    rng = np.random.default_rng(73)
    x = rng.standard_normal((B, S, H))
    wq = rng.standard_normal((H, 4 * 16)) / 5
    wk = rng.standard_normal((H, 2 * 16)) / 5
    wv = rng.standard_normal((H, 2 * 8))
    wo = rng.standard_normal((4 * 8, 10))
    s = rng.standard_normal(4).astype(np.float32)
    pos = _positions(B, S, [0, 2])
    P = _params(w)
    base = oracle.layer_prefill(P, x, wq, wk, wv, wo, pos, s)
    np.testing.assert_allclose(oracle.layer_prefill(P, x, wq, wk, wv, 3 * wo, pos, s), 3 * base,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.layer_prefill(P, x, wq, wk, -2 * wv, wo, pos, s), -2 * base,
                               rtol=1e-12, atol=1e-12)
    # the value scale and a scale of Wo are interchangeable (folding v_scale into o_proj)
    P2 = _params(w, v_scale=1.0)
    np.testing.assert_allclose(oracle.layer_prefill(P2, x, wq, wk, wv, wo * P.v_scale, pos, s), base,
                               rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- MoE router


def _router_scores(x, bias):
    """torch route: fp64 sigmoid rounded to fp32, plus the bias in fp32."""
    s = torch.sigmoid(torch.from_numpy(np.asarray(x, np.float64))).float()
    return s, s + torch.from_numpy(np.asarray(bias, np.float32))


def test_router_sigmoid_is_the_rounded_fp64_sigmoid():
    x = np.concatenate([np.linspace(-30, 30, 2001), np.random.default_rng(80).standard_normal(5000) * 4])
    x = x.astype(np.float32)
    mine = np.array([oracle.router_sigmoid(v) for v in x], np.float32)
    ref = torch.sigmoid(torch.from_numpy(x.astype(np.float64))).float().numpy()
    assert np.array_equal(mine, ref)


@pytest.mark.parametrize("groups", [(1, 1), (8, 8)])
def test_router_keeping_every_group_is_plain_topk(groups):
    """One group, or every group kept: the choice is torch.topk of the selection scores, the
    weights the chosen sigmoids normalised and scaled."""
    G, TG = groups
    rng = np.random.default_rng(81)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    b = (rng.standard_normal(256) * 0.1).astype(np.float32)
    P = oracle.RouterParams(num_experts=256, n_group=G, topk_group=TG, top_k=8,
                            norm_topk_prob=True, routed_scaling_factor=2.5)
    idx, w = oracle.router(P, x, b)
    s, c = _router_scores(x, b)
    ref = torch.topk(c, 8, dim=1).indices.numpy()
    assert np.array_equal(idx, ref)
    sw = torch.gather(s, 1, torch.from_numpy(ref).long()).double().numpy()
    np.testing.assert_allclose(w, 2.5 * sw / sw.sum(1, keepdims=True), rtol=1e-15, atol=0)
    P.norm_topk_prob = False
    _, w2 = oracle.router(P, x, b)
    np.testing.assert_allclose(w2, 2.5 * sw, rtol=1e-15, atol=0)


@pytest.mark.parametrize("shape", [(8, 4, 2, 3), (12, 4, 2, 5), (16, 8, 3, 4)])
def test_router_brute_force_subsets(shape):
    """Tiny expert counts: the kept groups are the topk_group-subset with the largest total group
    score (group score = sum of its two best selection scores), and the chosen experts the
    top_k-subset of the kept groups' experts with the largest total selection score."""
    import itertools
    E, G, TG, K = shape
    gs = E // G
    rng = np.random.default_rng(82 + E)
    x = rng.standard_normal((40, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3 - 1.5).astype(np.float32)   # negative scores: -inf masking
    P = oracle.RouterParams(num_experts=E, n_group=G, topk_group=TG, top_k=K)
    idx, _ = oracle.router(P, x, b)
    _, c = _router_scores(x, b)
    c = c.double().numpy()
    for t in range(x.shape[0]):
        gsc = [np.sort(c[t, g * gs:(g + 1) * gs])[-2:].sum() for g in range(G)]
        keep = max(itertools.combinations(range(G), TG), key=lambda sub: sum(gsc[g] for g in sub))
        pool = [e for g in keep for e in range(g * gs, (g + 1) * gs)]
        best = max(itertools.combinations(pool, K), key=lambda sub: sum(c[t, e] for e in sub))
        assert set(idx[t]) == set(best), (t, idx[t], best)
        # rank order: selection scores descending
        assert all(c[t, idx[t][i]] >= c[t, idx[t][i + 1]] for i in range(K - 1))
        # masked with -inf: every chosen expert lies in a kept group, although scores are < 0
        assert all(e // gs in keep for e in idx[t])


def test_router_equal_scores_rank_lower_indices_first():
    """Every score equal: the first groups are kept and the lowest expert indices chosen, in
    index order (the tie rule)."""
    P = oracle.RouterParams(num_experts=256, n_group=8, topk_group=4, top_k=8)
    idx, w = oracle.router(P, np.zeros((3, 256), np.float32), np.zeros(256, np.float32))
    assert np.array_equal(idx, np.tile(np.arange(8, dtype=np.int32), (3, 1)))
    np.testing.assert_allclose(w, 1.0 / 8, rtol=1e-15)
    # a tie inside a later group that is kept: groups with equal scores also go by index
    x = np.zeros((1, 256), np.float32)
    x[0, 100] = 5.0     # group 3 gets the best score; the other groups tie
    idx, _ = oracle.router(P, x, np.zeros(256, np.float32))
    assert idx[0, 0] == 100 and list(idx[0, 1:]) == [0, 1, 2, 3, 4, 5, 6]


def test_oracle_rejects_invalid_arguments():
    w = _small()
    q, k, v, s = synth.layer_inputs(w, seed=1)
    pos = _positions(w.batch, w.seq, [0, 0])
    for bad in [dict(rope_dims=5), dict(rope_dims=18), dict(rope_theta=0.0), dict(window=0),
                dict(layer_kind=2)]:
        with pytest.raises(ValueError):
            oracle.prefill(_params(w, **bad), _np(q), _np(k), _np(v), pos, _np(s))
