"""Ideal bf16 arithmetic of the attention layer: a model of rounding, for the parity tests.

Test infrastructure only.  It takes the oracle's exact rotated queries and keys (oracle.rotate)
and computes the layer the way any bf16-operand / fp32-accumulate implementation has to, with
every value exact except for these roundings, each round-to-nearest-even to bf16 through fp32:
  * the rotated query and the rotated key (the matrix-core operands; inputs that are bf16 already,
    such as cache contents, are unchanged by it).  Where the query operand carries the score
    scale (prefill: q' times fp32(tau * log2 e), rounded once, the scores then taken in the log2
    domain), every query dim is rounded, not only the rotated ones;
  * the softmax weights e^{z - m} before the product with V (the sum in the denominator is taken
    from the unrounded weights);
  * the output v_scale * O / l.
Nothing else is rounded (scores, maxima and sums exact).  The difference between this model and the
fp64 oracle is the error that bf16 operands alone cause; a kernel that rounds at these points and
accumulates in fp32 should show about the same error, element by element and in L2.  It shares no
code with the HIP path and is not a second oracle: the oracle stays the reference the tests gate on.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def bf16(x) -> np.ndarray:
    """Round to bf16 through fp32 (RNE at both steps), returned as float64."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float64)))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _head(qr, kr, v, vis, sink, tau, v_scale):
    """One query head: qr [n, dqk], kr [m, dqk], v [m, dv] (already rounded operands), vis [n, m]."""
    z = tau * (qr @ kr.T)
    z = np.where(vis, z, -np.inf)
    m = z.max(axis=1) if z.shape[1] else np.full(z.shape[0], -np.inf)
    m = np.maximum(m, sink)
    mu = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - mu[:, None])
    l = e.sum(axis=1) + (np.exp(sink - mu) if np.isfinite(sink) else 0.0)
    o = bf16(e) @ v
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, v_scale * o / l[:, None], 0.0)
    return bf16(out)


U = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits, round to nearest)
BOUND_SIGMAS = 5.0


def error_bound(qr, kr, v, vis, sink, tau, v_scale, r, k_rotated, rq=None):
    """Per-element bound on |ideal bf16 arithmetic - exact| for one query head, derived from the
    rounding points above (first order).  qr [n, dqk] and kr [m, dqk] are the exact rotated rows;
    the first rq dims of the query (rq = r unless given: the query operand carries the score scale
    when rq = dqk) and the first r dims of the keys are rounded (the others are the bf16 inputs
    themselves), and only keys with k_rotated[j] (rotated in this call; cache contents are stored
    bf16 values) are rounded.
    Each rounding is an independent error of at most U relative, uniform (variance U^2/3):
      * score z_ij = tau q'_i.k'_j moves by tau sum_d (e_d + h_jd) q'_id k'_jd (e: query rounding,
        shared by every key of the row; h: key rounding), which moves o_i by
        sum_j p_ij (v_j - o_i) dz_ij;
      * a softmax weight's rounding moves o_i by p_ij rho_ij v_j;
    so the error of an output element has a standard deviation sigma computed here exactly from
    the exact p, o, q', k', v; the bound is BOUND_SIGMAS * sigma plus the output's own rounding
    (U |out|).  Returns (bound [n, dv], exact output [n, dv])."""
    n, m = vis.shape
    z = np.where(vis, tau * (qr @ kr.T), -np.inf)
    mx = np.maximum(z.max(axis=1) if m else np.full(n, -np.inf), sink)
    mu = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(z - mu[:, None])
    l = e.sum(axis=1) + (np.exp(sink - mu) if np.isfinite(sink) else 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        pm = np.where(l[:, None] > 0, e / l[:, None], 0.0)       # [n, m]
    o = pm @ v                                                   # [n, dv]
    var = (U * U / 3.0) * ((pm * pm) @ (v * v))                  # softmax-weight roundings
    rq = r if rq is None else rq
    if rq > 0:
        qa = qr[:, :rq]
        ka = kr[:, :rq]
        # query roundings: sum_d q'_id^2 (sum_j p_ij (v_jc - o_ic) k'_jd)^2
        cq = np.empty_like(o)
        for i0 in range(0, n, 32):
            sl = slice(i0, i0 + 32)
            a = np.matmul((pm[sl, :, None] * v[None]).transpose(0, 2, 1), ka)   # [i, dv, r]
            a -= o[sl, :, None] * (pm[sl] @ ka)[:, None, :]
            cq[sl] = np.einsum("id,icd->ic", qa[sl] * qa[sl], a * a)
        var += (tau * tau * U * U / 3.0) * cq
    if r > 0:
        qa = qr[:, :r]
        ka = kr[:, :r]
        # key roundings (independent per key and dim)
        wk = (qa * qa) @ (ka * ka * k_rotated[:, None]).T        # [n, m]
        x = pm * pm * wk
        var += (tau * tau * U * U / 3.0) * (x @ (v * v) - 2.0 * o * (x @ v) + o * o * x.sum(1)[:, None])
    sig = np.sqrt(np.maximum(var, 0.0))
    out = v_scale * o
    return v_scale * BOUND_SIGMAS * sig + U * np.abs(out) + 1e-6, out


# Rows that see more keys than this average their roundings away: their error stays inside the
# fixed 1e-2 + 2e-2 |x| bound (rel L2 ~2e-3), so the derived bound is left at 0 there (no widening)
# and the cost of computing it (rows x keys x dv x dqk) stays small.
BOUND_MAX_KEYS = 64


def _bound_rows(qr, K, V, vis, sink, tau, v_scale, r, k_rotated, rq, out):
    """error_bound for the rows of vis that see at most BOUND_MAX_KEYS keys (in blocks of 32
    rows, keys cut to the block's visible range); other rows keep out's value (0)."""
    cnt = vis.sum(axis=1)
    for i0 in range(0, vis.shape[0], 32):
        rows = np.arange(i0, min(i0 + 32, vis.shape[0]))
        rows = rows[cnt[rows] <= BOUND_MAX_KEYS]
        if rows.size == 0:
            continue
        cols = np.nonzero(vis[rows].any(axis=0))[0]
        if cols.size == 0:
            lo, hi = 0, 0
        else:
            lo, hi = int(cols[0]), int(cols[-1]) + 1
        out[rows] = error_bound(qr[rows], K[lo:hi], V[lo:hi], vis[rows][:, lo:hi], sink, tau,
                                v_scale, r, k_rotated[lo:hi], rq=rq)[0]


def prefill_bound(p: "oracle.OracleParams", q, k, v, positions, sinks=None, rows=None):
    """error_bound over a prefill (every key rotated in the call, the query operand carrying the
    score scale); rows not listed are NaN, rows seeing more than BOUND_MAX_KEYS keys 0."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    pos = np.asarray(positions, np.int32)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tau = p.softmax_scale if p.softmax_scale else 1.0 / np.sqrt(D)
    sel = np.arange(S) if rows is None else np.asarray(rows)
    bound = np.full((B, S, Hq, v.shape[-1]), np.nan)
    for b in range(B):
        qr = oracle.rotate(q[b, sel], p.rope_dims, p.rope_theta, np.repeat(pos[b, sel][:, None], Hq, 1))
        kr = oracle.rotate(k[b], p.rope_dims, p.rope_theta, np.repeat(pos[b][:, None], Hkv, 1))
        d = pos[b, sel][:, None] - pos[b][None, :]
        vis = d >= 0
        if p.layer_kind == 1:
            vis &= d < p.window
        for h in range(Hq):
            s = -np.inf if sinks is None else float(sinks[h])
            out = np.zeros((len(sel), v.shape[-1]))
            _bound_rows(qr[:, h], kr[:, h // G], v[b, :, h // G], vis, s, tau, p.v_scale,
                        p.rope_dims, np.ones(S, bool), D, out)
            bound[b, sel, h] = out
    return bound


def extend_bound(p: "oracle.OracleParams", q, k, v, start, kc=None, vc=None, kpos=None, count=None,
                 sinks=None, q_scaled=None):
    """error_bound over an extend (same arguments as oracle.extend): the cached keys are stored
    values (not rounded again), the new tokens' keys are rotated and rounded in the call.
    q_scaled: the query operand carries the score scale (every query dim rounded); by default
    when more than 16 tokens are new (the library's prefill kernel takes those).  Rows seeing
    more than BOUND_MAX_KEYS keys get 0."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    st = np.asarray(start, np.int32)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tau = p.softmax_scale if p.softmax_scale else 1.0 / np.sqrt(D)
    bound = np.zeros((B, S, Hq, v.shape[-1]))
    if q_scaled is None:
        q_scaled = S > 16
    for b in range(B):
        pos = st[b] + np.arange(S, dtype=np.int32)
        qr = oracle.rotate(q[b], p.rope_dims, p.rope_theta, np.repeat(pos[:, None], Hq, 1))
        kr = oracle.rotate(k[b], p.rope_dims, p.rope_theta, np.repeat(pos[:, None], Hkv, 1))
        n = 0 if kc is None else int(count[b])
        kp = np.concatenate([np.zeros(0, np.int32) if kc is None else np.asarray(kpos[b, :n]), pos])
        order = np.argsort(kp, kind="stable")   # keys by position, so visible ranges are contiguous
        kp = kp[order]
        d = pos[:, None] - kp[None, :]
        vis = d >= 0
        if p.layer_kind == 1:
            vis &= d < p.window
        rot = np.concatenate([np.zeros(n, bool), np.ones(S, bool)])[order]
        for h in range(Hq):
            g = h // G
            K = np.concatenate([np.asarray(kc[b, g, :n], np.float64) if n else np.zeros((0, D)), kr[:, g]])[order]
            V = np.concatenate([np.asarray(vc[b, g, :n], np.float64) if n else
                                np.zeros((0, v.shape[-1])), v[b, :, g]])[order]
            s = -np.inf if sinks is None else float(sinks[h])
            out = np.zeros((S, v.shape[-1]))
            _bound_rows(qr[:, h], K, V, vis, s, tau, p.v_scale, p.rope_dims, rot,
                        D if q_scaled else None, out)
            bound[b, :, h] = out
    return bound


def prefill(p: "oracle.OracleParams", q, k, v, positions, sinks=None, rows=None, block=256):
    """Model output of a prefill (same arguments as oracle.prefill); rows not listed are NaN.
    The query operand carries the score scale: q~ = bf16(q' * fp32(fp32(tau) * fp32(log2 e))),
    scores z = ln 2 * <q~, bf16(k')>."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    pos = np.asarray(positions, np.int32)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tau = p.softmax_scale if p.softmax_scale else 1.0 / np.sqrt(D)
    sel = np.arange(S) if rows is None else np.asarray(rows)
    out = np.full((B, S, Hq, v.shape[-1]), np.nan)
    for b in range(B):
        sc = float(np.float32(np.float32(tau) * np.float32(1.4426950408889634)))
        qr = bf16(sc * oracle.rotate(q[b, sel], p.rope_dims, p.rope_theta,
                                     np.repeat(pos[b, sel][:, None], Hq, 1)))
        kr = bf16(oracle.rotate(k[b], p.rope_dims, p.rope_theta,
                                np.repeat(pos[b][:, None], Hkv, 1)))
        vb = v[b]
        for i0 in range(0, len(sel), block):
            rs = sel[i0:i0 + block]
            pi = pos[b, rs]
            lo = 0 if p.layer_kind == 0 else max(0, int(rs.min()) - p.window + 1)
            hi = int(rs.max()) + 1
            d = pi[:, None] - pos[b, lo:hi][None, :]
            vis = d >= 0
            if p.layer_kind == 1:
                vis &= d < p.window
            for h in range(Hq):
                g = h // G
                s = -np.inf if sinks is None else float(sinks[h])
                out[b, rs, h] = _head(qr[i0:i0 + block, h], kr[lo:hi, g], vb[lo:hi, g], vis, s,
                                      np.log(2.0), p.v_scale)
    return out


def decode(p: "oracle.OracleParams", q, k_new, v_new, pos, kc=None, vc=None, kpos=None,
           count=None, sinks=None):
    """Model output of one decode step (same arguments as oracle.decode): the cached keys are taken
    as given (rotated, and bf16 when they come from a bf16 cache), the new token is rotated and
    rounded like the query."""
    q, k_new, v_new = (np.asarray(a, np.float64) for a in (q, k_new, v_new))
    pos = np.asarray(pos, np.int32)
    B, Hq, D = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    tau = p.softmax_scale if p.softmax_scale else 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, v_new.shape[-1]))
    for b in range(B):
        P = int(pos[b])
        qr = bf16(oracle.rotate(q[b], p.rope_dims, p.rope_theta, np.full(Hq, P, np.int32)))
        kn = bf16(oracle.rotate(k_new[b], p.rope_dims, p.rope_theta, np.full(Hkv, P, np.int32)))
        n = 0 if kc is None else int(count[b])
        kp = np.zeros(0, np.int32) if kc is None else np.asarray(kpos[b, :n])
        keep = kp <= P - 1
        if p.layer_kind == 1:
            keep &= kp > P - p.window
        for h in range(Hq):
            g = h // G
            ks = [kn[g][None]]
            vs = [v_new[b, g][None]]
            if n:
                ks.insert(0, np.asarray(kc[b, g, :n], np.float64)[keep])
                vs.insert(0, np.asarray(vc[b, g, :n], np.float64)[keep])
            K, V = np.concatenate(ks), np.concatenate(vs)
            s = -np.inf if sinks is None else float(sinks[h])
            out[b, h] = _head(qr[h][None], K, V, np.ones((1, len(K)), bool), s, tau,
                              p.v_scale)[0]
    return out


def rel_l2(x, ref) -> float:
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def layer_prefill(p: "oracle.OracleParams", x, wq, wk, wv, wo, positions, sinks=None, rows=None):
    """Model output of the layer with its projections (same arguments as oracle.layer_prefill),
    with the roundings of the library's path: q = bf16(x Wq) and v = bf16(x Wv) (products exact,
    rounded once); keys rotated from the exact product x Wk and rounded once; then the prefill's
    own roundings (the rotated query scaled and rounded, softmax weights, output) over those q, k,
    v with v_scale 1; out = bf16(v_scale * attn Wo).  Rows not listed are NaN."""
    x = np.asarray(x, np.float64)
    B, S, H = x.shape
    wq, wk, wv, wo = (np.asarray(a, np.float64) for a in (wq, wk, wv, wo))
    pos = np.asarray(positions, np.int32)
    Hq, Hkv, D, DVv = p.num_q_heads, p.num_kv_heads, p.qk_head_dim, p.v_head_dim
    G = Hq // Hkv
    sel = np.arange(S) if rows is None else np.asarray(rows)
    q = np.zeros((B, S, Hq, D))
    q[:, sel] = bf16(x[:, sel] @ wq).reshape(B, len(sel), Hq, D)
    k = (x @ wk).reshape(B, S, Hkv, D)
    v = bf16(x @ wv).reshape(B, S, Hkv, DVv)
    tau = p.softmax_scale if p.softmax_scale else 1.0 / np.sqrt(D)
    sc = float(np.float32(np.float32(tau) * np.float32(1.4426950408889634)))
    attn = np.full((B, S, Hq, DVv), np.nan)
    for b in range(B):
        qr = bf16(sc * oracle.rotate(q[b, sel], p.rope_dims, p.rope_theta,
                                     np.repeat(pos[b, sel][:, None], Hq, 1)))
        kr = bf16(oracle.rotate(k[b], p.rope_dims, p.rope_theta, np.repeat(pos[b][:, None], Hkv, 1)))
        d = pos[b, sel][:, None] - pos[b][None, :]
        vis = d >= 0
        if p.layer_kind == 1:
            vis &= d < p.window
        for h in range(Hq):
            s = -np.inf if sinks is None else float(sinks[h])
            attn[b, sel, h] = _head(qr[:, h], kr[:, h // G], v[b, :, h // G], vis, s, np.log(2.0), 1.0)
    out = np.full((B, S, wo.shape[1]), np.nan)
    out[:, sel] = bf16(p.v_scale * (attn[:, sel].reshape(B, len(sel), -1) @ wo))
    return out


def layer_row_tolerance(model, ref, sigmas=6.0):
    """Per-element tolerance of the layer output derived from the model: sigmas times the RMS of
    the model's own error over the element's row (rows that see few keys keep larger errors, and
    each row has out_dim elements to estimate it from), plus two roundings of the output."""
    e = np.asarray(model, np.float64) - np.asarray(ref, np.float64)
    rms_row = np.sqrt(np.nanmean(e * e, axis=-1, keepdims=True))
    return sigmas * rms_row + 2 * U * np.abs(ref)
