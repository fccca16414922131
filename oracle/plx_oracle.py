"""fp64 CPU oracle of the Parallax operator -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
does, and this module imports nothing from the product path.

What it computes (the Parallax output, eta = 0):

    o_i = o_i^SA - Sigma_KV^(i) rho_i

* o^SA is softmax attention: the write-ups' formula o_PLX = o_SA - Sigma_KV rho
  ("当注意力学会追问：Parallax如何给Transformer装上第二只眼", section 1.3) and the
  technical summary ("Riepilogo Tecnico: Parallax ...", section "Meccanismo
  Principale") define the output as softmax attention minus a KV-covariance
  correction applied to a per-token probe rho_i.
* eta, the boundary-amplification factor, is set to zero (same summary,
  bullet "Rimozione dell'Amplificazione del Confine").
* Sigma_KV^(i) is written out here as the softmax-weighted covariance
      Sigma_KV^(i) = sum_j w_ij (v_j - vbar_i)(k_j - kbar_i)^T,
      w_ij = softmax_j(tau q_i . k_j),  vbar_i = sum_j w_ij v_j,  kbar_i = sum_j w_ij k_j,
  a d_v x d_k matrix built explicitly for every query.  The pages only call it
  "the weighted covariance of KV"; the explicit weighted form, with weights
  that sum to one (a population covariance, no n-1), is the reading used.

Readings where the pages are silent: causal key set j <= i (diagonal
included) for prefill; a decode query sees all ctx_len[b] cache rows; query
head h uses KV head floor(h / (Hq / Hkv)); LSE is the natural log-sum-exp of
the scaled scores; there is no window (the bandwidth is the softmax
temperature tau).

Backward: the pages give none.  ``row_backward`` is the reverse-mode chain
rule taken step by step through the explicit forward above (scores ->
softmax -> moments -> covariance -> output), with rho an independent input.

Family corners (``uniform_weights``, ``row_family``, ``prefill_forward_family``,
``decode_forward_family``): the unified family ("当注意力学会追问...", section
2.1) places Parallax at softmax weights + learned probe + intercept and names
two other axes taken here as switches: the bandwidth axis's far end
(h -> infinity) gives every key of the set the weight 1/n, and the affine
axis's no-intercept end sets vbar = kbar = 0, so the covariance becomes the
uncentred second moment sum_j w_j v_j k_j^T and o = -Sigma rho (with uniform
weights: causal linear attention with query -rho and 1/n normalisation).
The correction-to-output ratio (the COR the technical summary tracks,
section "Risultati Sperimentali", and the metric of "Внимание нового
поколения...", section "Анализ Parallax: Выводы из внутренних метрик") is read
as ||Sigma_KV rho||_2 / ||o||_2 per query, Euclidean norms over d_v.

Projection (``project_qkvr``): the probe is a learned linear map of the
layer input, rho_i = W_R x_i ("当注意力学会追问...", section 1.3; technical
summary, section "Meccanismo Principale"), an extra projection beside the
query, key and value ones.  Read here as one stacked weight
[W_Q; W_K; W_V; W_R] applied to every token, each block split into heads of
d rows, head-major, and the results laid out [B, H, T, d].

All arithmetic is float64 on the exact (already dtype-rounded) inputs.  The
per-row functions only use +, -, *, @ and sums once the weights are known, so
``row_from_weights`` also runs on numpy object arrays of ``fractions.Fraction``
for exact-arithmetic checks.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "softmax_weights",
    "row_from_weights",
    "row_forward",
    "prefill_forward",
    "prefill_rows",
    "decode_forward",
    "row_backward",
    "prefill_backward",
    "prefill_backward_kv_rows",
    "prefill_backward_rows",
    "prefill_backward_group",
    "uniform_weights",
    "row_family",
    "correction_to_output",
    "prefill_forward_family",
    "decode_forward_family",
    "project_qkvr",
]


def softmax_weights(scores: np.ndarray):
    """w = softmax(scores), and LSE = log sum exp(scores) (natural log)."""
    m = np.max(scores)
    e = np.exp(scores - m)
    z = np.sum(e)
    return e / z, m + np.log(z)


def row_from_weights(w, K, V, rho):
    """Parallax output of one query given its attention weights.

    w: (n,) weights summing to one; K: (n, d_k); V: (n, d_v); rho: (d_k,).
    Returns (o, vbar, kbar, Sigma) with Sigma the explicit d_v x d_k weighted
    KV covariance and o = vbar - Sigma @ rho.
    """
    vbar = w @ V
    kbar = w @ K
    dv = V - vbar  # rows v_j - vbar
    dk = K - kbar  # rows k_j - kbar
    sigma = (dv * w[:, None]).T @ dk  # sum_j w_j (v_j - vbar)(k_j - kbar)^T
    o = vbar - sigma @ rho
    return o, vbar, kbar, sigma


def row_forward(q, K, V, rho, scale):
    """One query row: returns (o, o_sa, lse, sigma)."""
    s = scale * (K @ q)
    w, lse = softmax_weights(s)
    o, vbar, _kbar, sigma = row_from_weights(w, K, V, rho)
    return o, vbar, lse, sigma


def _kv_head(h, Hq, Hkv):
    return h // (Hq // Hkv)


def prefill_forward(q, k, v, rho, scale):
    """Causal prefill.  q, rho: [B, Hq, T, d]; k, v: [B, Hkv, T, d] (float64).

    Returns dict(o, o_sa, lse, c) with o, o_sa [B, Hq, T, d_v], lse [B, Hq, T]
    and c = kbar_i . rho_i [B, Hq, T] (the probe's projection on the mean key).
    """
    B, Hq, T, _ = q.shape
    Hkv = k.shape[1]
    dv = v.shape[-1]
    o = np.empty((B, Hq, T, dv))
    o_sa = np.empty((B, Hq, T, dv))
    lse = np.empty((B, Hq, T))
    c = np.empty((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            for i in range(T):
                K, V = k[b, hk, : i + 1], v[b, hk, : i + 1]
                w, lse[b, h, i] = softmax_weights(scale * (K @ q[b, h, i]))
                o[b, h, i], o_sa[b, h, i], kbar, _ = row_from_weights(w, K, V, rho[b, h, i])
                c[b, h, i] = kbar @ rho[b, h, i]
    return {"o": o, "o_sa": o_sa, "lse": lse, "c": c}


def prefill_rows(get_row, rows, Hq, Hkv, scale):
    """Causal prefill on sampled rows only.

    ``get_row(b, h, hk, i)`` returns (q_i, K[:i+1], V[:i+1], rho_i) as float64;
    ``rows`` is an iterable of (b, h, i).  Returns (o, lse) stacked in row order.
    """
    outs, lses = [], []
    for b, h, i in rows:
        hk = _kv_head(h, Hq, Hkv)
        qi, K, V, ri = get_row(b, h, hk, i)
        o, _, lse, _ = row_forward(qi, K, V, ri, scale)
        outs.append(o)
        lses.append(lse)
    return np.array(outs), np.array(lses)


def decode_forward(q, rho, k_cache, v_cache, ctx_len, scale, heads=None):
    """Decode: one query per (b, h) against cache rows [0, ctx_len[b]).

    q, rho: [B, Hq, d]; k_cache, v_cache: [B, Hkv, S_max, d] (float64 or a
    callable ``kv(b, hk, n) -> (K, V)``).  ``heads`` optionally restricts the
    work to a list of (b, h).  Returns dict(o, lse) over the requested heads.
    """
    B, Hq, _ = q.shape
    if callable(k_cache):
        Hkv = v_cache
        fetch = k_cache
    else:
        Hkv = k_cache.shape[1]

        def fetch(b, hk, n):
            return k_cache[b, hk, :n], v_cache[b, hk, :n]

    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    o, lse = [], []
    for b, h in heads:
        hk = _kv_head(h, Hq, Hkv)
        K, V = fetch(b, hk, int(ctx_len[b]))
        ob, _, lb, _ = row_forward(q[b, h], K, V, rho[b, h], scale)
        o.append(ob)
        lse.append(lb)
    return {"o": np.array(o), "lse": np.array(lse), "heads": heads}


def row_backward(q, K, V, rho, g, scale):
    """Gradients of <g, o> for one query row, by reverse mode through the
    explicit forward.  Returns (dq, dK, dV, drho) with dK, dV shaped like K, V.
    """
    n = K.shape[0]
    # forward, keeping every intermediate
    s = scale * (K @ q)
    w, _ = softmax_weights(s)
    vbar = w @ V
    kbar = w @ K
    a = V - vbar  # a_j = v_j - vbar
    bk = K - kbar  # b_j = k_j - kbar
    sigma = (a * w[:, None]).T @ bk
    # o = vbar - sigma @ rho
    d_vbar = g.copy()
    d_sigma = -np.outer(g, rho)
    d_rho = -sigma.T @ g
    # sigma = sum_j w_j a_j b_j^T
    a_ds = a @ d_sigma  # row j: a_j^T dSigma
    d_w = np.sum(a_ds * bk, axis=1)  # a_j^T dSigma b_j
    d_a = w[:, None] * (bk @ d_sigma.T)  # w_j dSigma b_j
    d_b = w[:, None] * a_ds  # w_j dSigma^T a_j
    dV = d_a.copy()
    dK = d_b.copy()
    d_vbar = d_vbar - d_a.sum(axis=0)  # a_j = v_j - vbar
    d_kbar = -d_b.sum(axis=0)  # b_j = k_j - kbar
    # vbar = sum_j w_j v_j ; kbar = sum_j w_j k_j
    d_w = d_w + V @ d_vbar + K @ d_kbar
    dV += np.outer(w, d_vbar)
    dK += np.outer(w, d_kbar)
    # w = softmax(s)
    d_s = w * (d_w - np.dot(w, d_w))
    # s = scale * K q
    dq = scale * (d_s @ K)
    dK += scale * np.outer(d_s, q)
    assert dK.shape == (n, K.shape[1])
    return dq, dK, dV, d_rho


def prefill_backward(q, k, v, rho, d_o, scale):
    """Full causal backward.  Returns dict(dq, dk, dv, drho), GQA K/V gradients
    summed over the query heads that share a KV head."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    drho = np.zeros_like(rho)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            for i in range(T):
                gq, gK, gV, gr = row_backward(q[b, h, i], k[b, hk, : i + 1], v[b, hk, : i + 1],
                                              rho[b, h, i], d_o[b, h, i], scale)
                dq[b, h, i] = gq
                drho[b, h, i] = gr
                dk[b, hk, : i + 1] += gK
                dv[b, hk, : i + 1] += gV
    return {"dq": dq, "dk": dk, "dv": dv, "drho": drho}


def prefill_backward_kv_rows(get_row, keys, T, Hq, Hkv, scale):
    """dK and dV of sampled keys (b, hk, j): sums over every query row i >= j of
    every query head of the group.  ``get_row(b, h, hk, i)`` returns
    (q_i, K[:i+1], V[:i+1], rho_i, g_i) as float64.  Returns (dk, dv) stacked."""
    group = Hq // Hkv
    dks, dvs = [], []
    for b, hk, j in keys:
        acc_k = None
        acc_v = None
        for h in range(hk * group, (hk + 1) * group):
            for i in range(j, T):
                qi, K, V, ri, gi = get_row(b, h, hk, i)
                _, gK, gV, _ = row_backward(qi, K, V, ri, gi, scale)
                acc_k = gK[j] if acc_k is None else acc_k + gK[j]
                acc_v = gV[j] if acc_v is None else acc_v + gV[j]
        dks.append(acc_k)
        dvs.append(acc_v)
    return np.array(dks), np.array(dvs)


def prefill_backward_rows(get_row, rows, Hq, Hkv, scale):
    """dQ and drho of sampled query rows (b, h, i).  ``get_row(b, h, hk, i)``
    returns (q_i, K[:i+1], V[:i+1], rho_i, g_i) as float64.  Returns (dq, drho)
    stacked in row order."""
    dqs, drs = [], []
    for b, h, i in rows:
        qi, K, V, ri, gi = get_row(b, h, _kv_head(h, Hq, Hkv), i)
        dq, _, _, dr = row_backward(qi, K, V, ri, gi, scale)
        dqs.append(dq)
        drs.append(dr)
    return np.array(dqs), np.array(drs)


def prefill_backward_group(q, k, v, rho, g, scale, magnitudes=False, rows_per_step=256):
    """Whole-group backward in closed form, on dense causal matrices.

    One KV head and the G query heads that share it: q, rho, g [G, T, d];
    k, v [T, d] (float64).  This is the second form of the backward, for
    sizes where ``row_backward``'s explicit d x d covariance per row is too
    slow (a full T = 4096 group).  It writes the gradient of <g, o> out
    directly from o_i = sum_j w_ij (1 + c_i - r_ij) v_j (the same o as
    ``row_from_weights``: vbar - Sigma rho expanded against rho):
        A_ij = g_i . v_j,  G_i = g_i . o_i,  delta_i = g_i . vbar_i,
        dV_j  = sum_i w_ij (1 + c_i - r_ij) g_i,
        dS_ij = w_ij [(1 + c_i - r_ij) A_ij - G_i + delta_i (r_ij - c_i)],
        dR_ij = -w_ij (A_ij - delta_i),
        dQ = tau dS K,  dK = tau dS^T Q + dR^T rho,  drho = dR K,
    with dK and dV summed over the G heads.  Query rows are taken
    ``rows_per_step`` at a time (each row against its causal keys, masked
    to j <= i); the CPU tests pin the result to ``prefill_backward``
    (reverse mode through the explicit covariance).

    Returns dict(dq, drho [G, T, d], dk, dv [T, d]).  With ``magnitudes`` it
    also returns, per gradient element, the sum of the absolute values of
    the products that make it up (``m_dq`` ...), each factor replaced by a
    bound on its own magnitude (|1 + c - r| by 1 + |c| + |r|, and so on): the
    scale against which a floating-point evaluation's rounding is measured.
    """
    G, T, d = q.shape
    out = {"dq": np.zeros((G, T, d)), "drho": np.zeros((G, T, d)),
           "dk": np.zeros((T, d)), "dv": np.zeros((T, d))}
    if magnitudes:
        for n in ("m_dq", "m_drho", "m_dk", "m_dv"):
            out[n] = np.zeros_like(out[n[2:]])
    for h in range(G):
        for i0 in range(0, T, rows_per_step):
            i1 = min(T, i0 + rows_per_step)
            K, V = k[:i1], v[:i1]  # every key some row of the step sees
            qh, rh, gh = q[h, i0:i1], rho[h, i0:i1], g[h, i0:i1]
            causal = np.arange(i1)[None, :] <= np.arange(i0, i1)[:, None]
            s = np.where(causal, scale * (qh @ K.T), -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            w = e / e.sum(axis=1, keepdims=True)
            r = rh @ K.T
            a = gh @ V.T
            c = np.sum(w * r, axis=1)
            vbar = w @ V
            o = vbar * (1.0 + c)[:, None] - (w * r) @ V
            Gi = np.sum(gh * o, axis=1)
            dl = np.sum(gh * vbar, axis=1)
            f = 1.0 + c[:, None] - r
            ds = w * (f * a - Gi[:, None] + dl[:, None] * (r - c[:, None]))
            dr = -w * (a - dl[:, None])
            out["dq"][h, i0:i1] = scale * (ds @ K)
            out["drho"][h, i0:i1] = dr @ K
            out["dk"][:i1] += scale * (ds.T @ qh) + dr.T @ rh
            out["dv"][:i1] += (w * f).T @ gh
            if magnitudes:
                fa = 1.0 + np.abs(c)[:, None] + np.abs(r)
                dsa = w * (fa * np.abs(a) + np.abs(Gi)[:, None]
                           + np.abs(dl)[:, None] * (np.abs(r) + np.abs(c)[:, None]))
                dra = w * (np.abs(a) + np.abs(dl)[:, None])
                out["m_dq"][h, i0:i1] = scale * (dsa @ np.abs(K))
                out["m_drho"][h, i0:i1] = dra @ np.abs(K)
                out["m_dk"][:i1] += scale * (dsa.T @ np.abs(qh)) + dra.T @ np.abs(rh)
                out["m_dv"][:i1] += (w * fa).T @ np.abs(gh)
    return out


# -- family corners and the correction-to-output ratio -------------------------


def uniform_weights(n):
    """Weights at the far end of the bandwidth axis: 1/n on each of the n keys.
    The LSE reported with them is ln n (every unnormalised weight is one)."""
    return np.full(n, 1.0 / n), np.log(n)


def row_family(w, K, V, rho, intercept=True):
    """Output and probe correction of one query for a corner of the family.

    intercept=True: the weighted moments are centred (the Parallax form),
    o = vbar - Sigma rho with Sigma the covariance of ``row_from_weights``.
    intercept=False: vbar = kbar = 0, Sigma = sum_j w_j v_j k_j^T and
    o = -Sigma rho.  Returns (o, corr) with corr = Sigma @ rho.
    Uses only +, -, * and @, so it runs on Fraction object arrays too.
    """
    if intercept:
        o, vbar, _kbar, sigma = row_from_weights(w, K, V, rho)
    else:
        sigma = (V * w[:, None]).T @ K  # sum_j w_j v_j k_j^T
        o = -(sigma @ rho)
    return o, sigma @ rho


def correction_to_output(corr, o):
    """||corr||_2 / ||o||_2 (IEEE: inf or nan when o = 0)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.float64(np.linalg.norm(corr)) / np.float64(np.linalg.norm(o))


def _family_row(q, K, V, rho, scale, uniform, intercept):
    if uniform:
        w, lse = uniform_weights(K.shape[0])
    else:
        w, lse = softmax_weights(scale * (K @ q))
    o, corr = row_family(w, K, V, rho, intercept)
    return o, lse, correction_to_output(corr, o)


def prefill_forward_family(q, k, v, rho, scale, uniform=False, intercept=True):
    """Causal prefill at a corner of the family.  Shapes as ``prefill_forward``.
    Returns dict(o, lse, cor); cor is [B, Hq, T]."""
    B, Hq, T, _ = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, Hq, T, v.shape[-1]))
    lse = np.empty((B, Hq, T))
    cor = np.empty((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            for i in range(T):
                o[b, h, i], lse[b, h, i], cor[b, h, i] = _family_row(
                    q[b, h, i], k[b, hk, : i + 1], v[b, hk, : i + 1], rho[b, h, i], scale,
                    uniform, intercept)
    return {"o": o, "lse": lse, "cor": cor}


def decode_forward_family(q, rho, k_cache, v_cache, ctx_len, scale, uniform=False,
                          intercept=True):
    """Decode at a corner of the family: q, rho [B, Hq, d]; caches
    [B, Hkv, S_max, d].  Returns dict(o [B, Hq, d], lse [B, Hq], cor [B, Hq])."""
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[1]
    o = np.empty((B, Hq, v_cache.shape[-1]))
    lse = np.empty((B, Hq))
    cor = np.empty((B, Hq))
    for b in range(B):
        n = int(ctx_len[b])
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            o[b, h], lse[b, h], cor[b, h] = _family_row(
                q[b, h], k_cache[b, hk, :n], v_cache[b, hk, :n], rho[b, h], scale, uniform,
                intercept)
    return {"o": o, "lse": lse, "cor": cor}


# -- the projection in front of the operator -----------------------------------


def project_qkvr(x, W, Hq, Hkv, d):
    """x: [B, T, D_model]; W: [(2 Hq + 2 Hkv) d, D_model], the row blocks
    W_Q (Hq d rows), W_K (Hkv d), W_V (Hkv d), W_R (Hq d), head-major inside a
    block.  Every token's projection is y = W x_t; block rows h d .. h d + d-1
    are head h.  Returns (q, k, v, rho) shaped [B, H, T, d]."""
    B, T, _ = x.shape
    y = x @ W.T  # [B, T, N]
    outs = []
    off = 0
    for H in (Hq, Hkv, Hkv, Hq):
        blk = y[:, :, off: off + H * d].reshape(B, T, H, d)
        outs.append(np.ascontiguousarray(blk.transpose(0, 2, 1, 3)))
        off += H * d
    assert off == W.shape[0]
    return tuple(outs)
