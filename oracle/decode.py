"""KVFetch oracle ("Verify Before You Fetch", Algorithm 2 and §4.2).

One decode decision = one query head of one request in one layer. For a
KV head g with resident rows R = H u S (exact K/V on the GPU), the inclusion
probabilities r (H <=> r == 1, L <=> r < 1, S = R n L) and a key sketch, the
oracle computes, in float64, in the order of Algorithm 2:

1. Exact logits l_j = <q, k_j>/sqrt(d) on R and planning logits s_i on L,
   either from the sketch, s_i = <P^T q, sk_i>/sqrt(d) (SKETCH), or from the
   exact keys (PERFECT, the "perfect sketch" of §4.2). A common shift m is
   subtracted (reading R5); w = exp(l - m), w~ = exp(s - m) (§3, eq. 1).
2. The plug-in denominator D~ = sum_H w + sum_L w~ (reading R7).
3. The bounded-shrinkage fixed point (Definition 2, eq. 5): beta* solves
   beta = sum_L w~_i (1 - lambda_i(beta)) with
   lambda_i(beta) = clip_[r_i,1](beta r_i / (w~_i (1 - r_i))); bisection in
   float64 (reading R8; Theorem 1 makes it the unique minimiser of eq. 6).
4. Lemma 1 / eq. 7: beta(L), V(L), b(L) and the certificate eps^(L).
   With the binary estimator of Appendix A.2 the coefficients are instead
   lambda_i in {1, r_i}: L is visited in decreasing w~_i (1 - r_i) / r_i
   and a token moves to lambda_i = r_i while that value exceeds twice the
   bias already accumulated.
5. If eps^(L) < eps: no fetch (reading R10: strict).
6. Otherwise gains g_i = eps^(L) - eps^(L \\ {i}) (eq. 9) in the
   cancellation-free closed form (reading R11), order L by (g desc,
   position asc) (reading R12), and take k* = the first k with
   eps^(L_g[k:]) < eps, evaluated with fixed coefficients and fixed D~
   (eq. 10, Theorem 2; reading R13).
7. Fetch F_h = L_g[:k*] minus S; the output uses exact weights on H u F_h and
   lambda_i w_i / r_i on S \\ F_h (Theorem 2's estimator; reading R15), with
   the same coefficients in the numerator (reading R16).

With the pages' deployed sketch (SKETCH2: 2-bit keys over 16 RoPE channel
pairs and an exact shortlist, Appendix A.1; oracle.sketch2), step 1 plans
with exact logits on S and on the shortlist and with the 2-bit sketch's
logits on the rest of L.
"""

import math

import numpy as np

from oracle import sketch2 as sk2

EST_CLIP = 0
EST_UNBIASED = 1
EST_BINARY = 2
W_SKETCH = 0
W_PERFECT = 1
W_SKETCH2 = 2


def bernstein_consts(delta):
    """l_delta = ln(2/delta) (natural log, reading R9) and a = l_delta / 3."""
    l = math.log(2.0 / delta)
    return l, l / 3.0


def lambdas(w, r, beta):
    """lambda_i = clip_[r_i, 1](beta r_i / (w_i (1 - r_i))) (Definition 2).

    A token with w_i == 0 contributes nothing; its lambda is set to 1.
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = beta * r / (w * (1.0 - r))
    lam = np.minimum(1.0, np.maximum(r, x))
    return np.where(w > 0, lam, 1.0)


def shrink_residual(beta, w, r):
    """h(beta) = sum_L w_i (1 - lambda_i(beta)) - beta; decreasing in beta."""
    return float(np.sum(w * (1.0 - lambdas(w, r, beta)))) - beta


def shrinkage_beta(w, r, max_iter=200):
    """Root beta* of the Definition 2 fixed point by float64 bisection.

    h(0) = sum w (1 - r) > 0 when L carries weight, h(sum w (1-r)) <= 0, and h
    is continuous and strictly decreasing, so the root is unique. The loop
    stops when the bracket is within 2^-52 of its upper end.
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    hi = float(np.sum(w * (1.0 - r)))
    if not hi > 0.0:
        return 0.0
    lo = 0.0
    for _ in range(max_iter):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if shrink_residual(mid, w, r) > 0.0:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 2.0 ** -52 * hi:
            break
    return 0.5 * (lo + hi)


def binary_lambdas(w, r, pos, moves=None):
    """Binary shrinkage (Appendix A.2, Figure 2): lambda_i in {1, r_i}.

    Moving token i from lambda_i = 1 to r_i adds the bias a_i = w_i (1 - r_i)
    and changes the MSE (eq. 6) by a_i (2 beta - w_i (1 - r_i) / r_i), beta
    being the bias of the tokens moved before it. Tokens are visited by
    kappa_i = w_i (1 - r_i) / r_i descending, ties by ascending position
    (reading: the order of equal kappa is left open; positions make it
    unique, as for the gain order), and moved while kappa_i > 2 beta
    (strict: a move that leaves the MSE unchanged is not made). Along the
    order kappa falls and beta grows, so the first token that fails ends the
    moves. Returns (lambda, beta, number moved).

    ``moves``: when given, exactly the first ``moves`` tokens of the order
    are moved instead of applying the stopping test (to evaluate the plan
    under another implementation's decision).
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    kappa = w * (1.0 - r) / r
    lam = np.ones_like(w)
    beta = 0.0
    moved = 0
    for i in np.lexsort((np.asarray(pos), -kappa)):
        if (moves is None and not kappa[i] > 2.0 * beta) or \
                (moves is not None and moved >= moves):
            break
        lam[i] = r[i]
        beta += w[i] * (1.0 - r[i])
        moved += 1
    return lam, beta, moved


def mse(lam, w, r):
    """MSE of the shrinkage estimator for fixed coefficients (Theorem 1, eq. 6)."""
    lam = np.asarray(lam, dtype=np.float64)
    bias = float(np.sum(w * (1.0 - lam)))
    var = float(np.sum(lam ** 2 * w ** 2 * (1.0 - r) / r))
    return bias * bias + var


def cert_terms(w, r, lam):
    """Per-token pieces of Lemma 1: bias w(1-lambda), variance
    lambda^2 w^2 (1-r)/r and range lambda w max(r, 1-r)/r."""
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    beta_i = w * (1.0 - lam)
    v_i = lam * lam * w * w * (1.0 - r) / r
    b_i = lam * w * np.maximum(r, 1.0 - r) / r
    return beta_i, v_i, b_i


def eps_hat(beta, var, bmax, dnorm, delta):
    """Lemma 1, eq. 7: (beta + b l/3 + sqrt((b l/3)^2 + 2 V l)) / D."""
    l, a = bernstein_consts(delta)
    beta = np.asarray(beta, dtype=np.float64)
    var = np.maximum(np.asarray(var, dtype=np.float64), 0.0)
    bmax = np.asarray(bmax, dtype=np.float64)
    return (beta + a * bmax + np.sqrt((a * bmax) ** 2 + 2.0 * var * l)) / dnorm


def top2(b_i):
    """Largest value, second largest (with multiplicity) and the index of the
    maximum when it is attained by exactly one token (else -1)."""
    if b_i.size == 0:
        return 0.0, 0.0, -1
    i1 = int(np.argmax(b_i))
    b1 = float(b_i[i1])
    if b_i.size == 1:
        return b1, 0.0, i1
    rest = np.delete(b_i, i1)
    b2 = float(rest.max())
    return b1, b2, (i1 if b2 < b1 else -1)


def gains(beta_i, v_i, b_i, dnorm, delta):
    """g_i = eps^(L) - eps^(L \\ {i}) (eq. 9) in rationalised form (R11).

    With s = sqrt((a b)^2 + 2 V l) and s' the same after removing token i
    (b' = b unless i is the unique argmax, then the second largest):
    g_i D = beta_i + a (b - b') + [a^2 (b - b')(b + b') + 2 v_i l] / (s + s').
    """
    l, a = bernstein_consts(delta)
    V = float(np.sum(v_i))
    b1, b2, imax = top2(b_i)
    bp = np.full(b_i.shape, b1, dtype=np.float64)
    if imax >= 0:
        bp[imax] = b2
    s = math.sqrt((a * b1) ** 2 + 2.0 * V * l)
    vp = np.maximum(V - v_i, 0.0)
    sp = np.sqrt((a * bp) ** 2 + 2.0 * vp * l)
    num = a * a * (b1 - bp) * (b1 + bp) + 2.0 * v_i * l
    den = s + sp
    with np.errstate(divide="ignore", invalid="ignore"):
        frac = np.where(den > 0, num / den, 0.0)
    return (beta_i + a * (b1 - bp) + frac) / dnorm


def gains_literal(beta_i, v_i, b_i, dnorm, delta):
    """eq. 9 by recomputing eq. 7 on L \\ {i} for every i (tiny inputs only)."""
    n = beta_i.size
    full = float(eps_hat(beta_i.sum(), v_i.sum(), b_i.max() if n else 0.0,
                         dnorm, delta))
    out = np.empty(n)
    for i in range(n):
        keep = np.ones(n, dtype=bool)
        keep[i] = False
        bm = b_i[keep].max() if n > 1 else 0.0
        out[i] = full - float(eps_hat(beta_i[keep].sum(), v_i[keep].sum(), bm,
                                      dnorm, delta))
    return out


def gain_order(g, pos):
    """L_g: indices into L sorted by gain descending, position ascending (R12)."""
    return np.lexsort((pos, -g))


def suffix_eps(order, beta_i, v_i, b_i, dnorm, delta):
    """eps^(L_g[k:]) for k = 0..|L| from float64 suffix sums/maxima taken
    right to left over the ordered list (eq. 10 with fixed coefficients)."""
    bs = beta_i[order]
    vs = v_i[order]
    bb = b_i[order]
    sb = np.concatenate([np.cumsum(bs[::-1])[::-1], [0.0]])
    sv = np.concatenate([np.cumsum(vs[::-1])[::-1], [0.0]])
    mb = np.concatenate([np.maximum.accumulate(bb[::-1])[::-1], [0.0]]) \
        if bb.size else np.zeros(1)
    return eps_hat(sb, sv, mb, dnorm, delta)


def first_below(e, eps):
    """k* = the first index with e[k] < eps (exists: e[|L|] = 0 < eps)."""
    k = int(np.argmax(e < eps))
    assert e[k] < eps
    return k


def plan_row(wt, r, pos, dnorm, eps, delta, estimator=EST_CLIP,
             binary_moves=None):
    """Plan one decision over L: beta*, lambda, certificate, gains, k*.

    ``wt``: planning weights on L (shifted), ``r``: their inclusion
    probabilities, ``pos``: their positions, ``dnorm``: D~.
    ``binary_moves``: see ``binary_lambdas(moves=...)``.
    """
    wt = np.asarray(wt, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if estimator == EST_CLIP:
        beta_star = shrinkage_beta(wt, r)
        lam = lambdas(wt, r, beta_star)
    elif estimator == EST_BINARY:
        lam, beta_star, _ = binary_lambdas(wt, r, pos, binary_moves)
    else:
        beta_star = 0.0
        lam = np.ones_like(wt)
    beta_i, v_i, b_i = cert_terms(wt, r, lam)
    b1 = float(b_i.max()) if b_i.size else 0.0
    e0 = float(eps_hat(beta_i.sum(), v_i.sum(), b1, dnorm, delta))
    out = dict(beta_star=beta_star, lam=lam, wt=wt, beta_i=beta_i, v_i=v_i,
               b_i=b_i,
               beta_L=float(beta_i.sum()), V_L=float(v_i.sum()), b_L=b1,
               eps_hat0=e0)
    if e0 < eps:
        out.update(k_star=0, eps_hat=e0, order=None, gains=None,
                   fetch_pos=np.zeros(0, dtype=np.int64))
        return out
    g = gains(beta_i, v_i, b_i, dnorm, delta)
    order = gain_order(g, pos)
    e = suffix_eps(order, beta_i, v_i, b_i, dnorm, delta)
    k = first_below(e, eps)
    out.update(k_star=k, eps_hat=float(e[k]), order=order, gains=g,
               suffix=e, fetch_pos=np.asarray(pos)[order[:k]].astype(np.int64))
    return out


def key_logits(qh, keys):
    """Exact logits <q, k_j> / sqrt(d) of the given key rows (§3, eq. 1)."""
    qh = np.asarray(qh, dtype=np.float64)
    return np.asarray(keys, dtype=np.float64) @ qh * (1.0 / math.sqrt(qh.size))


def sketch_logits(qh, sk, proj):
    """Planning logits from the key sketch (Algorithm 2, first step: the
    weights w^ come from the sketch M_A): s_i = <P^T q, sk_i> / sqrt(d).

    ``sk``: [m][s] sketch rows sk_i = P^T k_i (reading R4); ``proj``: P,
    [d][s]. Whenever E[P P^T] = I (Gaussian entries of variance 1/s, or an
    orthogonal P), s_i estimates the exact logit <q, k_i> / sqrt(d) without
    bias; the scale is the attention's 1/sqrt(d), not 1/sqrt(s).
    """
    qh = np.asarray(qh, dtype=np.float64)
    qp = np.asarray(proj, dtype=np.float64).T @ qh
    return np.asarray(sk, dtype=np.float64) @ qp * (1.0 / math.sqrt(qh.size))


def output_coefficients(w_res, r_res, lam_res, exact_res):
    """Coefficients alpha_j of the resident rows in Theorem 2's estimator:
    the exact weight w_j on H and on the fetched part F_h (``exact_res``),
    lambda_j w_j / r_j on the sampled rows S minus F_h (reading R15: those
    rows are resident, so their exact weight is used)."""
    w_res = np.asarray(w_res, dtype=np.float64)
    return np.where(exact_res, w_res, np.asarray(lam_res) * w_res /
                    np.asarray(r_res, dtype=np.float64))


def combine(alpha, v_res, w_f, v_f):
    """The estimate from its parts: D^ = sum alpha_j + sum w_f, the
    numerator N^ = sum alpha_j v_j + sum w_f v_f with the same coefficients
    (reading R16), and o = N^ / D^. Returns (D^, N^, o)."""
    d_hat = float(alpha.sum() + w_f.sum())
    num = alpha @ v_res + w_f @ v_f
    return d_hat, num, num / d_hat


def decode_group(q, res_kv, res_idx, sketch, proj, r, host_kv, eps, delta,
                 estimator=EST_CLIP, weights=W_SKETCH, fetch_override=None,
                 binary_moves=None, sketch2=None, n_short=128,
                 shortlist_override=None):
    """KVFetch for the query heads sharing one KV head.

    q: [grp][d]; res_kv: [count][2][d]; res_idx: [count] ascending positions;
    sketch: [n][s]; proj: [d][s]; r: [n] float32; host_kv: [n][2][d] (full
    cache, only rows outside R and PERFECT planning read it).
    ``fetch_override``: optional list (per head, None = the plan's own) of
    fetch sets F_h to use instead of the planned ones (to evaluate the
    output of another plan); ``binary_moves``: optional list (per head,
    None = the stopping test) of how many tokens binary shrinkage moves.
    With ``weights`` == W_SKETCH2, ``sketch2`` is the 2-bit sketch of this
    KV head (oracle.sketch2.build) and ``n_short`` the shortlist size;
    ``shortlist_override`` replaces the selected shortlist (positions).
    Returns (list of per-head dicts, union of fetched positions).
    """
    q = np.asarray(q, dtype=np.float64)
    grp, d = q.shape
    r = np.asarray(r, dtype=np.float32)
    n = r.size
    in_h = r == np.float32(1.0)
    in_l = ~in_h
    res_idx = np.asarray(res_idx, dtype=np.int64)
    resident = np.zeros(n, dtype=bool)
    resident[res_idx] = True
    if not np.all(resident[in_h]):
        raise ValueError("a token with r == 1 is not resident")
    in_s = in_l & resident
    r64 = r.astype(np.float64)
    kres = np.asarray(res_kv[:, 0, :], dtype=np.float64)
    vres = np.asarray(res_kv[:, 1, :], dtype=np.float64)
    res_h = in_h[res_idx]
    slot = np.full(n, -1, dtype=np.int64)
    slot[res_idx] = np.arange(res_idx.size)
    lpos = np.nonzero(in_l)[0]
    rl = r64[lpos]
    host_kv = None if host_kv is None else np.asarray(host_kv)
    heads = []
    union = set()
    short = np.zeros(0, dtype=np.int64)
    if weights == W_SKETCH2:
        s2 = [sk2.sketch_logits(q[h], sketch2) for h in range(grp)]
        if shortlist_override is not None:
            short = np.sort(np.asarray(shortlist_override, dtype=np.int64))
        else:
            short = sk2.shortlist(np.array(s2).astype(np.float32),
                                  in_l & ~resident, n_short)
    for h in range(grp):
        qh = q[h]
        ell = key_logits(qh, kres)
        if weights == W_SKETCH:
            s_l = sketch_logits(qh, np.asarray(sketch)[lpos], proj)
        elif weights == W_SKETCH2:
            # exact logits on S and on the shortlist, the sketch's elsewhere
            s_all = s2[h].copy()
            s_all[res_idx] = ell
            if short.size:
                s_all[short] = key_logits(qh, host_kv[short, 0, :])
            s_l = s_all[lpos]
        else:
            s_l = key_logits(qh, host_kv[lpos, 0, :])
        m = max(ell.max() if ell.size else -np.inf,
                s_l.max() if s_l.size else -np.inf)
        w_res = np.exp(ell - m)
        wt = np.exp(s_l - m)
        dnorm = float(np.sum(w_res[res_h]) + np.sum(wt))
        plan = plan_row(wt, rl, lpos, dnorm, eps, delta, estimator,
                        None if binary_moves is None else binary_moves[h])
        fpos = plan["fetch_pos"] \
            if fetch_override is None or fetch_override[h] is None \
            else np.asarray(fetch_override[h], dtype=np.int64)
        in_f = np.zeros(n, dtype=bool)
        in_f[fpos] = True
        # coefficients on resident rows
        lam_full = np.ones(n)
        lam_full[lpos] = plan["lam"]
        alpha = output_coefficients(w_res, r64[res_idx], lam_full[res_idx],
                                    res_h | in_f[res_idx])
        # exact contributions of fetched rows outside S
        fetch_rows = np.array(sorted(set(fpos.tolist()) - set(res_idx.tolist())),
                              dtype=np.int64)
        if fetch_rows.size:
            kf = np.asarray(host_kv[fetch_rows, 0, :], dtype=np.float64)
            vf = np.asarray(host_kv[fetch_rows, 1, :], dtype=np.float64)
            wf = np.exp(key_logits(qh, kf) - m)
        else:
            vf = np.zeros((0, d))
            wf = np.zeros(0)
        union.update(fetch_rows.tolist())
        d_hat, _, o = combine(alpha, vres, wf, vf)
        plan.update(m=m, dnorm=dnorm, d_hat=d_hat, o=o, fetch_rows=fetch_rows,
                    lpos=lpos, n_s=int(in_s.sum()), shortlist=short)
        heads.append(plan)
    return heads, np.array(sorted(union), dtype=np.int64)


def decode_step(q, res_kv, res_idx, sketch, proj, r, host_kv, eps, delta,
                estimator=EST_CLIP, weights=W_SKETCH, sketch2=None, n_short=128):
    """All requests and KV heads of one layer.

    q: [B][Hq][d]; res_kv[b][g]: [count][2][d]; res_idx[b][g]: [count];
    sketch: [B][G][n][s]; proj: [G][d][s]; r: [B][G][n]; host_kv:
    [B][G][n][2][d]; sketch2[b][g]: 2-bit sketches (W_SKETCH2 only).
    Returns (heads[b][h] dicts, unions[b][g]).
    """
    B, Hq, _ = q.shape
    G = r.shape[1]
    grp = Hq // G
    heads = [[None] * Hq for _ in range(B)]
    unions = [[None] * G for _ in range(B)]
    for b in range(B):
        for g in range(G):
            hs, un = decode_group(q[b, g * grp:(g + 1) * grp], res_kv[b][g],
                                  res_idx[b][g],
                                  None if sketch is None else sketch[b, g],
                                  None if proj is None else proj[g],
                                  r[b, g], host_kv[b, g], eps, delta,
                                  estimator, weights,
                                  sketch2=None if sketch2 is None else sketch2[b][g],
                                  n_short=n_short)
            for j, hd in enumerate(hs):
                heads[b][g * grp + j] = hd
            unions[b][g] = un
    return heads, unions


def dense_step(q, kv):
    """The Dense baselines of section 5: exact attention (eq. 1) of every
    query head over every token of its KV head. q [B][Hq][d], kv
    [B][G][n][2][d]; returns (o [B][Hq][d], log D [B][Hq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    G = kv.shape[1]
    grp = Hq // G
    o = np.zeros((B, Hq, d))
    logd = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            o[b, h], logd[b, h] = exact_attention(q[b, h], kv[b, g, :, 0, :],
                                                  kv[b, g, :, 1, :])
    return o, logd


def exact_attention(q, k, v):
    """Textbook softmax attention o = sum w v / sum w, w = exp(<k,q>/sqrt(d))
    (§3, eq. 1), float64; returns (o, log D)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lg = k @ q / math.sqrt(q.size)
    m = lg.max()
    w = np.exp(lg - m)
    return (w @ v) / w.sum(), math.log(w.sum()) + m
