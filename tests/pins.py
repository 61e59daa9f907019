"""Pin checks for the oracle: each function raises AssertionError when the
oracle disagrees with something fixed independently of it (a brute force, a
closed form from the proofs, a library routine, an exact enumeration).

They are plain functions so that ``test_oracle_mutations.py`` can plant a
plausible mistake in the oracle and confirm that some pin fails.
"""

import itertools
import math
from fractions import Fraction

import mpmath
import numpy as np
from scipy.optimize import brentq, minimize

from oracle import compress as oc
from oracle import decode as od
from oracle import sketch2 as sk2

mpmath.mp.dps = 50


# ---------------------------------------------------------------- PoissonComp
def check_water_level_bruteforce(tq, b_free):
    """Every j in 0..|U| is tried in exact rationals; the valid one (the top j
    saturate, the rest do not, and the rates sum to the budget) must give the
    oracle's c."""
    tq = [int(x) for x in tq]
    j_star, num, den = oc.water_level(np.array(tq, dtype=np.int64), b_free)
    if den == 0:
        assert b_free >= len(tq)
        return
    c_or = Fraction(num, den)
    srt = sorted(tq, reverse=True)
    valid = []
    for j in range(len(srt)):
        # candidate: the top j saturate, the others get c * tau
        c = Fraction(b_free - j, sum(srt[j:]))
        if c < 0:
            continue
        total = sum(min(Fraction(1), c * t) for t in srt)
        if total == b_free:
            valid.append(c)
    assert valid, "brute force found no water level"
    assert all(v == valid[0] for v in valid)
    assert c_or == valid[0], (c_or, valid[0])
    # the exact rates sum to the budget
    total = sum(min(Fraction(1), c_or * t) for t in tq)
    assert total == b_free


def check_water_level_brentq(tau, budget, n_sink, n_local):
    """scipy brentq on sum_U min(1, c tau) - B_U must find the oracle's c."""
    sl = oc.compress_slice(tau, budget, n_sink, n_local, 0, 0, 0)
    tq = sl["tq"][~sl["forced"]].astype(np.float64)
    b_free = budget - int(sl["forced"].sum())
    if sl["den"] == 0:
        return
    f = lambda c: np.minimum(1.0, c * tq).sum() - b_free  # noqa: E731
    c_ref = brentq(f, 0.0, 1.0, xtol=1e-300, rtol=1e-15, maxiter=500)
    c_or = sl["num"] / sl["den"]
    assert abs(c_or - c_ref) <= 1e-12 * c_ref, (c_or, c_ref)


def check_rates_sum(tau, budget, n_sink, n_local):
    """sum_i r_i = budget: exactly in rationals, and to 1e-6 in float."""
    sl = oc.compress_slice(tau, budget, n_sink, n_local, 0, 0, 0)
    r = sl["r"].astype(np.float64)
    assert abs(r.sum() - budget) <= 1e-6 * budget, (r.sum(), budget)
    if sl["den"]:
        in_h = sl["in_h"]
        exact = int(in_h.sum()) * sl["den"] + \
            int(sl["tq"][~in_h].sum()) * sl["num"]
        assert exact == budget * sl["den"]
    # monotone in tau among the free tokens; H/L partition
    free = ~sl["forced"]
    o = np.argsort(sl["tq"][free], kind="stable")
    assert np.all(np.diff(sl["r"][free][o]) >= 0)
    assert np.all(sl["in_h"] ^ sl["in_l"])
    assert np.all(sl["r"][sl["in_l"]] < 1.0) and np.all(sl["r"] > 0)
    assert np.all(sl["in_h"][sl["forced"]])


# ---------------------------------------------------------------- shrinkage
def check_shrinkage_lbfgsb(w, r):
    """Theorem 1: the Definition 2 coefficients minimise eq. 6 over the box
    [r_i, 1]; scipy's L-BFGS-B from several starts must agree."""
    beta = od.shrinkage_beta(w, r)
    lam = od.lambdas(w, r, beta)
    f = lambda x: od_mse_plain(x, w, r)  # noqa: E731

    def grad(x):
        bias = np.sum(w * (1 - x))
        return -2 * w * bias + 2 * w * w * x * (1 - r) / r

    best = None
    for x0 in (r.copy(), np.ones_like(r), 0.5 * (r + 1)):
        res = minimize(f, x0, jac=grad, method="L-BFGS-B",
                       bounds=list(zip(r, np.ones_like(r))),
                       options=dict(ftol=1e-15, gtol=1e-13, maxiter=10000))
        if best is None or res.fun < best.fun:
            best = res
    assert np.max(np.abs(best.x - lam)) <= 1e-6, (best.x, lam)
    # and the fixed point: beta = sum w (1 - lambda)
    assert abs(np.sum(w * (1 - lam)) - beta) <= 1e-12 * max(beta, 1e-300)


def od_mse_plain(lam, w, r):
    """eq. 6 written out independently of the oracle's own mse()."""
    bias = 0.0
    var = 0.0
    for li, wi, ri in zip(lam, w, r):
        bias += wi - li * wi
        var += li * li * wi * wi * (1 - ri) / ri
    return bias * bias + var


def check_kkt(w, r):
    """First-order conditions of eq. 6 on the box (proof of Theorem 1):
    df/dlambda_i = -2 w_i beta + 2 w_i^2 lambda_i (1 - r_i)/r_i is >= 0 at the
    lower bound, 0 inside and <= 0 at the upper bound."""
    beta = od.shrinkage_beta(w, r)
    lam = od.lambdas(w, r, beta)
    assert np.all(lam >= r * (1 - 1e-15)) and np.all(lam <= 1.0)
    bias = np.sum(w * (1 - lam))
    gr = -2 * w * bias + 2 * w * w * lam * (1 - r) / r
    tol = 1e-9 * np.max(np.abs(2 * w * bias)) + 1e-300
    at_lo = np.isclose(lam, r, rtol=0, atol=1e-14)
    at_hi = np.isclose(lam, 1.0, rtol=0, atol=1e-14)
    inner = ~(at_lo | at_hi)
    assert np.all(gr[at_lo & ~at_hi] >= -tol)
    assert np.all(gr[at_hi & ~at_lo] <= tol)
    assert np.all(np.abs(gr[inner]) <= tol)
    # better than both endpoints of the box (Figure 2's shape)
    m = od_mse_plain(lam, w, r)
    assert m <= od_mse_plain(np.ones_like(r), w, r) * (1 + 1e-12)
    assert m <= od_mse_plain(r, w, r) * (1 + 1e-12)


def check_binary_prefix(w, r, pos=None):
    """Binary shrinkage (Appendix A.2, Figure 2), in exact rationals: the
    moved tokens (lambda = r) are a prefix of the order by w (1 - r) / r
    descending (positions ascending on ties); that prefix is the first
    minimum of the MSE (eq. 6) over every prefix of the order; each move
    changes the MSE by a_i (2 beta - w_i (1 - r_i) / r_i) with a_i =
    w_i (1 - r_i) and beta the bias before it; and the result lies between
    the clipped minimiser of Theorem 1 and the two endpoints lambda = 1 and
    lambda = r."""
    n = len(w)
    pos = np.arange(n) if pos is None else np.asarray(pos)
    lam, beta, moved = od.binary_lambdas(w, r, pos)
    W = [Fraction(float(x)) for x in w]
    R = [Fraction(float(x)) for x in r]
    kap = [W[i] * (1 - R[i]) / R[i] for i in range(n)]
    order = sorted(range(n), key=lambda i: (-kap[i], int(pos[i])))

    def mse_of(k):
        S = set(order[:k])
        bias = sum((W[i] * (1 - R[i]) for i in S), Fraction(0))
        var = sum(((R[i] if i in S else 1) ** 2 * W[i] ** 2 * (1 - R[i]) / R[i]
                   for i in range(n)), Fraction(0))
        return bias * bias + var

    curve = [mse_of(k) for k in range(n + 1)]
    best = min(curve)
    assert moved == curve.index(best), (moved, curve.index(best))
    assert sorted(np.nonzero(lam != 1.0)[0].tolist()) == sorted(order[:moved])
    assert np.all(lam[order[:moved]] == np.asarray(r, np.float64)[order[:moved]])
    bias = Fraction(0)
    for k, i in enumerate(order):
        a = W[i] * (1 - R[i])
        assert curve[k + 1] - curve[k] == a * (2 * bias - kap[i])
        bias += a
    assert abs(beta - float(sum((W[i] * (1 - R[i]) for i in order[:moved]),
                                Fraction(0)))) <= 1e-12 * max(beta, 1e-300)
    m_bin = od_mse_plain(lam, w, r)
    assert m_bin <= od_mse_plain(np.ones(n), w, r) * (1 + 1e-12)
    assert m_bin <= od_mse_plain(np.asarray(r, np.float64), w, r) * (1 + 1e-12)
    lam_c = od.lambdas(w, r, od.shrinkage_beta(w, r))
    assert od_mse_plain(lam_c, w, r) <= m_bin * (1 + 1e-12)


def check_exact_attention_mp(q, k, v):
    """eq. 1 term by term at 50 digits: w_i = exp(<q, k_i>/sqrt(d)),
    o = sum w_i v_i / sum w_i, log D = log sum w_i."""
    o, logd = od.exact_attention(q, k, v)
    d = len(q)
    sd = mpmath.sqrt(d)
    ws = [mpmath.exp(mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                 for a, b in zip(q, ki)) / sd) for ki in k]
    D = mpmath.fsum(ws)
    assert abs(logd - float(mpmath.log(D))) <= 1e-12 * max(1.0, abs(logd))
    for c in range(v.shape[1]):
        oc = mpmath.fsum(wi * mpmath.mpf(float(vi[c])) for wi, vi in zip(ws, v)) / D
        assert abs(o[c] - float(oc)) <= 1e-12 * (1 + abs(float(oc)))


# ---------------------------------------------------------------- certificate
def check_bernstein_root(V, b, delta):
    """Lemma 1's proof: t = D * (eps^ - beta/D) is the positive root of
    t^2 = 2 l (V + b t / 3), and Bernstein's two-sided tail
    2 exp(-t^2 / (2V + 2bt/3)) equals delta there."""
    D = 3.0
    e = float(od.eps_hat(0.0, V, b, D, delta))
    t = mpmath.mpf(e) * D
    l = mpmath.log(mpmath.mpf(2) / mpmath.mpf(delta))
    lhs = t * t
    rhs = 2 * l * (mpmath.mpf(V) + mpmath.mpf(b) * t / 3)
    assert abs(lhs - rhs) <= 1e-12 * abs(rhs), (lhs, rhs)
    tail = 2 * mpmath.exp(-t * t / (2 * mpmath.mpf(V) + 2 * mpmath.mpf(b) * t / 3))
    assert abs(tail - delta) <= 1e-10 * delta, (tail, delta)
    # and with a bias: eps^ D = beta + t
    e2 = float(od.eps_hat(0.7, V, b, D, delta))
    assert abs(e2 * D - 0.7 - float(t)) <= 1e-12 * (float(t) + 0.7)


def enumerate_estimator(wH, w, r, lam):
    """All 2^|L| outcomes of the Poisson sample: returns (values, probs)."""
    nl = len(w)
    vals = []
    probs = []
    for z in itertools.product((0, 1), repeat=nl):
        z = np.array(z)
        vals.append(np.sum(wH) + np.sum(z * lam * w / r))
        probs.append(np.prod(np.where(z == 1, r, 1 - r)))
    return np.array(vals), np.array(probs)


def check_enumeration(wH, w, r, delta, estimator=od.EST_CLIP):
    """Exact enumeration with exact weights (the perfect sketch): the bias is
    -beta(L), the variance V(L) (proof of Theorem 1), and
    Pr(|D^ - D|/D > eps^(L)) <= delta (Lemma 1)."""
    D = float(np.sum(wH) + np.sum(w))
    pos = np.arange(len(w))
    plan = od.plan_row(w, r, pos, D, 1e9, delta, estimator)
    vals, probs = enumerate_estimator(wH, w, r, plan["lam"])
    mean = float(np.sum(vals * probs))
    var = float(np.sum((vals - mean) ** 2 * probs))
    beta_l = float(np.sum(w * (1 - plan["lam"])))
    assert abs((mean - D) + beta_l) <= 1e-10 * D, (mean - D, -beta_l)
    assert abs(var - plan["V_L"]) <= 1e-9 * max(var, 1e-300), (var, plan["V_L"])
    assert abs(plan["beta_L"] - beta_l) <= 1e-12 * D
    fail = float(np.sum(probs[np.abs(vals - D) / D > plan["eps_hat0"]]))
    assert fail <= delta, (fail, delta)
    if estimator == od.EST_UNBIASED:
        assert abs(mean - D) <= 1e-12 * D


# ---------------------------------------------------------------- gains / k*
def mp_eps(beta_i, v_i, b_i, keep, D, delta):
    l = mpmath.log(mpmath.mpf(2) / mpmath.mpf(delta))
    a = l / 3
    be = mpmath.fsum(mpmath.mpf(x) for x, k in zip(beta_i, keep) if k)
    V = mpmath.fsum(mpmath.mpf(x) for x, k in zip(v_i, keep) if k)
    bs = [mpmath.mpf(x) for x, k in zip(b_i, keep) if k]
    b = max(bs) if bs else mpmath.mpf(0)
    return (be + a * b + mpmath.sqrt((a * b) ** 2 + 2 * V * l)) / mpmath.mpf(D)


def check_gains_loo(beta_i, v_i, b_i, D, delta):
    """eq. 9 by brute force: recompute eps^(L \\ {i}) from scratch at 50
    digits for every i and compare with the closed form (R11)."""
    n = len(beta_i)
    g = od.gains(beta_i, v_i, b_i, D, delta)
    full = mp_eps(beta_i, v_i, b_i, [True] * n, D, delta)
    for i in range(n):
        keep = [True] * n
        keep[i] = False
        ref = full - mp_eps(beta_i, v_i, b_i, keep, D, delta)
        assert abs(mpmath.mpf(g[i]) - ref) <= 1e-11 * abs(full) + 1e-300, \
            (i, g[i], ref)
        assert g[i] >= 0.0


def check_kstar_bruteforce(w, r, D, eps, delta):
    """eq. 10 by brute force: recompute eps^(L_g[k:]) from scratch for every
    k at 50 digits; it must be non-increasing and give the oracle's k*."""
    n = len(w)
    pos = np.arange(n)
    plan = od.plan_row(w, r, pos, D, eps, delta)
    if plan["order"] is None:
        assert plan["eps_hat0"] < eps
        return plan
    order = plan["order"]
    # order must sort the closed-form gains descending, ties by position
    g = plan["gains"]
    for a_, b_ in zip(order[:-1], order[1:]):
        assert g[a_] > g[b_] or (g[a_] == g[b_] and pos[a_] < pos[b_])
    prev = None
    k_ref = None
    for k in range(n + 1):
        keep = [False] * n
        for idx in order[k:]:
            keep[idx] = True
        e = mp_eps(plan["beta_i"], plan["v_i"], plan["b_i"], keep, D, delta)
        if prev is not None:
            assert e <= prev * (1 + mpmath.mpf("1e-14")) + mpmath.mpf("1e-300")
        prev = e
        if k_ref is None and e < eps:
            k_ref = k
        assert abs(mpmath.mpf(plan["suffix"][k]) - e) <= 1e-12 * abs(e) + 1e-300
    assert plan["k_star"] == k_ref, (plan["k_star"], k_ref)
    return plan


def check_range_bound(w, r):
    """Lemma 1's proof bounds each centred term X_i = lambda_i w_i (Z_i - r_i)
    / r_i by b_i; the bound is attained by one of the two outcomes."""
    beta = od.shrinkage_beta(w, r)
    lam = od.lambdas(w, r, beta)
    _, _, b_i = od.cert_terms(w, r, lam)
    x1 = np.abs(lam * w * (1 - r) / r)
    x0 = np.abs(lam * w * (0 - r) / r)
    top = np.maximum(x0, x1)
    assert np.allclose(top, b_i, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- sketch logits
def _exact_logit_mp(q, k):
    """<q, k> / sqrt(d) at 50 digits (the logit of eq. 1)."""
    d = len(q)
    return mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                       for a, b in zip(q, k)) / mpmath.sqrt(d)


def check_sketch_orthogonal(seed, d=16, m=12):
    """An orthogonal projection (s = d) preserves inner products,
    <P^T q, P^T k> = <q, k>, so the planning logits of a sketch sk = P^T k
    must equal the exact logits <q, k> / sqrt(d). P is a random orthogonal
    matrix (not symmetric), so using P q instead of P^T q fails."""
    rng = np.random.default_rng(seed)
    P, _ = np.linalg.qr(rng.standard_normal((d, d)))
    assert np.max(np.abs(P - P.T)) > 0.1
    q = rng.standard_normal(d)
    K = 2.0 * rng.standard_normal((m, d))
    s = od.sketch_logits(q, K @ P, P)
    for i in range(m):
        ref = float(_exact_logit_mp(q, K[i]))
        tol = 1e-12 * np.linalg.norm(q) * np.linalg.norm(K[i]) / math.sqrt(d)
        assert abs(s[i] - ref) <= tol, (i, s[i], ref)


def check_sketch_blocks(seed, d=16, s=4, m=12):
    """E[P P^T] = I makes the sketch logit an unbiased estimate of the exact
    one (reading R4). A uniform draw among the d/s signed coordinate blocks
    P_j = sqrt(d/s) E_j (E_j: s distinct coordinates, random signs) has
    E[P_j P_j^T] = I exactly, so the mean of the sketch logits over the d/s
    blocks must equal <q, k> / sqrt(d) (a scale of 1/sqrt(s) is off by
    sqrt(d/s))."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(d)
    sgn = rng.choice([-1.0, 1.0], d)
    q = rng.standard_normal(d)
    K = 2.0 * rng.standard_normal((m, d))
    acc = np.zeros(m)
    for j in range(d // s):
        P = np.zeros((d, s))
        for t in range(s):
            c = perm[j * s + t]
            P[c, t] = sgn[c] * math.sqrt(d / s)
        acc += od.sketch_logits(q, K @ P, P)
    acc /= d // s
    for i in range(m):
        ref = float(_exact_logit_mp(q, K[i]))
        tol = 1e-12 * np.linalg.norm(q) * np.linalg.norm(K[i])
        assert abs(acc[i] - ref) <= tol, (i, acc[i], ref)


def tiny_layer(seed, d=8, n_h=3, n_l=8, grp=1, s=4):
    """A small KV head for the estimator pins: n_h tokens with r = 1 and n_l
    tokens of L with r in (0.15, 0.85), spread logits, a Gaussian sketch
    (entries of variance 1/s). Returns a dict of float64/float32 arrays."""
    rng = np.random.default_rng(seed)
    n = n_h + n_l
    pos = rng.permutation(n)
    h_pos = np.sort(pos[:n_h])
    l_pos = np.sort(pos[n_h:])
    K = 1.5 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    r = np.ones(n, dtype=np.float32)
    r[l_pos] = rng.uniform(0.15, 0.85, n_l).astype(np.float32)
    P = rng.standard_normal((d, s)) / math.sqrt(s)
    return dict(q=rng.standard_normal((grp, d)), K=K, V=V, r=r, P=P,
                sketch=K @ P, host_kv=np.stack([K, V], axis=1),
                h_pos=h_pos, l_pos=l_pos, n=n, d=d)


def check_sketch_decode_identity(seed):
    """With P = I (s = d) the sketch is the keys themselves, so every output
    of the decode step (plan, fetch set, estimate) in sketch mode must equal
    the exact-weight (perfect sketch) mode bit for bit: the sketch rows are
    looked up at the positions of L and scaled like the exact logits."""
    t = tiny_layer(seed, d=8, n_h=4, n_l=24, grp=2)
    rng = np.random.default_rng(seed + 1)
    samp = t["l_pos"][rng.random(t["l_pos"].size) < t["r"][t["l_pos"]]]
    res_idx = np.sort(np.concatenate([t["h_pos"], samp]))
    res_kv = t["host_kv"][res_idx]
    eye = np.eye(t["d"])
    outs = []
    for wm in (od.W_SKETCH, od.W_PERFECT):
        heads, union = od.decode_group(t["q"], res_kv, res_idx, t["K"].copy(),
                                       eye, t["r"], t["host_kv"], 0.02, 0.1,
                                       od.EST_CLIP, wm)
        outs.append((heads, union))
    (ha, ua), (hb, ub) = outs
    assert np.array_equal(ua, ub)
    for a, b in zip(ha, hb):
        for k in ("m", "dnorm", "beta_star", "eps_hat0", "k_star", "eps_hat",
                  "d_hat"):
            assert a[k] == b[k], (k, a[k], b[k])
        assert np.array_equal(a["fetch_pos"], b["fetch_pos"])
        assert np.array_equal(a["o"], b["o"])
    assert any(h["k_star"] > 0 for h in ha)


# ---------------------------------------------------------------- estimator
def check_estimator_enumeration(seed, estimator, weights, n_l=8, n_fetch=2):
    """Theorem 2's estimator, through the decode step itself, over all 2^|L|
    Poisson samples: with a fixed fetch set F (so S minus F is not empty),
    coefficients w on H u F and lambda w / r on S minus F, the expectations
    of the denominator and the numerator are
        E[D^] = D - sum_{L'} w_i (1 - lambda_i),
        E[N^] = N - sum_{L'} w_i (1 - lambda_i) v_i,   L' = L minus F,
    with D = sum_i w_i and N = sum_i w_i v_i over every token (exact weights
    w_i = exp(<q, k_i>/sqrt(d)), eq. 1); with lambda = 1 both are unbiased.
    Each sample's estimate is taken as D^ = d_hat e^m and N^ = D^ o."""
    t = tiny_layer(seed, n_l=n_l)
    l_pos, h_pos = t["l_pos"], t["h_pos"]
    # fetch the lightest tokens of L, so that the heavy (shrunk) ones stay
    # in L' = L minus F
    lw = t["K"][l_pos] @ t["q"][0]
    F = np.sort(l_pos[np.argsort(lw)[:n_fetch]])
    rl = t["r"][l_pos].astype(np.float64)
    ED = mpmath.mpf(0)
    EN = [mpmath.mpf(0)] * t["d"]
    lam0 = None
    for z in itertools.product((0, 1), repeat=n_l):
        z = np.array(z, dtype=bool)
        res_idx = np.sort(np.concatenate([h_pos, l_pos[z]]))
        heads, _ = od.decode_group(t["q"], t["host_kv"][res_idx], res_idx,
                                   t["sketch"], t["P"], t["r"], t["host_kv"],
                                   0.1, 0.1, estimator, weights,
                                   fetch_override=[F])
        hd = heads[0]
        assert np.array_equal(hd["lpos"], l_pos)
        if lam0 is None:
            lam0 = hd["lam"].copy()
        # lambda is fixed before the sample is seen (up to rounding of the
        # shift, which scales every planning weight alike)
        assert np.allclose(hd["lam"], lam0, rtol=1e-12, atol=0)
        prob = mpmath.mpf(float(np.prod(np.where(z, rl, 1.0 - rl))))
        dh = mpmath.mpf(hd["d_hat"]) * mpmath.exp(mpmath.mpf(hd["m"]))
        ED += prob * dh
        for c in range(t["d"]):
            EN[c] += prob * dh * mpmath.mpf(float(hd["o"][c]))
    q = t["q"][0]
    w = [mpmath.exp(_exact_logit_mp(q, t["K"][i])) for i in range(t["n"])]
    lam = np.ones(t["n"])
    lam[l_pos] = lam0
    rest = set(l_pos.tolist()) - set(F.tolist())
    D = mpmath.fsum(w)
    bias = mpmath.fsum(w[i] * (1 - mpmath.mpf(float(lam[i]))) for i in rest)
    assert abs(ED - (D - bias)) <= mpmath.mpf("1e-11") * D, (ED, D - bias)
    scale = mpmath.fsum(w[i] * mpmath.fsum(abs(mpmath.mpf(float(x)))
                                           for x in t["V"][i])
                        for i in range(t["n"]))
    for c in range(t["d"]):
        N = mpmath.fsum(w[i] * mpmath.mpf(float(t["V"][i, c]))
                        for i in range(t["n"]))
        bn = mpmath.fsum(w[i] * (1 - mpmath.mpf(float(lam[i]))) *
                         mpmath.mpf(float(t["V"][i, c])) for i in rest)
        assert abs(EN[c] - (N - bn)) <= mpmath.mpf("1e-11") * scale, \
            (c, EN[c], N - bn)
    if estimator == od.EST_UNBIASED:
        assert np.all(lam0 == 1.0)
    else:
        # the case is not degenerate: some coefficient on L' is shrunk
        assert max(1.0 - lam[i] for i in rest) > 1e-3


# ---------------------------------------------------------------- Philox
def check_philox_kat():
    """The published known-answer vectors of Philox4x32-10 (Salmon et al.,
    SC'11), stored in tests/golden/philox_kat.json."""
    import json
    import os
    from oracle import philox
    path = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ctr = [int(x, 16) for x in c["ctr"]]
        key = [int(x, 16) for x in c["key"]]
        out = philox.philox4x32_10(*ctr, *key)
        assert [int(x) for x in out] == [int(x, 16) for x in c["out"]], c


# ---------------------------------------------------------------- 2-bit sketch
# "Verify Before You Fetch", Appendix A.1 (Key Sketch) and section 5.1.

def _levels_keys(seed, n=300, d=128, planted=None):
    """Keys whose planted pairs (j, j + d/2) take, per 128-token group and
    channel, exactly the four levels z + k s (k = 0..3, each present), with z
    and s exact in fp16; every other channel is small noise. Returns
    (keys float32 [n][d], planted pairs, z [ngroups][d], s [ngroups][d],
    level index [n][d])."""
    rng = np.random.default_rng(seed)
    if planted is None:
        planted = np.sort(rng.choice(d // 2, sk2.N_PAIRS, replace=False))
    chan = sk2.kept_channels(planted, d)
    keys = (0.05 * rng.standard_normal((n, d))).astype(np.float32)
    ng = (n + sk2.GROUP - 1) // sk2.GROUP
    z = np.zeros((ng, d), dtype=np.float32)
    s = np.zeros((ng, d), dtype=np.float32)
    lev = np.zeros((n, d), dtype=np.int64)
    for gi in range(ng):
        lo, hi = gi * sk2.GROUP, min(n, (gi + 1) * sk2.GROUP)
        m = hi - lo
        for c in chan:
            zz = -float(rng.integers(8, 64)) / 8.0       # exact in fp16
            ss = float(rng.integers(16, 64)) / 16.0      # exact in fp16
            k = rng.integers(0, 4, m)
            k[:4] = rng.permutation(4)                   # every level present
            keys[lo:hi, c] = zz + k * ss
            z[gi, c], s[gi, c] = zz, ss
            lev[lo:hi, c] = k
    return keys, np.asarray(planted), z, s, lev


def check_sketch2_levels(seed, n=300):
    """Quantisation closed form: a channel that holds exactly four equally
    spaced levels between its group minimum and maximum is stored without
    loss. The zero point is the minimum, the scale a third of the range, the
    code the level index, and dequantisation returns every key bit for bit.
    The pairs of largest energy are the planted ones."""
    keys, planted, z, s, lev = _levels_keys(seed, n)
    sk = sk2.build(keys)
    assert np.array_equal(sk["pairs"], planted), (sk["pairs"], planted)
    chan = sk["chan"]
    assert np.array_equal(chan, np.sort(np.concatenate([planted, planted + 64])))
    assert np.array_equal(sk["zero"], z[:, chan])
    assert np.array_equal(sk["scale"], s[:, chan])
    assert np.array_equal(sk["codes"], lev[:, chan])
    assert np.array_equal(sk2.dequantize(sk), keys[:, chan])


def check_sketch2_error(seed, n=700, d=128):
    """Uniform 2-bit quantisation between the group's minimum and maximum:
    codes in 0..3, and every dequantised key within half a step (plus the
    fp16 rounding of zero and scale) of the key."""
    rng = np.random.default_rng(seed)
    keys = (rng.standard_normal((n, d)) * rng.uniform(0.2, 4.0, d)).astype(np.float32)
    sk = sk2.build(keys)
    chan = sk["chan"]
    assert sk["codes"].max() <= 3
    kh = sk2.dequantize(sk)
    for gi in range(sk["zero"].shape[0]):
        lo, hi = gi * sk2.GROUP, min(n, (gi + 1) * sk2.GROUP)
        v = keys[lo:hi][:, chan].astype(np.float64)
        step = (v.max(axis=0) - v.min(axis=0)) / 3.0
        slack = 2.0 ** -10 * (np.abs(v).max(axis=0) + step) * 4
        err = np.abs(kh[lo:hi].astype(np.float64) - v)
        assert np.all(err <= step / 2 + slack), float((err - step / 2 - slack).max())
        # the codes of each group's extremes
        assert np.all(sk["codes"][lo:hi][v.argmin(axis=0), np.arange(chan.size)] == 0)
        assert np.all(sk["codes"][lo:hi][v.argmax(axis=0), np.arange(chan.size)] == 3)


def check_sketch2_rotation(seed, n=400, d=128):
    """RoPE rotates the two channels of a pair together, so a pair's energy,
    and with it the choice of pairs, does not change when every token's key
    is rotated within each pair (j, j + d/2) by any angle. The pairs chosen
    are the planted high-energy ones."""
    rng = np.random.default_rng(seed)
    planted = np.sort(rng.choice(d // 2, sk2.N_PAIRS, replace=False))
    amp = np.ones(d // 2)
    amp[planted] = 3.0
    keys = rng.standard_normal((n, d))
    keys[:, :d // 2] *= amp
    keys[:, d // 2:] *= amp
    ang = rng.uniform(0, 2 * np.pi, (n, d // 2))
    a, b = keys[:, :d // 2], keys[:, d // 2:]
    rot = np.concatenate([a * np.cos(ang) - b * np.sin(ang),
                          a * np.sin(ang) + b * np.cos(ang)], axis=1)
    e0 = sk2.pair_energy(keys.astype(np.float32))
    e1 = sk2.pair_energy(rot.astype(np.float32))
    assert np.allclose(e0, e1, rtol=1e-5)
    assert np.array_equal(sk2.build(keys.astype(np.float32))["pairs"], planted)
    assert np.array_equal(sk2.build(rot.astype(np.float32))["pairs"], planted)


def check_sketch2_cost():
    """The pages' cost figure: the sketch holds 1.76% of the full bf16 K/V
    cache (2 bits for a quarter of the key channels, with an fp16 zero point
    and scale per channel and 128-token group)."""
    rng = np.random.default_rng(0)
    for n in (32768, 131072):
        d = 128
        keys = np.zeros((n, d), dtype=np.float32)
        keys[:, :] = rng.standard_normal(d).astype(np.float32)  # cheap content
        sk = sk2.build(keys[:sk2.GROUP * 2])
        # scale the stored sizes of a two-group build to n tokens
        per_token = sk["codes"].shape[1] * 2 / 8
        per_group = (sk["zero"].shape[1] + sk["scale"].shape[1]) * 2
        total = n * per_token + (n // sk2.GROUP) * per_group
        assert sk2.storage_bytes(sk) == 2 * sk2.GROUP * per_token + 2 * per_group
        assert sk["codes"].shape[1] == d // 4
        assert round(100.0 * total / (n * 2 * d * 2), 2) == 1.76


def check_sketch2_logit_identity(seed, n=300, d=128):
    """With keys the sketch stores without loss (four levels per group and
    kept channel) and a query that is zero outside the kept channels, the
    sketch logit is the exact logit <q, k> / sqrt(d) of every token."""
    keys, planted, _, _, _ = _levels_keys(seed, n)
    sk = sk2.build(keys)
    rng = np.random.default_rng(seed + 7)
    q = np.zeros(d)
    q[sk["chan"]] = rng.standard_normal(sk["chan"].size)
    s = sk2.sketch_logits(q, sk)
    exact = keys.astype(np.float64) @ q / math.sqrt(d)
    assert np.allclose(s, exact, rtol=1e-12, atol=1e-12)
    # and a query on the other channels adds nothing
    q2 = rng.standard_normal(d)
    q2[sk["chan"]] = 0.0
    assert np.all(sk2.sketch_logits(q2, sk) == 0.0)


def check_shortlist_bruteforce(seed, n=500, grp=4):
    """Shortlist against a plain sort of (largest score over the heads
    descending, position ascending) over the eligible tokens, with planted
    equal scores."""
    rng = np.random.default_rng(seed)
    sc = rng.standard_normal((grp, n)).astype(np.float32)
    sc[:, 50:60] = sc[0, 40]          # ties across positions
    elig = rng.random(n) < 0.7
    for ns in (0, 1, 7, 128, int(elig.sum()), int(elig.sum()) + 5):
        got = sk2.shortlist(sc, elig, ns)
        cand = [(-max(float(sc[h, i]) for h in range(grp)), i)
                for i in range(n) if elig[i]]
        cand.sort()
        want = sorted(i for _, i in cand[:max(ns, 0)])
        assert list(got) == want, ns


def check_sketch2_full_shortlist(seed):
    """A shortlist that covers every non-resident token of L makes every
    planning weight exact, so the plan, fetch set and estimate equal the
    perfect-sketch mode's."""
    t = tiny_layer(seed, d=128, n_h=6, n_l=120, grp=2)
    rng = np.random.default_rng(seed + 1)
    samp = t["l_pos"][rng.random(t["l_pos"].size) < t["r"][t["l_pos"]]]
    res_idx = np.sort(np.concatenate([t["h_pos"], samp]))
    res_kv = t["host_kv"][res_idx]
    sk = sk2.build(t["K"].astype(np.float32))
    outs = []
    for wm, ns in ((od.W_SKETCH2, t["n"]), (od.W_PERFECT, 0)):
        outs.append(od.decode_group(t["q"], res_kv, res_idx, None, None, t["r"],
                                    t["host_kv"], 0.02, 0.1, od.EST_CLIP, wm,
                                    sketch2=sk, n_short=ns))
    (ha, ua), (hb, ub) = outs
    assert np.array_equal(ua, ub)
    for a, b in zip(ha, hb):
        assert a["k_star"] == b["k_star"]
        assert np.array_equal(a["fetch_pos"], b["fetch_pos"])
        for k in ("m", "dnorm", "beta_star", "eps_hat0", "eps_hat", "d_hat"):
            assert abs(a[k] - b[k]) <= 1e-12 * max(1.0, abs(b[k])), (k, a[k], b[k])
        assert np.allclose(a["o"], b["o"], rtol=1e-12, atol=1e-12)
    assert any(h["k_star"] > 0 for h in ha)
    n_nonres = int(np.sum((t["r"] < 1)) - samp.size)
    assert ha[0]["shortlist"].size == n_nonres


# ---------------------------------------------------------------- maintenance
# "Verify Before You Fetch", section 3 and Appendix A.3.1-A.3.2.

def check_append_invariants(seed, B=2, G=3, ns=40, n=25, d=128, s=16):
    """After appending tokens: every resident list stays ascending and ends
    at the new position, counts grow by one, r = 1 there, the host row is
    the new K/V, and the projected sketch row is within one bf16 rounding
    of P^T k evaluated in float64."""
    from oracle import maintain as om
    rng = np.random.default_rng(seed)
    hkv = rng.integers(0, 2 ** 15, (B, G, ns, 2, d)).astype(np.uint16)
    r = rng.uniform(0.1, 0.9, (B, G, ns)).astype(np.float32)
    res_idx = [[np.sort(rng.choice(n, 6, replace=False)).astype(np.int64)
                for _ in range(G)] for _ in range(B)]
    res_kv = [[hkv[b, g, res_idx[b][g]] for g in range(G)] for b in range(B)]
    proj = (rng.standard_normal((G, d, s)) / np.sqrt(s)).astype(np.float32)
    st = dict(host_kv=hkv, r=r, res_idx=res_idx, res_kv=res_kv,
              sketch=np.zeros((B, G, ns, s), dtype=np.uint16))
    for pos in (n, n + 1, n + 2):
        kf = rng.standard_normal((B, G, d)).astype(np.float32)
        k_new = om.bf16_rne(kf)
        v_new = om.bf16_rne(rng.standard_normal((B, G, d)).astype(np.float32))
        before = [[st["res_idx"][b][g].size for g in range(G)] for b in range(B)]
        om.append_token(st, pos, k_new, v_new, proj)
        for b in range(B):
            for g in range(G):
                idx = st["res_idx"][b][g]
                assert idx.size == before[b][g] + 1 and idx[-1] == pos
                assert np.all(np.diff(idx) > 0)
                assert np.array_equal(st["res_kv"][b][g][-1, 0], k_new[b, g])
                assert np.array_equal(st["res_kv"][b][g][-1, 1], v_new[b, g])
                assert st["r"][b, g, pos] == 1.0
                assert np.array_equal(st["host_kv"][b, g, pos, 0], k_new[b, g])
                k64 = (k_new[b, g].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                exact = proj[g].astype(np.float64).T @ k64
                got = (st["sketch"][b, g, pos].astype(np.uint32) << 16).view(np.float32)
                # bf16 keeps 8 significant bits: within 2^-8 relative, plus
                # the fp32 sum's rounding
                assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-5)
    # appending out of order is refused
    try:
        om.append_token(st, n, k_new, v_new, proj)
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-order append accepted")


def check_staged_hits(seed):
    """Staged rows: the hits are exactly the rows in both unions, so the
    host bytes of a step with staging plus the saved bytes equal those of
    the same step without it."""
    from oracle import maintain as om
    rng = np.random.default_rng(seed)
    a = np.sort(rng.choice(1000, 120, replace=False))
    b = np.sort(rng.choice(1000, 150, replace=False))
    hits = om.staged_hits(a, b)
    assert set(hits.tolist()) == set(a.tolist()) & set(b.tolist())
    miss = np.setdiff1d(b, hits)
    assert miss.size * 512 + hits.size * 512 == b.size * 512
    assert om.staged_hits(a, a).size == a.size
    assert om.staged_hits(a, np.zeros(0, dtype=np.int64)).size == 0
