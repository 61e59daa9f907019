"""Pins for the KVFetch oracle (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import compress as oc
from oracle import decode as od
from tests import pins
from workloads import bf16_to_f32, make_decode_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_lr(rng, n, spread=3.0):
    w = np.exp(rng.normal(0, spread, n))
    r = rng.uniform(0.02, 0.95, n)
    return w, r


def test_shrinkage_golden():
    with open(os.path.join(GOLDEN, "shrinkage_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w, r = np.array(c["w"]), np.array(c["r"])
        beta = od.shrinkage_beta(w, r)
        assert abs(beta - c["beta"]) <= 1e-14 * c["beta"]
        lam = od.lambdas(w, r, beta)
        assert np.allclose(lam, c["lam"], rtol=0, atol=1e-14)
        bi, vi, b_i = od.cert_terms(w, r, lam)
        assert abs(vi.sum() - c["V"]) <= 1e-14 * c["V"]
        b1, b2, im = od.top2(b_i)
        assert (abs(b1 - c["b"]), abs(b2 - c["b2"]), im) == \
            (pytest.approx(0, abs=1e-14), pytest.approx(0, abs=1e-14),
             c["argmax_unique"])
        assert od.mse(lam, w, r) == pytest.approx(c["mse"], rel=1e-14)
        assert od.mse(np.ones_like(r), w, r) == pytest.approx(
            c["mse_unbiased"], rel=1e-14)
        assert od.mse(r, w, r) == pytest.approx(c["mse_lower"], rel=1e-14)


@pytest.mark.parametrize("seed", range(8))
def test_shrinkage_is_mse_minimiser(seed):
    rng = np.random.default_rng(100 + seed)
    w, r = _rand_lr(rng, int(rng.integers(2, 13)))
    pins.check_shrinkage_lbfgsb(w, r)
    pins.check_kkt(w, r)


def _heavy(rng, n):
    w = np.exp(rng.normal(0, 1, n))
    r = rng.uniform(0.2, 0.9, n)
    k = max(1, n // 8)
    w[:k] *= 50.0
    r[:k] = rng.uniform(0.02, 0.1, k)
    return w, r


@pytest.mark.parametrize("seed", range(6))
def test_shrinkage_heavy_tokens(seed):
    """Heavy tokens with small r. At the fixed point beta* >= max_i w_i(1-r_i)
    (below that, the heaviest token alone would contribute more than beta), so
    lambda_i >= r_i holds without the lower clip."""
    rng = np.random.default_rng(150 + seed)
    w, r = _heavy(rng, int(rng.integers(4, 13)))
    beta = od.shrinkage_beta(w, r)
    assert beta >= np.max(w * (1 - r)) * (1 - 1e-15)
    assert beta <= np.sum(w * (1 - r)) * (1 + 1e-15)
    pins.check_shrinkage_lbfgsb(w, r)
    pins.check_kkt(w, r)
    pins.check_range_bound(w, r)


def test_binary_golden():
    with open(os.path.join(GOLDEN, "binary_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w, r = np.array(c["w"], float), np.array(c["r"], float)
        lam, beta, moved = od.binary_lambdas(w, r, np.array(c["pos"]))
        assert lam.tolist() == c["lam"]
        assert (beta, moved) == (c["beta"], c["moved"])
        assert od.mse(lam, w, r) == c["mse"]
        assert od.mse(np.ones_like(r), w, r) == c["mse_unbiased"]
        pins.check_binary_prefix(w, r, np.array(c["pos"]))


@pytest.mark.parametrize("seed", range(8))
def test_binary_is_prefix_minimum(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 40))
    w, r = _rand_lr(rng, n) if seed % 2 else _heavy(rng, n)
    pins.check_binary_prefix(w, r, rng.permutation(n))


def test_binary_equal_tokens_closed_form():
    """n equal tokens with r = 1/m: token k (1-based) moves iff
    (1 - r)/r > 2 (k - 1)(1 - r), i.e. k - 1 < m / 2, so min(n, ceil(m / 2))
    move (exact in binary floating point for m a power of two)."""
    for m in (2, 4, 8, 16, 64):
        for n in (1, 3, 40):
            w = np.full(n, 0.75)
            r = np.full(n, 1.0 / m)
            lam, beta, moved = od.binary_lambdas(w, r, np.arange(n))
            assert moved == min(n, math.ceil(m / 2))
            assert np.all(lam[:moved] == 1.0 / m) and np.all(lam[moved:] == 1.0)


@pytest.mark.parametrize("seed", range(4))
def test_binary_exact_enumeration(seed):
    rng = np.random.default_rng(400 + seed)
    w, r = _heavy(rng, 10)
    pins.check_enumeration(np.exp(rng.normal(0, 1, 3)), w, r, 0.1,
                           od.EST_BINARY)


@pytest.mark.parametrize("seed", range(3))
def test_exact_attention_mp(seed):
    rng = np.random.default_rng(500 + seed)
    n, d = int(rng.integers(1, 12)), 16
    q, k, v = (rng.normal(0, 2, (d,)), rng.normal(0, 2, (n, d)),
               rng.normal(0, 1, (n, 3)))
    pins.check_exact_attention_mp(q, k, v)


def test_exact_attention_two_keys():
    """Logits 1 and 0 (d = 4, q = (2, 0, 0, 0)): o = (e v1 + v2)/(e + 1)."""
    q = np.array([2.0, 0, 0, 0])
    k = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, logd = od.exact_attention(q, k, v)
    e = math.e
    assert np.allclose(o, [e / (e + 1), 1 / (e + 1)], rtol=1e-15, atol=0)
    assert logd == pytest.approx(math.log(e + 1), rel=1e-15)


def test_dense_step_layout():
    """dense_step maps query head h to KV head h // (Hq/G)."""
    rng = np.random.default_rng(7)
    q = rng.normal(size=(2, 4, 8))
    kv = rng.normal(size=(2, 2, 5, 2, 8))
    o, logd = od.dense_step(q, kv)
    for b in range(2):
        for h in range(4):
            oo, ll = od.exact_attention(q[b, h], kv[b, h // 2, :, 0], kv[b, h // 2, :, 1])
            assert np.array_equal(o[b, h], oo) and logd[b, h] == ll


@pytest.mark.parametrize("seed", range(6))
def test_kkt_large(seed):
    rng = np.random.default_rng(200 + seed)
    w, r = _rand_lr(rng, 5000, spread=4.0)
    pins.check_kkt(w, r)


@pytest.mark.parametrize("V,b,delta", [(1.0, 0.5, 0.05), (1e-6, 3.0, 0.1),
                                       (250.0, 1e-9, 0.01), (0.0, 2.0, 0.2)])
def test_bernstein_root(V, b, delta):
    pins.check_bernstein_root(V, b, delta)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("est", [od.EST_CLIP, od.EST_UNBIASED])
def test_exact_enumeration(seed, est):
    rng = np.random.default_rng(300 + seed)
    nl = int(rng.integers(1, 12))
    w, r = _rand_lr(rng, nl, spread=1.5)
    wH = np.exp(rng.normal(0, 1, 3))
    pins.check_enumeration(wH, w, r, float(rng.choice([0.05, 0.1, 0.3])), est)


def _plan_terms(seed, n):
    rng = np.random.default_rng(400 + seed)
    w, r = _rand_lr(rng, n, spread=2.0)
    beta = od.shrinkage_beta(w, r)
    lam = od.lambdas(w, r, beta)
    return w, r, od.cert_terms(w, r, lam)


@pytest.mark.parametrize("seed", range(6))
def test_gains_leave_one_out(seed):
    w, r, (bi, vi, b_i) = _plan_terms(seed, 48)
    D = float(w.sum() + 5.0)
    pins.check_gains_loo(bi, vi, b_i, D, 0.05)
    # a tied maximum: removing either copy leaves b unchanged
    b_t = b_i.copy()
    j = int(np.argmax(b_t))
    b_t[(j + 1) % b_t.size] = b_t[j]
    pins.check_gains_loo(bi, vi, b_t, D, 0.05)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("eps", [0.02, 0.1, 0.3])
def test_kstar_bruteforce(seed, eps):
    rng = np.random.default_rng(500 + seed)
    w, r = _rand_lr(rng, int(rng.integers(8, 64)), spread=2.0)
    D = float(w.sum() * rng.uniform(1.0, 3.0))
    pins.check_kstar_bruteforce(w, r, D, eps, 0.05)


def _c1_inputs(seed=0, budget=None, n=None):
    w = make_decode_workload("c1", seed=seed, n=n, budget=budget)
    kf = bf16_to_f32(w["host_kv"][..., 0, :])
    vf = bf16_to_f32(w["host_kv"][..., 1, :])
    cm = oc.compress(w["tau"], kf, vf, w["budget"], w["n_sink"], w["n_local"],
                     w["seed"])
    sl = cm[0][0]
    return w, sl


def _decode_c1(w, sl, eps, weights, estimator=od.EST_CLIP):
    return od.decode_group(bf16_to_f32(w["q"][0]), sl["resident_kv"],
                           sl["resident_idx"], bf16_to_f32(w["sketch"][0, 0]),
                           w["proj"][0], sl["r"], bf16_to_f32(w["host_kv"][0, 0]),
                           eps, w["delta"], estimator, weights)


@pytest.mark.parametrize("weights", [od.W_SKETCH, od.W_PERFECT])
def test_fetch_all_is_exact_attention(weights):
    """eps -> 0 forces k* = |L|: the output is textbook attention (eq. 1)."""
    w, sl = _c1_inputs()
    heads, union = _decode_c1(w, sl, 1e-300, weights)
    hd = heads[0]
    assert hd["k_star"] == int(sl["in_l"].sum())
    kv = bf16_to_f32(w["host_kv"][0, 0])
    o_ref, logd = od.exact_attention(bf16_to_f32(w["q"][0, 0]), kv[:, 0], kv[:, 1])
    assert np.allclose(hd["o"], o_ref, rtol=1e-12, atol=1e-12)
    assert abs(math.log(hd["d_hat"]) + hd["m"] - logd) < 1e-12
    assert set(union.tolist()) == set(np.nonzero(sl["in_l"] & ~sl["in_s"])[0])


def test_all_resident_is_exact():
    """eta = 1: L is empty, eps^ = 0 and the estimate is exact."""
    w, sl = _c1_inputs(budget=1024)
    assert sl["in_l"].sum() == 0
    heads, union = _decode_c1(w, sl, 0.1, od.W_SKETCH)
    kv = bf16_to_f32(w["host_kv"][0, 0])
    o_ref, logd = od.exact_attention(bf16_to_f32(w["q"][0, 0]), kv[:, 0], kv[:, 1])
    assert heads[0]["eps_hat0"] == 0.0 and heads[0]["k_star"] == 0
    assert np.allclose(heads[0]["o"], o_ref, rtol=1e-12, atol=1e-12)
    assert union.size == 0


def test_perfect_sketch_denominator_is_exact():
    """With exact planning weights D~ equals the full denominator."""
    w, sl = _c1_inputs()
    heads, _ = _decode_c1(w, sl, 0.1, od.W_PERFECT)
    kv = bf16_to_f32(w["host_kv"][0, 0])
    _, logd = od.exact_attention(bf16_to_f32(w["q"][0, 0]), kv[:, 0], kv[:, 1])
    assert abs(math.log(heads[0]["dnorm"]) + heads[0]["m"] - logd) < 1e-12


def test_plan_scale_invariance():
    """Shifting every logit by a constant (scaling all weights and D~) leaves
    lambda, eps^, the gain order and k* unchanged (reading R5)."""
    rng = np.random.default_rng(7)
    w, r = _rand_lr(rng, 300, 2.0)
    D = float(w.sum() * 1.5)
    pos = np.arange(300)
    a = od.plan_row(w, r, pos, D, 0.05, 0.05)
    b = od.plan_row(w * 2.0 ** -30, r, pos, D * 2.0 ** -30, 0.05, 0.05)
    assert np.allclose(a["lam"], b["lam"], rtol=1e-12)
    assert a["k_star"] == b["k_star"] and a["k_star"] > 0
    assert abs(a["eps_hat"] - b["eps_hat"]) <= 1e-12 * a["eps_hat"]
    assert np.array_equal(a["order"][:a["k_star"]], b["order"][:b["k_star"]])


def test_monte_carlo_coverage_perfect():
    """Theorem 2 with exact weights: over fresh Poisson samples the estimate
    stays within eps^(L') of D with frequency >= 1 - delta."""
    w, sl = _c1_inputs()
    delta = w["delta"]
    kv = bf16_to_f32(w["host_kv"][0, 0])
    qv = bf16_to_f32(w["q"][0, 0])
    _, logd = od.exact_attention(qv, kv[:, 0], kv[:, 1])
    n_trials = 150
    fails = 0
    for s in range(n_trials):
        cm = oc.compress_slice(w["tau"][0, 0], w["budget"], w["n_sink"],
                               w["n_local"], 1000 + s, 0, 0)
        idx = cm["resident_idx"]
        res_kv = np.stack([kv[idx, 0], kv[idx, 1]], axis=1)
        heads, _ = od.decode_group(qv[None], res_kv, idx,
                                   bf16_to_f32(w["sketch"][0, 0]), w["proj"][0],
                                   cm["r"], kv, 0.1, delta, od.EST_CLIP,
                                   od.W_PERFECT)
        hd = heads[0]
        err = abs(math.exp(math.log(hd["d_hat"]) + hd["m"] - logd) - 1.0)
        fails += err > hd["eps_hat"]
    assert fails <= delta * n_trials + 3 * math.sqrt(delta * n_trials)


def test_monte_carlo_coverage_plan_vectorised():
    """The same property over 10^5 samples of a fixed plan (Theorem 2 holds
    for any sample-independent coefficients and order)."""
    rng = np.random.default_rng(11)
    w, r = _rand_lr(rng, 2000, 1.5)
    wH = np.exp(rng.normal(2, 1, 50))
    D = float(wH.sum() + w.sum())
    delta = 0.1
    plan = od.plan_row(w, r, np.arange(w.size), D, 0.05, delta)
    k = plan["k_star"]
    assert k > 0
    fetched = np.zeros(w.size, dtype=bool)
    fetched[plan["order"][:k]] = True
    coef = plan["lam"] * w / r
    fails = 0
    n_tot = 0
    for chunk in range(10):
        z = rng.random((10000, w.size)) < r
        est = wH.sum() + w[fetched].sum() + (z[:, ~fetched] * coef[~fetched]).sum(1)
        fails += int(np.sum(np.abs(est - D) / D > plan["eps_hat"]))
        n_tot += 10000
    assert fails / n_tot <= delta


def test_c2_shape_runs_and_certifies():
    """A reduced c2 layer: every decision ends with eps^(L') < eps and the
    fetch union is disjoint from the resident set."""
    w = make_decode_workload("c2", seed=1, n=4096, G=2)
    kf = bf16_to_f32(w["host_kv"][..., 0, :])
    vf = bf16_to_f32(w["host_kv"][..., 1, :])
    cm = oc.compress(w["tau"], kf, vf, w["budget"], w["n_sink"], w["n_local"],
                     w["seed"])
    res_kv = [[cm[0][g]["resident_kv"] for g in range(2)]]
    res_idx = [[cm[0][g]["resident_idx"] for g in range(2)]]
    r = np.stack([cm[0][g]["r"] for g in range(2)])[None]
    heads, unions = od.decode_step(bf16_to_f32(w["q"]), res_kv, res_idx,
                                   bf16_to_f32(w["sketch"]), w["proj"], r,
                                   bf16_to_f32(w["host_kv"]), w["eps"], w["delta"])
    for h in range(w["Hq"]):
        hd = heads[0][h]
        assert hd["eps_hat"] < w["eps"]
        if hd["k_star"]:
            assert hd["suffix"][hd["k_star"] - 1] >= w["eps"]
    for g in range(2):
        assert not set(unions[0][g].tolist()) & set(res_idx[0][g].tolist())


@pytest.mark.parametrize("seed", range(10))
def test_fixed_point_single_breakpoint_form(seed):
    """Because beta* >= max_i w_i(1 - r_i), every token sits on or above its
    lower clip at the root, so beta* is also the root of
    sum_i max(0, w_i - beta r_i/(1 - r_i)) - beta, a function with one
    breakpoint per token (scipy brentq on that form must agree)."""
    from scipy.optimize import brentq
    rng = np.random.default_rng(600 + seed)
    if seed % 2:
        w, r = _heavy(rng, int(rng.integers(3, 300)))
    else:
        w, r = _rand_lr(rng, int(rng.integers(3, 3000)), spread=3.0)
    beta = od.shrinkage_beta(w, r)
    rho = r / (1 - r)
    f = lambda b: float(np.sum(np.maximum(0.0, w - b * rho))) - b  # noqa: E731
    ref = brentq(f, 0.0, float(np.sum(w)), xtol=1e-300, rtol=1e-15, maxiter=500)
    assert abs(beta - ref) <= 1e-12 * ref
    # and the two-breakpoint residual of Definition 2 is never below the
    # one-breakpoint form
    for b in np.linspace(0, 2 * beta, 9):
        assert od.shrink_residual(b, w, r) <= f(b) + 1e-13 * float(np.sum(w))


# ---------------------------------------------------------------- sketch logits
@pytest.mark.parametrize("seed", range(4))
def test_sketch_logits_orthogonal_projection(seed):
    """An orthogonal P preserves inner products: sketch logits = exact
    logits <q, k>/sqrt(d) (Algorithm 2's sketch weights, reading R4)."""
    pins.check_sketch_orthogonal(900 + seed)


@pytest.mark.parametrize("seed", range(4))
def test_sketch_logits_unbiased_over_coordinate_blocks(seed):
    """E[P P^T] = I exactly over signed coordinate blocks: the mean sketch
    logit is the exact logit (the scale is 1/sqrt(d), not 1/sqrt(s))."""
    pins.check_sketch_blocks(910 + seed)


def test_sketch_logits_unbiased_gaussian_projection():
    """The sketch of the decode workloads: P with N(0, 1/s) entries
    (E[P P^T] = I). Over 4000 seeded draws of P the mean sketch logit of a
    key must match <q, k>/sqrt(d) within five standard errors, at d = 128,
    s = 32 (a 1/sqrt(s) scale or a missing 1/sqrt(d) would be off by a
    factor of 2 or 11)."""
    rng = np.random.default_rng(920)
    d, s, m_draws = 128, 32, 4000
    q = rng.standard_normal(d)
    k = 0.5 * q + rng.standard_normal(d)  # a logit well away from 0
    exact = float(q @ k) / math.sqrt(d)
    vals = np.empty(m_draws)
    for j in range(m_draws):
        P = rng.standard_normal((d, s)) / math.sqrt(s)
        vals[j] = od.sketch_logits(q, (k @ P)[None], P)[0]
    se = vals.std(ddof=1) / math.sqrt(m_draws)
    assert abs(vals.mean() - exact) <= 5 * se, (vals.mean(), exact, se)
    assert exact > 20 * se


@pytest.mark.parametrize("seed", range(3))
def test_sketch_mode_with_identity_projection_is_perfect_mode(seed):
    """P = I, s = d: sketch mode and exact-weight mode agree bit for bit in
    every output of the decode step."""
    pins.check_sketch_decode_identity(930 + seed)


# ---------------------------------------------------------------- estimator
@pytest.mark.parametrize("est", [od.EST_CLIP, od.EST_UNBIASED, od.EST_BINARY])
@pytest.mark.parametrize("weights", [od.W_SKETCH, od.W_PERFECT])
def test_estimator_bias_by_exact_enumeration(est, weights):
    """Theorem 2's estimator through decode_group over every Poisson sample
    of a 10-token L with a fixed fetch set: E[D^] and E[N^] fall short of D
    and N by exactly the shrinkage bias on L' (zero with lambda = 1)."""
    pins.check_estimator_enumeration(940 + 3 * est + weights, est, weights,
                                     n_l=10, n_fetch=3)
