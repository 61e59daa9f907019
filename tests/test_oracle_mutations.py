"""Plant plausible mistakes in the oracle (CPU only) and confirm that at
least one pin catches each of them. Nothing here touches the library."""

import math

import numpy as np
import pytest

from oracle import compress as oc
from oracle import decode as od
from oracle import philox
from oracle import maintain as om
from oracle import sketch2 as sk2
from tests import pins


def _orig(mod, name):
    return getattr(mod, name)


def _w_r(seed, n, spread=2.0):
    rng = np.random.default_rng(seed)
    return np.exp(rng.normal(0, spread, n)), rng.uniform(0.02, 0.95, n)


def run_pins():
    """A compact battery of the pins; returns the names of those that fail."""
    failed = []

    def attempt(name, fn):
        try:
            fn()
        except (AssertionError, ValueError, ZeroDivisionError):
            failed.append(name)

    w, r = _w_r(1, 10)
    attempt("lbfgsb", lambda: pins.check_shrinkage_lbfgsb(w, r))
    attempt("lbfgsb_heavy", lambda: pins.check_shrinkage_lbfgsb(*_heavy(8, 10)))
    attempt("kkt", lambda: pins.check_kkt(*_w_r(2, 400)))
    attempt("kkt_heavy", lambda: pins.check_kkt(*_heavy(9, 400)))
    attempt("golden_shrink", _golden_shrink)
    attempt("bernstein", lambda: pins.check_bernstein_root(1.0, 0.5, 0.05))
    attempt("range", lambda: pins.check_range_bound(*_w_r(3, 50)))
    we, re_ = _w_r(4, 9, 1.5)
    attempt("enum", lambda: pins.check_enumeration(np.ones(2), we, re_, 0.1))
    wg, rg = _w_r(5, 30)
    lam = od.lambdas(wg, rg, od.shrinkage_beta(wg, rg))
    bi, vi, b_i = od.cert_terms(wg, rg, lam)
    attempt("gains", lambda: pins.check_gains_loo(bi, vi, b_i, wg.sum() + 3, 0.05))
    wk, rk = _w_r(6, 40)
    attempt("kstar", lambda: pins.check_kstar_bruteforce(wk, rk, wk.sum() * 1.3,
                                                         0.05, 0.05))
    rng = np.random.default_rng(7)
    tq = rng.integers(1, 2 ** 16, size=25)
    attempt("waterfill", lambda: [pins.check_water_level_bruteforce(tq, b)
                                  for b in (1, 5, 12, 24)])
    tau = rng.beta(0.5, 5, size=3000).astype(np.float32)
    attempt("rates", lambda: pins.check_rates_sum(tau, 300, 4, 16))
    attempt("golden_wf", _golden_wf)
    wb, rb = _w_r(10, 30)
    attempt("binary", lambda: pins.check_binary_prefix(wb, rb))
    attempt("binary_heavy", lambda: pins.check_binary_prefix(*_heavy(11, 30)))
    attempt("golden_binary", _golden_binary)
    rng = np.random.default_rng(12)
    attempt("attention_mp", lambda: pins.check_exact_attention_mp(
        rng.normal(0, 2, 16), rng.normal(0, 2, (6, 16)), rng.normal(0, 1, (6, 3))))
    attempt("sketch_orthogonal", lambda: pins.check_sketch_orthogonal(13))
    attempt("sketch_blocks", lambda: pins.check_sketch_blocks(14))
    attempt("sketch_identity", lambda: pins.check_sketch_decode_identity(15))
    attempt("estimator_enum", lambda: pins.check_estimator_enumeration(
        16, od.EST_CLIP, od.W_SKETCH, n_l=6))
    attempt("estimator_enum_unbiased", lambda: pins.check_estimator_enumeration(
        17, od.EST_UNBIASED, od.W_PERFECT, n_l=6))
    attempt("philox_kat", pins.check_philox_kat)
    attempt("sketch2_levels", lambda: pins.check_sketch2_levels(18))
    attempt("sketch2_error", lambda: pins.check_sketch2_error(19))
    attempt("sketch2_rotation", lambda: pins.check_sketch2_rotation(20))
    attempt("sketch2_cost", pins.check_sketch2_cost)
    attempt("sketch2_identity", lambda: pins.check_sketch2_logit_identity(21))
    attempt("shortlist", lambda: pins.check_shortlist_bruteforce(22))
    attempt("sketch2_full", lambda: pins.check_sketch2_full_shortlist(23))
    attempt("append", lambda: pins.check_append_invariants(24))
    attempt("staged", lambda: pins.check_staged_hits(25))
    return failed


def _golden_binary():
    # ten equal tokens with r = 1/8: four move, the fifth is an exact tie
    lam, beta, moved = od.binary_lambdas(np.ones(10), np.full(10, 0.125),
                                         np.arange(10))
    assert (moved, beta) == (4, 3.5)


def _heavy(seed, n):
    """A few heavy tokens with small inclusion probabilities: the regime in
    which the lower end of the clip box is active."""
    rng = np.random.default_rng(seed)
    w = np.exp(rng.normal(0, 1, n))
    r = rng.uniform(0.2, 0.9, n)
    k = max(1, n // 8)
    w[:k] *= 50.0
    r[:k] = rng.uniform(0.02, 0.1, k)
    return w, r


def _golden_shrink():
    w = np.array([4.0, 1.0, 0.01])
    r = np.array([0.5, 0.5, 0.5])
    beta = od.shrinkage_beta(w, r)
    assert abs(beta - 2.0) < 1e-12
    assert np.allclose(od.lambdas(w, r, beta), [0.5, 1.0, 1.0], atol=1e-12)


def _golden_wf():
    sl = oc.compress_slice(np.array([1.0, 0.75, 0.5, 0.125, 0.125], np.float32),
                           3, 1, 0, 0, 0, 0)
    assert sl["in_h"].tolist() == [True, True, False, False, False]
    assert sl["r"][2] == np.float32(2 / 3)


def test_unmutated_oracle_passes_all_pins():
    assert run_pins() == []


def _eps_no_ab(beta, var, bmax, dnorm, delta):
    l, a = od.bernstein_consts(delta)
    return (beta + np.sqrt((a * bmax) ** 2 + 2.0 * var * l)) / dnorm


def _eps_log10(beta, var, bmax, dnorm, delta):
    l = math.log10(2.0 / delta)
    a = l / 3
    return (beta + a * bmax + np.sqrt((a * bmax) ** 2 + 2.0 * var * l)) / dnorm


def _lam_no_1mr(w, r, beta):
    with np.errstate(divide="ignore", invalid="ignore"):
        x = beta * r / w
    return np.where(w > 0, np.minimum(1.0, np.maximum(r, x)), 1.0)


def _lam_swapped(w, r, beta):
    with np.errstate(divide="ignore", invalid="ignore"):
        x = beta * (1.0 - r) / (w * r)
    return np.where(w > 0, np.minimum(1.0, np.maximum(r, x)), 1.0)


def _terms_no_1mr(w, r, lam):
    return w * (1 - lam), lam * lam * w * w / r, lam * w * np.maximum(r, 1 - r) / r


def _terms_min(w, r, lam):
    return (w * (1 - lam), lam * lam * w * w * (1 - r) / r,
            lam * w * np.minimum(r, 1 - r) / r)


def _gains_no_argmax(beta_i, v_i, b_i, dnorm, delta):
    l, a = od.bernstein_consts(delta)
    V = float(np.sum(v_i))
    b1 = float(b_i.max())
    s = math.sqrt((a * b1) ** 2 + 2.0 * V * l)
    sp = np.sqrt((a * b1) ** 2 + 2.0 * np.maximum(V - v_i, 0) * l)
    return (beta_i + 2.0 * v_i * l / (s + sp)) / dnorm


def _suffix_prefix(order, beta_i, v_i, b_i, dnorm, delta):
    bs, vs, bb = beta_i[order], v_i[order], b_i[order]
    sb = np.concatenate([[0.0], np.cumsum(bs)])[::-1]
    sv = np.concatenate([[0.0], np.cumsum(vs)])[::-1]
    mb = np.concatenate([[0.0], np.maximum.accumulate(bb)])[::-1]
    return od.eps_hat(sb, sv, mb, dnorm, delta)


def _order_ascending(g, pos):
    return np.lexsort((pos, g))


def _wl_offbyone(tq_free, b_free):
    j, num, den = _orig_wl(tq_free, b_free)
    if den == 0 or j == 0:
        return j, num, den
    srt = np.sort(np.asarray(tq_free, np.int64))[::-1]
    return j - 1, num + 1, int(srt[j - 1:].sum())


def _rates_strict(tq, forced, num, den):
    r, in_h = _orig_rates(tq, forced, num, den)
    if den == 0:
        return r, in_h
    free = ~forced
    prod = tq[free].astype(np.int64) * np.int64(num)
    in_h[free] = prod > den
    r[free] = np.where(prod > den, np.float32(1.0),
                       np.minimum(r[free], oc.ONE_MINUS_ULP))
    return r, in_h


def _beta_upper(w, r, max_iter=200):
    return float(np.sum(w * (1.0 - r)))


def _binary_variant(key, stop, add):
    """binary_lambdas with the order key, stop test or bias term replaced."""
    def f(w, r, pos):
        w = np.asarray(w, np.float64)
        r = np.asarray(r, np.float64)
        kappa = key(w, r)
        lam = np.ones_like(w)
        beta = 0.0
        moved = 0
        for i in np.lexsort((np.asarray(pos), -kappa)):
            if not stop(kappa[i], beta):
                break
            lam[i] = r[i]
            beta += add(w[i], r[i])
            moved += 1
        return lam, beta, moved
    return f


_bin_ok_key = lambda w, r: w * (1 - r) / r
_bin_ok_stop = lambda k, b: k > 2 * b
_bin_ok_add = lambda w, r: w * (1 - r)

def _attention_no_scale(q, k, v):
    q = np.asarray(q, np.float64)
    lg = np.asarray(k, np.float64) @ q
    m = lg.max()
    w = np.exp(lg - m)
    return (w @ np.asarray(v, np.float64)) / w.sum(), math.log(w.sum()) + m


def _sketch_scale_s(qh, sk, proj):
    qh = np.asarray(qh, np.float64)
    qp = np.asarray(proj, np.float64).T @ qh
    return np.asarray(sk, np.float64) @ qp / math.sqrt(np.asarray(proj).shape[1])


def _sketch_unscaled(qh, sk, proj):
    qp = np.asarray(proj, np.float64).T @ np.asarray(qh, np.float64)
    return np.asarray(sk, np.float64) @ qp


def _sketch_p_not_transposed(qh, sk, proj):
    qh = np.asarray(qh, np.float64)
    qp = np.asarray(proj, np.float64) @ qh
    return np.asarray(sk, np.float64) @ qp / math.sqrt(qh.size)


def _sketch_first_rows(qh, sk, proj):
    # the sketch rows of tokens 0..m-1 instead of the rows passed in (an
    # indexing slip: scores the wrong tokens whenever L is not a prefix)
    return _orig_sketch(qh, sk, proj)[::-1]


def _coef_no_r(w_res, r_res, lam_res, exact_res):
    w_res = np.asarray(w_res, np.float64)
    return np.where(exact_res, w_res, np.asarray(lam_res) * w_res)


def _coef_no_lambda(w_res, r_res, lam_res, exact_res):
    w_res = np.asarray(w_res, np.float64)
    return np.where(exact_res, w_res, w_res / np.asarray(r_res, np.float64))


def _combine_num_no_fetched(alpha, v_res, w_f, v_f):
    d_hat = float(alpha.sum() + w_f.sum())
    num = alpha @ v_res
    return d_hat, num, num / d_hat


def _combine_den_no_fetched(alpha, v_res, w_f, v_f):
    d_hat = float(alpha.sum())
    num = alpha @ v_res + w_f @ v_f
    return d_hat, num, num / d_hat


def _philox_nine_rounds(c0, c1, c2, c3, k0, k1):
    # the reference round function, applied nine times
    from oracle import philox as ph
    c0 = np.asarray(c0, dtype=np.uint64) & ph.MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & ph.MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & ph.MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & ph.MASK32
    ka, kb = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(9):
        p0 = ph.M0 * c0
        p1 = ph.M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(ka),
                          p1 & ph.MASK32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(kb),
                          p0 & ph.MASK32)
        ka = (ka + ph.W0) & 0xFFFFFFFF
        kb = (kb + ph.W1) & 0xFFFFFFFF
    return c0, c1, c2, c3


def _pairs_interleaved(d):
    return np.stack([np.arange(0, d, 2), np.arange(1, d, 2)], axis=1)


def _channels_interleaved(pairs, d):
    pairs = np.asarray(pairs, dtype=np.int64)
    return np.sort(np.concatenate([2 * pairs, 2 * pairs + 1]))


def _quant_one_range(vals):
    # one zero point and scale for the whole group
    v = np.asarray(vals, dtype=np.float32)
    z = np.full(v.shape[1], v.min(), dtype=np.float32)
    s = np.full(v.shape[1], (v.max() - v.min()) / np.float32(3), dtype=np.float32)
    z = z.astype(np.float16).astype(np.float32)
    s = s.astype(np.float16).astype(np.float32)
    c = np.clip(np.rint((v - z) / s), 0, 3).astype(np.uint8)
    return z, s, c


def _quant_floor(vals):
    # codes truncated instead of rounded
    v = np.asarray(vals, dtype=np.float32)
    z, s, _ = _orig_quant(v)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.clip(np.floor((v - z) / s), 0, 3)
    return z, s, np.where(s > 0, c, 0).astype(np.uint8)


def _sk2_unscaled(qh, sk):
    return _orig_sk2_logits(qh, sk) * np.sqrt(np.asarray(qh).size)


def _sk2_channel_shift(qh, sk):
    # query entries taken from the pair's other channel
    qh = np.asarray(qh, dtype=np.float64)
    d = qh.size
    sh = np.concatenate([qh[d // 2:], qh[:d // 2]])
    return _orig_sk2_logits(sh, sk)


def _shortlist_min_heads(scores32, eligible, n_short):
    s = np.asarray(scores32, dtype=np.float32)
    return _orig_shortlist(np.broadcast_to(s.min(axis=0), s.shape), eligible, n_short)


def _shortlist_smallest(scores32, eligible, n_short):
    return _orig_shortlist(-np.asarray(scores32, dtype=np.float32), eligible, n_short)


def _energy_sum_abs(keys):
    k = np.abs(np.asarray(keys, dtype=np.float64))
    h = k.shape[1] // 2
    return k[:, :h].sum(axis=0) + k[:, h:].sum(axis=0) * 0.0


def _bf16_truncate(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def _hits_union(prev_union, union):
    return np.union1d(np.asarray(prev_union), np.asarray(union)).astype(np.int64)


def _sketch_row_fp16(proj_g, k):
    # the sum kept in half precision
    acc = (np.asarray(proj_g, dtype=np.float16).T @ np.asarray(k, dtype=np.float16))
    return om.bf16_rne(acc.astype(np.float32))


_orig_quant = sk2.quantize_group
_orig_sk2_logits = sk2.sketch_logits
_orig_shortlist = sk2.shortlist
_orig_wl = oc.water_level
_orig_rates = oc.rates
_orig_sketch = od.sketch_logits

MUTATIONS = [
    ("eps_hat drops the b*l/3 term", od, "eps_hat", _eps_no_ab),
    ("eps_hat uses log10", od, "eps_hat", _eps_log10),
    ("lambda drops the (1-r) factor", od, "lambdas", _lam_no_1mr),
    ("lambda with r and 1-r swapped", od, "lambdas", _lam_swapped),
    ("variance term drops (1-r)", od, "cert_terms", _terms_no_1mr),
    ("range term uses min(r, 1-r)", od, "cert_terms", _terms_min),
    ("gains ignore the unique argmax", od, "gains", _gains_no_argmax),
    ("suffix sums taken as prefix sums", od, "suffix_eps", _suffix_prefix),
    ("gain order ascending", od, "gain_order", _order_ascending),
    ("water level one saturated token short", oc, "water_level", _wl_offbyone),
    ("exact saturation left in L", oc, "rates", _rates_strict),
    ("beta* is the bracket's upper end", od, "shrinkage_beta", _beta_upper),
    ("binary order ascending", od, "binary_lambdas",
     _binary_variant(lambda w, r: -w * (1 - r) / r, _bin_ok_stop, _bin_ok_add)),
    ("binary order by w / r", od, "binary_lambdas",
     _binary_variant(lambda w, r: w / r, _bin_ok_stop, _bin_ok_add)),
    ("binary stop compares with beta, not 2 beta", od, "binary_lambdas",
     _binary_variant(_bin_ok_key, lambda k, b: k > b, _bin_ok_add)),
    ("binary stop not strict", od, "binary_lambdas",
     _binary_variant(_bin_ok_key, lambda k, b: k >= 2 * b, _bin_ok_add)),
    ("binary bias accumulates w", od, "binary_lambdas",
     _binary_variant(_bin_ok_key, _bin_ok_stop, lambda w, r: w)),
    ("attention logits not scaled by 1/sqrt(d)", od, "exact_attention",
     _attention_no_scale),
    ("sketch logits scaled by 1/sqrt(s)", od, "sketch_logits", _sketch_scale_s),
    ("sketch logits not scaled", od, "sketch_logits", _sketch_unscaled),
    ("sketch logits project q by P, not P^T", od, "sketch_logits",
     _sketch_p_not_transposed),
    ("sketch logits of the wrong tokens", od, "sketch_logits", _sketch_first_rows),
    ("S minus F_h coefficients drop 1/r", od, "output_coefficients", _coef_no_r),
    ("S minus F_h coefficients drop lambda", od, "output_coefficients",
     _coef_no_lambda),
    ("numerator omits the fetched rows", od, "combine", _combine_num_no_fetched),
    ("denominator omits the fetched rows", od, "combine", _combine_den_no_fetched),
    ("Philox Weyl constant W0 off by one", philox, "W0", 0x9E3779B8),
    ("Philox multiplier M1 wrong", philox, "M1", np.uint64(0xCD9E8D55)),
    ("Philox with nine rounds", philox, "philox4x32_10", _philox_nine_rounds),
    ("RoPE pairs taken as (2j, 2j+1)", sk2, "rope_pairs", _pairs_interleaved),
    ("kept channels taken as (2j, 2j+1)", sk2, "kept_channels",
     _channels_interleaved),
    ("2-bit scale a quarter of the range", sk2, "LEVELS", 4),
    ("one zero point and scale per group", sk2, "quantize_group", _quant_one_range),
    ("2-bit codes truncated", sk2, "quantize_group", _quant_floor),
    ("8 kept pairs instead of 16", sk2, "N_PAIRS", 8),
    ("groups of 64 tokens", sk2, "GROUP", 64),
    ("sketch2 logits not scaled", sk2, "sketch_logits", _sk2_unscaled),
    ("sketch2 query channels of the other half", sk2, "sketch_logits",
     _sk2_channel_shift),
    ("shortlist by the smallest score over the heads", sk2, "shortlist",
     _shortlist_min_heads),
    ("shortlist of the lowest scores", sk2, "shortlist", _shortlist_smallest),
    ("pair energy from one channel of the pair", sk2, "pair_energy",
     _energy_sum_abs),
    ("appended sketch row truncated to bf16", om, "bf16_rne", _bf16_truncate),
    ("appended sketch row summed in fp16", om, "sketch_row", _sketch_row_fp16),
    ("staged hits taken as the union", om, "staged_hits", _hits_union),
]


@pytest.mark.parametrize("label,mod,name,fn", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, label, mod, name, fn):
    monkeypatch.setattr(mod, name, fn)
    failed = run_pins()
    assert failed, f"no pin caught: {label}"
