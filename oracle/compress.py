"""PoissonComp oracle ("Verify Before You Fetch", Algorithm 1 and §4.1, eq. 3).

Per (layer, KV head) slice of n tokens with importance scores tau in [0, 1]:

1. Scores are read on a 2^-32 fixed-point grid and floored at one grid step,
   so that every token gets r > 0 (reading R1: the proofs need r_i > 0 on L,
   and a zero score could never be sampled).
2. Sink and local tokens (the forced set F) go straight to H; the budget
   (eta*n, rounded) includes them (reading R2).
3. The water level c solves sum_{i not in F} min(1, c*tau_i) = budget - |F|
   exactly in integers; r_i = min(1, c*tau_i) (eq. 3).
4. H = F plus the saturated tokens, L = the rest; Z_i ~ Bernoulli(r_i) is drawn
   from Philox4x32-10 keyed on (seed, layer, head, token) (reading R3).
5. The resident set H u S is listed in ascending position and its K/V rows are
   gathered into a compact cache (rows are K then V of one token).

Exactness: all sums are Python/numpy integers; r_i is one correctly rounded
float64 division of two integers below 2^53 followed by one round-to-nearest
conversion to float32, so the library can reproduce r bit for bit.
"""

import numpy as np

from .philox import uniform24

TAU_SCALE = 2 ** 32
ONE_MINUS_ULP = np.float32(1.0 - 2.0 ** -24)  # largest float32 below 1


def tau_fixed(tau):
    """tau in [0,1] -> integer grid value in [1, 2^32] (reading R1)."""
    t = np.asarray(tau, dtype=np.float32).astype(np.float64) * float(TAU_SCALE)
    t = np.floor(t)
    t = np.clip(t, 1.0, float(TAU_SCALE))
    return t.astype(np.int64)


def forced_mask(n, n_sink, n_local):
    """Sink tokens (first n_sink) and local tokens (last n_local) -> H."""
    m = np.zeros(n, dtype=bool)
    m[:min(n_sink, n)] = True
    if n_local > 0:
        m[max(0, n - n_local):] = True
    return m


def water_level(tq_free, b_free):
    """Saturation count j* and exact water level c = num/den (eq. 3).

    ``tq_free``: integer scores of the non-forced tokens; ``b_free``: budget
    left after the forced set. Sorting the scores in decreasing order, the
    top j tokens saturate (c*tau >= 1) and the rest get c*tau with
    c = (b_free - j) / T_j, T_j the sum of the unsaturated scores. j* is the
    smallest j for which the (j+1)-th score stays unsaturated:
    (b_free - j) * tau_(j+1) < T_j.

    Returns (j_star, num, den); den == 0 means every token saturates (c = inf).
    """
    tq = np.asarray(tq_free, dtype=np.int64)
    u = tq.size
    if b_free < 0:
        raise ValueError("budget smaller than the forced set")
    if b_free >= u:
        return u, 1, 0
    srt = np.sort(tq)[::-1]
    suffix = np.cumsum(srt[::-1])[::-1]          # suffix[j] = sum srt[j:]
    j = np.arange(u, dtype=np.int64)
    ok = (b_free - j) * srt < suffix
    j_star = int(np.argmax(ok))                  # first True (exists: j=b_free)
    assert ok[j_star]
    return j_star, int(b_free - j_star), int(suffix[j_star])


def rates(tq, forced, num, den):
    """r_i (float32) and the H mask from the exact water level num/den."""
    n = tq.size
    r = np.ones(n, dtype=np.float32)
    in_h = forced.copy()
    if den == 0:
        in_h[:] = True
        return r, in_h
    free = ~forced
    prod = tq[free].astype(np.int64) * np.int64(num)     # < 2^53, exact
    sat = prod >= den
    q = (prod.astype(np.float64) / float(den)).astype(np.float32)
    q = np.where(sat, np.float32(1.0), np.minimum(q, ONE_MINUS_ULP))
    r[free] = q
    in_h[free] = sat
    return r, in_h


def water_level_tau_units(num, den):
    """c in units of tau (not of the integer grid): num * 2^32 / den."""
    if den == 0:
        return float("inf")
    return float(num) * float(TAU_SCALE) / float(den)


def compress_slice(tau, budget, n_sink, n_local, seed, layer, head):
    """PoissonComp for one (layer, KV head) slice.

    Returns a dict with r (float32), in_h, in_l, in_s (bool masks),
    resident_idx (ascending int32), water level (num, den, c) and j*.
    """
    tau = np.asarray(tau, dtype=np.float32)
    n = tau.size
    tq = tau_fixed(tau)
    forced = forced_mask(n, n_sink, n_local)
    b_free = int(budget) - int(forced.sum())
    j_star, num, den = water_level(tq[~forced], b_free)
    r, in_h = rates(tq, forced, num, den)
    in_l = ~in_h
    u = uniform24(seed, np.arange(n, dtype=np.uint64), head, layer)
    z = u < r.astype(np.float64)
    in_s = in_l & z
    resident = in_h | in_s
    return dict(r=r, in_h=in_h, in_l=in_l, in_s=in_s,
                resident_idx=np.nonzero(resident)[0].astype(np.int32),
                num=num, den=den, j_star=j_star,
                c=water_level_tau_units(num, den), tq=tq, forced=forced)


def compress(tau, k, v, budget, n_sink, n_local, seed, layer0=0):
    """PoissonComp over [layers][kv_heads][n] scores with K/V [..][n][d].

    K/V may be any float arrays (typically bf16 values held as float32);
    resident rows are gathered as [count][2][d] (K row then V row).
    """
    tau = np.asarray(tau)
    n_layers, n_heads, n = tau.shape
    out = []
    for li in range(n_layers):
        row = []
        for g in range(n_heads):
            sl = compress_slice(tau[li, g], budget, n_sink, n_local, seed,
                                layer0 + li, g)
            idx = sl["resident_idx"]
            if k is not None:
                sl["resident_kv"] = np.stack([k[li, g][idx], v[li, g][idx]],
                                             axis=1)
            row.append(sl)
        out.append(row)
    return out
