"""Pins for the PoissonComp oracle (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import compress as oc
from oracle import philox
from tests import pins
from workloads import make_c5_tau

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tau_fixed_grid():
    t = np.array([0.0, 1.0, 0.5, 2.0 ** -33, 2.0 ** -32, 0.75], np.float32)
    assert oc.tau_fixed(t).tolist() == [1, 2 ** 32, 2 ** 31, 1, 1, 3 * 2 ** 30]


@pytest.mark.parametrize("seed", range(12))
def test_water_level_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    # include ties and wide dynamic range
    tq = rng.integers(1, 2 ** 20, size=n)
    if n > 3:
        tq[: n // 3] = tq[0]
    for b_free in sorted({0, 1, n // 4, n // 2, n - 1, n, n + 3}):
        if b_free < 0:
            continue
        pins.check_water_level_bruteforce(tq, b_free)


def test_water_level_golden():
    """Hand-worked example of eq. 3 (tests/golden/waterfill_small.json)."""
    with open(os.path.join(GOLDEN, "waterfill_small.json")) as f:
        g = json.load(f)
    sl = oc.compress_slice(np.array(g["tau"], np.float32), g["budget"],
                           g["n_sink"], g["n_local"], 0, 0, 0)
    assert sl["j_star"] == g["j_star"]
    assert abs(sl["c"] - g["c"]) <= 1e-15 * g["c"]
    assert sl["r"].tolist() == [float(np.float32(x)) for x in g["r"]]
    assert sl["in_h"].tolist() == g["in_h"]


@pytest.mark.parametrize("eta", [1 / 8, 1 / 16, 1 / 32])
def test_rates_sum_and_brentq(eta):
    tau = make_c5_tau(seed=0, layers=1, G=2, n=131072)
    for g in range(2):
        budget = int(round(eta * tau.shape[-1]))
        pins.check_rates_sum(tau[0, g], budget, 4, 256)
        pins.check_water_level_brentq(tau[0, g], budget, 4, 256)


def test_all_saturate_and_zero_scores():
    tau = np.zeros(100, np.float32)
    sl = oc.compress_slice(tau, 100, 2, 2, 1, 0, 0)
    assert np.all(sl["r"] == 1) and sl["den"] == 0 and np.isinf(sl["c"])
    sl = oc.compress_slice(tau, 10, 2, 2, 1, 0, 0)  # all-zero scores: R1 floor
    assert np.all(sl["r"][~sl["forced"]] == np.float32(6 / 96))
    pins.check_rates_sum(tau, 10, 2, 2)
    with pytest.raises(ValueError):
        oc.compress_slice(tau, 3, 2, 2, 1, 0, 0)


def test_philox_uniformity_and_avalanche():
    n = 1 << 20
    u = philox.uniform24(12345, np.arange(n, dtype=np.uint64), 3, 7)
    hist = np.histogram(u, bins=64, range=(0, 1))[0]
    exp = n / 64
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert chi2 < 63 + 6 * np.sqrt(2 * 63)  # ~6 sigma
    assert abs(u.mean() - 0.5) < 6 * np.sqrt(1 / 12 / n)
    # lag-1 serial correlation
    c = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(c) < 6 / np.sqrt(n)
    # flipping one counter bit changes about half of the 128 output bits
    base = np.array(philox.philox4x32_10(np.arange(4096), 5, 9, 0, 77, 88))
    flip = np.array(philox.philox4x32_10(np.arange(4096) ^ 1, 5, 9, 0, 77, 88))
    x = base ^ flip
    bits = sum(int(bin(int(v)).count("1")) for v in x.ravel())
    frac = bits / (4096 * 128)
    assert abs(frac - 0.5) < 0.01
    # a bijection on counters: no collisions among 2^16 counters
    words = np.array(philox.philox4x32_10(np.arange(1 << 16), 0, 0, 0, 1, 2))
    assert len({tuple(col) for col in words.T}) == 1 << 16


def test_bernoulli_frequencies():
    """Per-token inclusion frequency over many seeds matches r_i; the sample
    size has mean sum_L r and variance sum_L r (1 - r) (independence)."""
    rng = np.random.default_rng(3)
    tau = rng.beta(0.5, 5, size=400).astype(np.float32)
    n_seeds = 4000
    sl0 = oc.compress_slice(tau, 60, 2, 8, 0, 4, 1)
    r = sl0["r"].astype(np.float64)
    lmask = sl0["in_l"]
    counts = np.zeros(tau.size)
    sizes = []
    for s in range(n_seeds):
        u = philox.uniform24(s, np.arange(tau.size, dtype=np.uint64), 1, 4)
        z = (u < r) & lmask
        counts += z
        sizes.append(int(z.sum()))
    freq = counts / n_seeds
    sd = np.sqrt(r * (1 - r) / n_seeds)
    assert np.all(np.abs(freq - r)[lmask] <= 5 * sd[lmask] + 1e-12)
    mu = float(np.sum(r[lmask]))
    var = float(np.sum(r[lmask] * (1 - r[lmask])))
    sizes = np.array(sizes)
    assert abs(sizes.mean() - mu) < 5 * np.sqrt(var / n_seeds)
    assert abs(sizes.var() / var - 1) < 0.15


def test_compress_layout():
    rng = np.random.default_rng(0)
    tau = rng.random((2, 3, 300)).astype(np.float32)
    k = rng.standard_normal((2, 3, 300, 8)).astype(np.float32)
    v = rng.standard_normal((2, 3, 300, 8)).astype(np.float32)
    out = oc.compress(tau, k, v, 40, 3, 5, seed=9, layer0=4)
    for li in range(2):
        for g in range(3):
            sl = out[li][g]
            idx = sl["resident_idx"]
            assert np.all(np.diff(idx) > 0)
            res = sl["in_h"] | sl["in_s"]
            assert np.array_equal(np.nonzero(res)[0], idx)
            assert np.array_equal(sl["resident_kv"][:, 0], k[li, g][idx])
            assert np.array_equal(sl["resident_kv"][:, 1], v[li, g][idx])
    # the sample depends on (seed, layer, head, token) only
    again = oc.compress_slice(tau[1, 2], 40, 3, 5, 9, 5, 2)
    assert np.array_equal(again["resident_idx"], out[1][2]["resident_idx"])


def test_philox_known_answer_vectors():
    """The three published Philox4x32-10 known-answer vectors (Salmon et
    al., SC'11), held in tests/golden/philox_kat.json."""
    pins.check_philox_kat()
