"""GPU parity of the pages' 2-bit key sketch ("Verify Before You Fetch",
Appendix A.1 and section 5.1): the library's sketch build against the
oracle's, bit for bit, and the decode step planning with the 2-bit sketch
and the exact shortlist against the oracle (MI355X only)."""

import numpy as np
import pytest

from oracle import decode as od
from oracle import sketch2 as sk2
from tests import gpu_cases as gc
from workloads import CONFIGS, bf16_bits, bf16_to_f32, resident_cap

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

W2 = od.W_SKETCH2


# ---------------------------------------------------------------- build
def _check_build(keys_bits, got, key_view=lambda x: x):
    """keys_bits [S][n][d] (bf16 bits); got: the library's sketch."""
    S, n, _ = keys_bits.shape
    codes = got["codes"].reshape(S, n).view(np.uint64)
    zs = got["zs"].reshape(S, -1, 2, 32).view(np.uint16)
    chan = got["chan"].reshape(S, 32)
    ties = 0
    for i in range(S):
        keys = bf16_to_f32(keys_bits[i])
        sk = sk2.build(keys)
        lp = np.sort(chan[i, :16].astype(np.int64))
        assert np.array_equal(chan[i], sk2.kept_channels(lp, 128)), i
        if not np.array_equal(lp, sk["pairs"]):
            e = sk["energy"]
            e16 = np.sort(e)[::-1][15]
            diff = np.setxor1d(lp, sk["pairs"])
            assert np.all(np.abs(e[diff] - e16) <= gc.PAIR_TIE * e16), (i, diff)
            sk = sk2.with_pairs(keys, lp)
            ties += 1
        assert np.array_equal(zs[i, :, 0, :],
                              sk["zero"].astype(np.float16).view(np.uint16)), i
        assert np.array_equal(zs[i, :, 1, :],
                              sk["scale"].astype(np.float16).view(np.uint16)), i
        assert np.array_equal(sk2.unpack_codes(codes[i]), sk["codes"]), i
    return ties


def _profile_keys(seed, S, n, d=128, scale=1.0):
    rng = np.random.default_rng(seed)
    amp = np.exp(rng.normal(0, 0.7, (S, 1, d // 2)))
    amp = np.concatenate([amp, amp], axis=2)
    k = rng.standard_normal((S, n, d)).astype(np.float32) * amp * scale
    return bf16_bits(k.astype(np.float32))


@pytest.mark.parametrize("S,n", [(3, 1000), (2, 128), (1, 1), (1, 129), (4, 4096)])
def test_build_bitexact(S, n):
    """Kept channels, zero points, scales and codes bit for bit, including
    a one-token context and ragged last groups."""
    gc.say(f"sketch2 build S={S} n={n}")
    kb = _profile_keys(S * 1000 + n, S, n)
    got = vk.sketch2_build(torch.from_numpy(kb.view(np.int16)).to("cuda"))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items() if k != "_ws"}
    _check_build(kb, got)


def test_build_flat_and_wide_channels():
    """A constant channel in a group (scale 0, codes 0) and values beyond the
    fp16 range (zero point and scale saturate)."""
    gc.say("sketch2 build flat / wide")
    kb = _profile_keys(7, 1, 300)
    k = bf16_to_f32(kb)
    k[0, :128, :] = 1.25                 # group 0 constant in every channel
    k[0, 200, 5] = 3.0e5                 # a value beyond fp16's range
    k[0, 201, 5] = -2.0e5
    k[0, :, 5] *= 1.0                    # channel 5 keeps its energy
    kb = bf16_bits(k)
    got = vk.sketch2_build(torch.from_numpy(kb.view(np.int16)).to("cuda"))
    torch.cuda.synchronize()
    got = {x: v.cpu().numpy() for x, v in got.items() if x != "_ws"}
    _check_build(kb, got)


def test_build_interleaved_rows():
    """Keys read out of interleaved K/V rows (key_stride 2 d), as the decode
    tests pass the cache."""
    gc.say("sketch2 build interleaved")
    rng = np.random.default_rng(3)
    kv = bf16_bits(rng.standard_normal((2, 2, 700, 2, 128)).astype(np.float32))
    t = torch.from_numpy(kv.view(np.int16)).to("cuda").view(2, 2, 700, 256)
    got = vk.sketch2_build(t)
    torch.cuda.synchronize()
    got = {x: v.cpu().numpy() for x, v in got.items() if x != "_ws"}
    _check_build(kv[:, :, :, 0, :].reshape(4, 700, 128),
                 {k: v.reshape((4,) + v.shape[2:]) for k, v in got.items()})


# ---------------------------------------------------------------- decode
def _case(cfg, eps=None, est=0, n_short=128, cap=None, **kw):
    w = gc.build_case(cfg, cap=cap, pair_profile=True, **kw)
    eps = w["eps"] if eps is None else eps
    gc.say(f"decode sketch2 {cfg} B={w['B']} G={w['G']} Hq={w['Hq']} n={w['n']} "
           f"eps={eps} est={est} n_short={n_short}")
    dev = gc.device_inputs(w)
    gpu = gc.run_library(w, dev, eps, w["delta"], est, W2, n_short=n_short)
    heads, unions = gc.run_oracle(w, eps, w["delta"], est, W2, n_short=n_short,
                                  gpu=gpu)
    return w, gpu, heads, unions, eps


@pytest.mark.parametrize("n_short", [0, 16, 128, 1024])
def test_decode_c1(n_short):
    """The tiny layer with no shortlist, short ones, and one longer than the
    non-resident part of L (every planning weight then exact)."""
    w, gpu, heads, unions, eps = _case("c1", n_short=n_short)
    s = gc.compare(w, gpu, heads, unions, eps, weights=W2)
    gc.say(f"  {s}")
    assert s["ties"] == 0


@pytest.mark.parametrize("est", [1, 2])
def test_decode_c1_estimators(est):
    w, gpu, heads, unions, eps = _case("c1", est=est)
    s = gc.compare(w, gpu, heads, unions, eps, est=est, weights=W2)
    gc.say(f"  {s}")


@pytest.mark.parametrize("cfg,kw", [
    ("c2", dict(n=5000, G=2)),
    ("c3", dict(n=6000, G=2, B=4, seed=1, shift_from=2)),
    ("c4", dict(n=20000, G=2, B=2)),
])
def test_decode_reduced(cfg, kw):
    w, gpu, heads, unions, eps = _case(cfg, **kw)
    s = gc.compare(w, gpu, heads, unions, eps, weights=W2)
    gc.say(f"  {s}")
    assert s["fetched"] > 0 and s["short_keys"] > 0


@pytest.mark.parametrize("n,sink,local,budget", [
    (1, 64, 64, 129),        # L empty: nothing to shortlist
    (300, 4, 4, 40),
    (513, 4, 8, 60),
    (2049, 16, 16, 160),
])
def test_decode_short_and_ragged(n, sink, local, budget):
    def forced(w):
        w["n_sink"], w["n_local"], w["budget"] = sink, local, budget
    w, gpu, heads, unions, eps = _case("c2", n=n, G=2, B=2, mutate=forced)
    s = gc.compare(w, gpu, heads, unions, eps, weights=W2)
    gc.say(f"  {s}")


@pytest.mark.parametrize("grp", [1, 2, 8])
def test_decode_head_groups(grp):
    w, gpu, heads, unions, eps = _case("c2", n=4000, G=2, grp=grp)
    s = gc.compare(w, gpu, heads, unions, eps, weights=W2)
    gc.say(f"  {s}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_decode_full_size(cfg):
    """Every row at full size, with the benchmark's capacities."""
    p = CONFIGS[cfg]
    kw = dict(shift_from=p["shift_from"]) if "shift_from" in p else {}
    w, gpu, heads, unions, eps = _case(cfg, cap=resident_cap(p["budget"]), **kw)
    s = gc.compare(w, gpu, heads, unions, eps, weights=W2)
    gc.say(f"  {s}")
    assert s["fetched"] > 0


def test_decode_deterministic():
    """Two runs give identical bits in every output."""
    w = gc.build_case("c3", n=6000, G=2, B=4, seed=1, shift_from=2,
                      pair_profile=True)
    dev = gc.device_inputs(w)
    a = gc.run_library(w, dev, w["eps"], w["delta"], 0, W2)
    b = gc.run_library(w, dev, w["eps"], w["delta"], 0, W2)
    for k in ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
              "fetch_idx", "fetch_count", "host_bytes", "row_stats", "row_path",
              "shortlist"):
        assert np.array_equal(np.asarray(a[k]).view(np.uint8),
                              np.asarray(b[k]).view(np.uint8)), k
