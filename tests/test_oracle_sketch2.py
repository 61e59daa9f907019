"""Pins of the 2-bit sketch oracle ("Verify Before You Fetch", Appendix A.1
and section 5.1): quantisation closed form, error bound, the RoPE-pair
choice, the 1.76% cost figure, the logit scale and channel mapping, the
shortlist against a plain sort, and the plan with a shortlist that covers L."""

import numpy as np
import pytest

from oracle import decode as od
from oracle import sketch2 as sk2
from tests import pins


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_levels_stored_without_loss(seed):
    pins.check_sketch2_levels(seed, n=300 + 37 * seed)


@pytest.mark.parametrize("seed", [4, 5])
def test_quantisation_error_bound(seed):
    pins.check_sketch2_error(seed)


@pytest.mark.parametrize("seed", [6, 7])
def test_pair_choice_rotation_invariant(seed):
    pins.check_sketch2_rotation(seed)


def test_cost_figure():
    pins.check_sketch2_cost()


@pytest.mark.parametrize("seed", [8, 9])
def test_logit_identity(seed):
    pins.check_sketch2_logit_identity(seed)


@pytest.mark.parametrize("seed", [10, 11])
def test_shortlist_bruteforce(seed):
    pins.check_shortlist_bruteforce(seed)


@pytest.mark.parametrize("seed", [12, 13, 14])
def test_full_shortlist_is_perfect_plan(seed):
    pins.check_sketch2_full_shortlist(seed)


def test_pack_roundtrip():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, (100, 32)).astype(np.uint8)
    words = sk2.pack_codes(codes)
    assert words.dtype == np.uint64
    assert np.array_equal(sk2.unpack_codes(words), codes)
    # slot c in bits 2c, 2c + 1
    one = np.zeros((1, 32), dtype=np.uint8)
    one[0, 5] = 3
    assert int(sk2.pack_codes(one)[0]) == 3 << 10


def test_flat_group_and_ragged_tail():
    """A constant channel has scale 0 and code 0; a ragged last group is
    quantised over its own tokens."""
    rng = np.random.default_rng(1)
    n = 128 + 5
    keys = rng.standard_normal((n, 128)).astype(np.float32)
    keys[:, :] *= np.where(np.arange(128) % 64 < 16, 4.0, 0.1).astype(np.float32)
    keys[:128, 0] = 1.5
    sk = sk2.build(keys)
    c0 = int(np.nonzero(sk["chan"] == 0)[0][0])
    assert sk["scale"][0, c0] == 0 and sk["zero"][0, c0] == 1.5
    assert np.all(sk["codes"][:128, c0] == 0)
    tail = keys[128:][:, sk["chan"]]
    z, s, c = sk2.quantize_group(tail)
    assert np.array_equal(sk["zero"][1], z) and np.array_equal(sk["codes"][128:], c)


def test_saturation():
    """Zero point and scale saturate at the largest finite fp16."""
    v = np.array([[-1e6], [0.0], [1e6]], dtype=np.float32)
    z, s, c = sk2.quantize_group(v)
    assert z[0] == -sk2.FP16_MAX and s[0] == sk2.FP16_MAX
    assert list(c[:, 0]) == [0, 1, 3]


def test_shortlist_excludes_resident():
    t = pins.tiny_layer(20, d=128, n_h=8, n_l=200, grp=4)
    rng = np.random.default_rng(21)
    samp = t["l_pos"][rng.random(t["l_pos"].size) < t["r"][t["l_pos"]]]
    res_idx = np.sort(np.concatenate([t["h_pos"], samp]))
    sk = sk2.build(t["K"].astype(np.float32))
    heads, _ = od.decode_group(t["q"], t["host_kv"][res_idx], res_idx, None,
                               None, t["r"], t["host_kv"], 0.05, 0.1,
                               od.EST_CLIP, od.W_SKETCH2, sketch2=sk, n_short=16)
    sl = heads[0]["shortlist"]
    assert sl.size == 16 and np.all(np.diff(sl) > 0)
    assert not np.any(np.isin(sl, res_idx))
    assert all(np.array_equal(h["shortlist"], sl) for h in heads)
    # the shortlist holds the largest fp32 scores among the eligible tokens
    s32 = np.array([sk2.sketch_logits(q, sk) for q in t["q"]]).astype(np.float32)
    best = s32.max(axis=0)
    elig = np.ones(t["n"], dtype=bool)
    elig[res_idx] = False
    rest = np.setdiff1d(np.nonzero(elig)[0], sl)
    assert best[sl].min() >= best[rest].max()
