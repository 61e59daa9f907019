"""Pins of the maintenance oracle ("Verify Before You Fetch", section 3 and
Appendix A.3.1-A.3.2): resident-list invariants after appends and the
staged-row accounting."""

import numpy as np
import pytest

from oracle import maintain as om
from tests import pins


@pytest.mark.parametrize("seed", [1, 2])
def test_append_invariants(seed):
    pins.check_append_invariants(seed)


@pytest.mark.parametrize("seed", [3, 4])
def test_staged_hits(seed):
    pins.check_staged_hits(seed)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], dtype=np.float32)
    got = om.bf16_rne(x)
    # halfway cases go to the even neighbour
    assert got[0] == 0x3F80 and got[1] == 0x3F82 and got[2] == 0xC020


def test_append_codes_and_groups():
    B, G, ns = 1, 2, 300
    st = dict(host_kv=np.zeros((B, G, ns, 2, 128), dtype=np.uint16),
              r=np.full((B, G, ns), 0.5, dtype=np.float32),
              res_idx=[[np.array([0, 5]), np.array([1])]],
              res_kv=[[np.zeros((2, 2, 128), np.uint16), np.zeros((1, 2, 128), np.uint16)]],
              codes=np.full((B, G, ns), 7, dtype=np.uint64),
              zs=np.full((B, G, 3, 2, 32), 9, dtype=np.uint16))
    kv = np.ones((B, G, 128), dtype=np.uint16)
    om.append_token(st, 256, kv, kv)
    assert np.all(st["codes"][:, :, 256] == 0) and np.all(st["zs"][:, :, 2] == 0)
    assert np.all(st["zs"][:, :, :2] == 9) and np.all(st["codes"][:, :, 255] == 7)
    om.append_token(st, 257, kv, kv)
    assert np.all(st["zs"][:, :, 2] == 0) and np.all(st["codes"][:, :, 257] == 0)
