"""GPU parity of the Dense baselines (exact whole-cache attention, eq. 1)
against the oracle, with the cache in device memory (Dense resident) and in
pinned host memory (Dense offload). Tolerances: o within 1e-3 relative L2 and
D within 1e-4 relative, as for the verified path."""

import numpy as np
import pytest

from oracle import decode as od
from tests import gpu_cases as gc
from workloads import bf16_bits, bf16_to_f32, make_decode_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402


def _run(q_bits, kv_bits, where):
    B, Hq, _ = q_bits.shape
    _, G, n, _, _ = kv_bits.shape
    dev = torch.device("cuda")
    tq = torch.from_numpy(q_bits.view(np.int16)).to(dev)
    tkv = torch.from_numpy(kv_bits.view(np.int16))
    tkv = tkv.to(dev) if where == "device" else tkv.pin_memory()
    run = vk.DenseAttention(B, Hq, G, n, dev).bind(tq, tkv)
    out = run.launch()
    torch.cuda.synchronize()
    return out["out"].cpu().numpy(), out["log_d"].cpu().numpy()


def _compare(q_bits, kv_bits, where):
    gc.say(f"dense {where} q {q_bits.shape} kv {kv_bits.shape}")
    o_g, l_g = _run(q_bits, kv_bits, where)
    o_o, l_o = od.dense_step(bf16_to_f32(q_bits), bf16_to_f32(kv_bits))
    B, Hq, _ = q_bits.shape
    worst_o = worst_d = 0.0
    for b in range(B):
        for h in range(Hq):
            eo = float(np.linalg.norm(o_g[b, h] - o_o[b, h]) /
                       np.linalg.norm(o_o[b, h]))
            ed = abs(float(np.expm1(float(l_g[b, h]) - l_o[b, h])))
            worst_o, worst_d = max(worst_o, eo), max(worst_d, ed)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(l_g))
    gc.say(f"  worst o {worst_o:.2e} D {worst_d:.2e}")
    assert worst_o <= gc.TOL_O and worst_d <= gc.TOL_D, (worst_o, worst_d)


def _random(B, Hq, G, n, seed, spread=1.0):
    rng = np.random.default_rng([77, seed])
    q = bf16_bits(rng.standard_normal((B, Hq, 128), dtype=np.float32) * spread)
    kv = bf16_bits(rng.standard_normal((B, G, n, 2, 128), dtype=np.float32))
    return q, kv


@pytest.mark.parametrize("where", ["device", "host"])
@pytest.mark.parametrize("n", [1, 7, 255, 257, 5000])
def test_dense_ragged_lengths(where, n):
    q, kv = _random(2, 8, 2, n, n)
    _compare(q, kv, where)


@pytest.mark.parametrize("grp", [1, 2, 8])
def test_dense_head_groups(grp):
    q, kv = _random(1, 2 * grp, 2, 3000, grp, spread=3.0)
    _compare(q, kv, "device")


@pytest.mark.parametrize("where", ["device", "host"])
def test_dense_c2_full(where):
    """Every query head of the 32K decode layer (heavy-tailed keys)."""
    w = make_decode_workload("c2", seed=0, with_queries=True)
    _compare(w["q"], w["host_kv"], where)


def test_dense_c4_one_request():
    """One request of the 128K layer, cache in pinned host memory."""
    w = make_decode_workload("c4", seed=0, with_queries=True, B=1)
    _compare(w["q"], w["host_kv"], "host")


def test_dense_pageable_rejected():
    q, kv = _random(1, 4, 1, 100, 3)
    dev = torch.device("cuda")
    tq = torch.from_numpy(q.view(np.int16)).to(dev)
    tkv = torch.from_numpy(kv.view(np.int16))  # pageable host memory
    run = vk.DenseAttention(1, 4, 1, 100, dev)
    run.args.q, run.args.kv = vk._ptr(tq), vk._ptr(tkv)
    rc = vk.vkv_dense_attention(run.args, vk._stream(None))
    assert rc == vk.VKV_ENOTPINNED, (rc, vk.vkv_last_error())
