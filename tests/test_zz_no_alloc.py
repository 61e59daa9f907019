"""vkv_decode_step_noalloc against vkv_decode_step through the C ABI: the
same kernels with the workspace in the library's own device buffer, so
every output must be bit-identical; two calls in a row, the second on a
smaller input (the buffer keeps the first call's contents), and the
smaller case also checked against the oracle."""

import numpy as np
import pytest

from tests import gpu_cases as gc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

KEYS = ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
        "fetch_count", "host_bytes", "row_stats", "row_path")


def _both(w, eps):
    dev = gc.device_inputs(w)
    ref = gc.run_library(w, dev, eps, w["delta"])
    step = vk.DecodeStep(w["B"], w["Hq"], w["G"], w["n"], w["s"], w["cap"],
                         w["n"], torch.device("cuda"))
    step.bind(dev["q"], dev["resident_kv"], dev["resident_idx"],
              dev["resident_count"], dev["sketch"], dev["proj"], dev["r"],
              dev["host_kv"], eps, w["delta"])
    step.args.workspace = None
    step.args.workspace_bytes = 0
    rc = vk.vkv_decode_step_noalloc(step.args, vk._stream(None))
    assert rc == vk.VKV_OK, vk.vkv_last_error()
    rc, bits = step.check_status()
    got = {k: v.cpu().numpy() for k, v in step.out.items()}
    got["rc"], got["bits"] = rc, bits
    return ref, got


def _same(ref, got, w):
    assert ref["rc"] == got["rc"] == 0
    for k in KEYS:
        assert ref[k].tobytes() == got[k].tobytes(), k
    for b in range(w["B"]):
        for g in range(w["G"]):
            c = int(ref["fetch_count"][b, g])
            assert np.array_equal(ref["fetch_idx"][b, g, :c],
                                  got["fetch_idx"][b, g, :c])


def test_noalloc_matches_decode_step_twice_smaller_second():
    from workloads import CONFIGS, resident_cap
    gc.say("noalloc: full 32K layer, then a smaller one")
    w1 = gc.build_case("c2", cap=resident_cap(CONFIGS["c2"]["budget"]))
    ref1, got1 = _both(w1, w1["eps"])
    _same(ref1, got1, w1)
    assert int(got1["host_bytes"][0]) > 0
    w2 = gc.build_case("c2", n=5000, G=2, seed=3)
    ref2, got2 = _both(w2, w2["eps"])
    _same(ref2, got2, w2)
    heads, unions = gc.run_oracle(w2, w2["eps"], w2["delta"])
    gc.compare(w2, got2, heads, unions, w2["eps"])


def test_noalloc_rejects_a_workspace_and_oversized_shapes():
    gc.say("noalloc: argument checks")
    a = vk.DecodeArgs(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
                      n_tokens=32768, sketch_dim=32, cap=4700, eps=0.05,
                      delta=0.05, estimator=0, weights=0, fetch_cap=32768)
    fake = vk.ctypes.c_void_p(0x1000)
    for f in ("q", "resident_kv", "resident_idx", "resident_count", "sketch",
              "proj", "r", "host_kv", "out", "d_hat", "log_shift", "eps_hat0",
              "eps_hat", "k_star", "fetch_idx", "fetch_count", "host_bytes",
              "status"):
        setattr(a, f, fake)
    assert vk.vkv_decode_workspace_bytes(a) > vk.NOALLOC_WORKSPACE_BYTES
    assert vk.vkv_decode_step_noalloc(a, None) == vk.VKV_EUNSUPPORTED
    assert "buffer" in vk.vkv_last_error()
    a.batch = 1
    a.workspace, a.workspace_bytes = fake, 1 << 20
    assert vk.vkv_decode_step_noalloc(a, None) == vk.VKV_EINVAL
