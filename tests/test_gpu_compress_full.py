"""PoissonComp at the full size that bench.py times: one launch over the c5
model cache (36 layers x 8 KV heads x 131072 tokens, K and V in HBM), with
sampled slices compared bit for bit against the oracle: r, the ascending
resident list, its count, the water level and the gathered K/V rows."""

import numpy as np
import pytest

from oracle import compress as oc
from tests import gpu_cases as gc
from workloads import C5, make_c5_tau, resident_cap

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

SAMPLES = [(0, 0), (7, 3), (21, 6), (35, 7)]  # (layer, KV head)


@pytest.mark.parametrize("eta", [1 / 8, 1 / 32])
def test_compress_full_c5_sampled_slices(eta):
    L, G, n = C5["layers"], C5["G"], C5["n"]
    gc.say(f"compress full c5 eta={eta}")
    dev = torch.device("cuda")
    tau = make_c5_tau(seed=0)
    t_tau = torch.from_numpy(tau).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    k, v = [torch.randn((L, G, n, 128), dtype=torch.bfloat16, device=dev,
                        generator=gen).view(torch.int16) for _ in range(2)]
    budget = int(round(eta * n))
    cap = resident_cap(budget)
    seed = 3
    out = vk.compress(t_tau, k, v, budget, C5["n_sink"], C5["n_local"], seed,
                      cap)
    rc, bits = vk.vkv_check_status(vk._ptr(out["status"]), vk._stream(None))
    assert rc == 0, (rc, bits, vk.vkv_last_error())
    for li, hh in SAMPLES:
        sl = oc.compress_slice(tau[li, hh], budget, C5["n_sink"],
                               C5["n_local"], seed, li, hh)
        r = out["r"][li, hh].cpu().numpy()
        assert np.array_equal(r.view(np.uint32), sl["r"].view(np.uint32)), (li, hh)
        idx = sl["resident_idx"]
        cnt = int(out["resident_count"][li, hh].item())
        assert cnt == idx.size and cnt <= cap, (li, hh, cnt, idx.size)
        assert np.array_equal(out["resident_idx"][li, hh, :cnt].cpu().numpy(), idx)
        wl = float(out["water_level"][li, hh].item())
        assert (np.isinf(wl) and np.isinf(sl["c"])) or \
            np.float64(wl).view(np.uint64) == np.float64(sl["c"]).view(np.uint64), \
            (li, hh, wl, sl["c"])
        pos = torch.from_numpy(idx.astype(np.int64)).to(dev)
        rkv = out["resident_kv"][li, hh, :cnt]
        assert torch.equal(rkv[:, 0], k[li, hh].index_select(0, pos))
        assert torch.equal(rkv[:, 1], v[li, hh].index_select(0, pos))
    del out, k, v, t_tau
    torch.cuda.empty_cache()
