"""GPU parity: the HIP library against the CPU oracle on identical seeded
inputs (MI355X only)."""

import math

import numpy as np
import pytest

from oracle import compress as oc
from oracle import decode as od
from tests import gpu_cases as gc
from workloads import (CONFIGS, bf16_bits, bf16_to_f32, make_c5_tau,
                       make_decode_workload, resident_cap)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402


# ---------------------------------------------------------------- compress
def _compress_both(tau, budget, n_sink, n_local, seed, cap, layer0=0,
                   with_kv=True, d=128):
    Ly, G, n = tau.shape
    rng = np.random.default_rng(seed + 17)
    kb = bf16_bits(rng.standard_normal((Ly, G, n, d), dtype=np.float32)) \
        if with_kv else None
    vb = bf16_bits(rng.standard_normal((Ly, G, n, d), dtype=np.float32)) \
        if with_kv else None
    dev = torch.device("cuda")
    t_tau = torch.from_numpy(tau).to(dev)
    t_k = torch.from_numpy(kb.view(np.int16)).to(dev) if with_kv else None
    t_v = torch.from_numpy(vb.view(np.int16)).to(dev) if with_kv else None
    out = vk.compress(t_tau, t_k, t_v, budget, n_sink, n_local, seed, cap,
                      layer0=layer0, with_kv=with_kv)
    rc, bits = vk.vkv_check_status(vk._ptr(out["status"]), vk._stream(None))
    g = {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()
         if k not in ("workspace", "_args")}
    g["rc"], g["bits"] = rc, bits
    orc = oc.compress(tau, None, None, budget, n_sink, n_local, seed, layer0)
    return g, orc, kb, vb


def _check_compress(g, orc, kb, vb, cap):
    Ly, G = g["resident_count"].shape
    for li in range(Ly):
        for hh in range(G):
            sl = orc[li][hh]
            assert np.array_equal(g["r"][li, hh].view(np.uint32),
                                  sl["r"].view(np.uint32)), (li, hh)
            idx = sl["resident_idx"]
            assert g["resident_count"][li, hh] == idx.size
            m = min(idx.size, cap)
            assert np.array_equal(g["resident_idx"][li, hh, :m], idx[:m])
            wl = g["water_level"][li, hh]
            assert (np.isinf(wl) and np.isinf(sl["c"])) or \
                np.float64(wl).view(np.uint64) == np.float64(sl["c"]).view(np.uint64), \
                (wl, sl["c"])
            if kb is not None:
                rk = g["resident_kv"][li, hh, :m].view(np.uint16)
                assert np.array_equal(rk[:, 0], kb[li, hh, idx[:m]])
                assert np.array_equal(rk[:, 1], vb[li, hh, idx[:m]])


def test_compress_c1_bitexact():
    gc.say("compress c1")
    w = gc.build_case("c1")
    tau = w["tau"]
    cap = 400
    g, orc, kb, vb = _compress_both(tau, w["budget"], w["n_sink"],
                                    w["n_local"], 0, cap)
    assert g["rc"] == 0
    _check_compress(g, orc, kb, vb, cap)


@pytest.mark.parametrize("eta", [1 / 8, 1 / 16, 1 / 32])
def test_compress_c5_slices_bitexact(eta):
    """Full-length c5 slices (n = 131072), 2 layers x 8 KV heads."""
    gc.say(f"compress c5 slices eta={eta}")
    tau = make_c5_tau(seed=0, layers=2, G=8)
    budget = int(round(eta * tau.shape[-1]))
    cap = budget + 1024
    g, orc, kb, vb = _compress_both(tau, budget, 4, 256, 7, cap, layer0=5,
                                    with_kv=(eta == 1 / 32))
    assert g["rc"] == 0
    _check_compress(g, orc, kb, vb, cap)
    # sum r = budget (float)
    assert np.allclose(g["r"].astype(np.float64).sum(-1), budget, rtol=1e-6)


@pytest.mark.parametrize("n,budget,sink,local", [
    (1, 1, 1, 0),          # single forced token
    (37, 37, 2, 3),        # budget covers everything: L empty
    (5000, 200, 0, 0),     # no forced tokens, ragged chunk
    (4097, 40, 30, 5),     # tiny free budget
    (9000, 2000, 100, 100),
])
def test_compress_edge_cases(n, budget, sink, local):
    gc.say(f"compress edge n={n} budget={budget}")
    rng = np.random.default_rng(n)
    tau = rng.beta(0.5, 5, size=(1, 2, n)).astype(np.float32)
    tau[0, 1, : n // 3] = 0.0          # zero scores (floored to the grid)
    tau[0, 1, n // 3: n // 2] = 1.0    # saturated scores
    cap = max(budget + 256, 8)
    g, orc, kb, vb = _compress_both(tau, budget, sink, local, 3, cap)
    assert g["rc"] == 0
    _check_compress(g, orc, kb, vb, cap)


def test_compress_cap_overflow_reported():
    gc.say("compress cap overflow")
    tau = make_c5_tau(seed=1, layers=1, G=1, n=8192)
    g, orc, _, _ = _compress_both(tau, 1024, 4, 64, 1, 100, with_kv=False)
    assert g["rc"] == vk.VKV_EOVERFLOW
    assert g["bits"] & vk.STATUS_RESIDENT_OVERFLOW
    sl = orc[0][0]
    assert g["resident_count"][0, 0] == sl["resident_idx"].size
    assert np.array_equal(g["resident_idx"][0, 0], sl["resident_idx"][:100])


# ---------------------------------------------------------------- decode
def _decode_case(cfg, eps=None, est=0, weights=0, seed=0, fetch_cap=None,
                 **kw):
    w = gc.build_case(cfg, seed=seed, **kw)
    eps = w["eps"] if eps is None else eps
    gc.say(f"decode {cfg} B={w['B']} G={w['G']} Hq={w['Hq']} n={w['n']} "
           f"eps={eps} est={est} weights={weights}")
    dev = gc.device_inputs(w)
    gpu = gc.run_library(w, dev, eps, w["delta"], est, weights, fetch_cap)
    heads, unions = gc.run_oracle(w, eps, w["delta"], est, weights)
    return w, gpu, heads, unions, eps


@pytest.mark.parametrize("weights", [0, 1])
def test_decode_c1(weights):
    w, gpu, heads, unions, eps = _decode_case("c1", weights=weights)
    s = gc.compare(w, gpu, heads, unions, eps, weights=weights)
    gc.say(f"  {s}")
    assert s["ties"] == 0  # the tiny case must match exactly


@pytest.mark.parametrize("weights", [0, 1])
def test_decode_c1_unbiased(weights):
    w, gpu, heads, unions, eps = _decode_case("c1", est=1, weights=weights)
    s = gc.compare(w, gpu, heads, unions, eps, est=1, weights=weights)
    gc.say(f"  {s}")


@pytest.mark.parametrize("weights", [0, 1])
def test_decode_c1_binary(weights):
    w, gpu, heads, unions, eps = _decode_case("c1", est=2, weights=weights)
    s = gc.compare(w, gpu, heads, unions, eps, est=2, weights=weights)
    gc.say(f"  {s}")
    assert s["ties"] == 0


@pytest.mark.parametrize("cfg,kw", [
    ("c2", dict(n=5000, G=2)),
    ("c3", dict(n=6000, G=2, B=4, seed=1, shift_from=2)),
    ("c4", dict(n=20000, G=2, B=2)),
])
def test_decode_binary_reduced(cfg, kw):
    """Binary shrinkage (lambda in {1, r}) on reduced shapes of each layer."""
    w, gpu, heads, unions, eps = _decode_case(cfg, est=2, **kw)
    s = gc.compare(w, gpu, heads, unions, eps, est=2)
    gc.say(f"  {s}")
    assert s["fetched"] > 0


def _uniform_planning(w):
    # every sketch row of a KV head equal and tau constant: every token of L
    # has the same planning weight and inclusion probability, so the binary
    # order and the gain order are decided by position alone
    w["sketch"][...] = w["sketch"][:, :, :1, :]
    w["tau"][...] = np.float32(0.5)


@pytest.mark.parametrize("est", [0, 2])
def test_decode_uniform_planning_weights(est):
    """The degenerate case of all-equal keys of the order: positions break
    every tie, on both sides."""
    w, gpu, heads, unions, eps = _decode_case("c2", est=est, n=3000, G=1,
                                              mutate=_uniform_planning)
    s = gc.compare(w, gpu, heads, unions, eps, est=est)
    gc.say(f"  {s}")


def _forced(n_sink, n_local, budget):
    def f(w):
        w["n_sink"], w["n_local"], w["budget"] = n_sink, n_local, budget
    return f


@pytest.mark.parametrize("n,sink,local,budget,est", [
    (1, 64, 64, 129, 0),       # one token, forced: L empty
    (100, 64, 64, 129, 0),     # every token forced: L empty
    (300, 4, 4, 40, 0),        # a short context
    (300, 4, 4, 40, 2),
    (513, 4, 8, 60, 0),        # one token past a scan chunk
    (2049, 16, 16, 160, 0),    # one token past a row sub-chunk
    (2049, 16, 16, 160, 2),
])
def test_decode_short_and_ragged_contexts(n, sink, local, budget, est):
    """Contexts shorter than a chunk or one token past one, and the empty L
    of a fully forced context (then nothing is estimated or fetched and the
    output is exact attention)."""
    w, gpu, heads, unions, eps = _decode_case("c2", est=est, n=n, G=2, B=2,
                                              mutate=_forced(sink, local, budget))
    s_ = gc.compare(w, gpu, heads, unions, eps, est=est)
    gc.say(f"  {s_}")
    if sink + local >= n:
        assert s_["fetched"] == 0 and np.all(gpu["eps_hat0"] == 0.0)
        for b in range(w["B"]):
            for h in range(w["Hq"]):
                kv = bf16_to_f32(w["host_kv"][b, h // (w["Hq"] // w["G"])])
                o_ref, _ = od.exact_attention(bf16_to_f32(w["q"][b, h]),
                                              kv[:, 0], kv[:, 1])
                err = np.linalg.norm(gpu["out"][b, h] - o_ref) / np.linalg.norm(o_ref)
                assert err <= gc.TOL_O, (b, h, err)


def test_decode_three_kv_heads_three_requests():
    """Request and KV-head counts that are not powers of two."""
    w, gpu, heads, unions, eps = _decode_case("c2", n=3000, G=3, B=3)
    s_ = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s_}")


def test_decode_c2_reduced():
    w, gpu, heads, unions, eps = _decode_case("c2", n=5000, G=2)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")
    assert s["fetched"] > 0


def test_decode_c3_reduced():
    w, gpu, heads, unions, eps = _decode_case("c3", n=6000, G=2, B=4,
                                              seed=1, shift_from=2)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")


def test_decode_c4_reduced():
    w, gpu, heads, unions, eps = _decode_case("c4", n=20000, G=2, B=2)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_decode_full_size(cfg):
    """Every row at the configuration's full size, with the resident capacity
    and fetch capacity the benchmark uses (so the same launch shapes)."""
    p = CONFIGS[cfg]
    kw = dict(shift_from=p["shift_from"]) if "shift_from" in p else {}
    w, gpu, heads, unions, eps = _decode_case(
        cfg, cap=resident_cap(p["budget"]), **kw)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")
    assert s["fetched"] > 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", ["c2", "c4"])
def test_decode_binary_full_size(cfg):
    """Binary shrinkage at full size, in the benchmark's launch shapes."""
    p = CONFIGS[cfg]
    w, gpu, heads, unions, eps = _decode_case(
        cfg, est=2, cap=resident_cap(p["budget"]))
    s = gc.compare(w, gpu, heads, unions, eps, est=2)
    gc.say(f"  {s}")
    assert s["fetched"] > 0


@pytest.mark.parametrize("grp,s", [(1, 32), (2, 32), (8, 32), (4, 16), (8, 16)])
def test_decode_head_groups_and_sketch_dims(grp, s):
    """Every supported query-heads-per-KV-head count and sketch width (the
    kernels are instantiated per pair)."""
    w, gpu, heads, unions, eps = _decode_case("c2", n=4000, G=2, grp=grp, s=s)
    st = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {st}")
    assert st["fetched"] > 0


def test_decode_fetch_all_is_exact_attention():
    """eps -> 0: every L token is fetched and the output is exact attention."""
    w, gpu, heads, unions, eps = _decode_case("c2", eps=1e-30, n=3000, G=1)
    s = gc.compare(w, gpu, heads, unions, eps)
    for h in range(w["Hq"]):
        kv = bf16_to_f32(w["host_kv"][0, 0])
        o_ref, logd = od.exact_attention(bf16_to_f32(w["q"][0, h]), kv[:, 0],
                                         kv[:, 1])
        o = gpu["out"][0, h].astype(np.float64)
        assert np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref) < 1e-3
    assert s["fetched"] > 0


def test_decode_no_fetch_large_eps():
    w, gpu, heads, unions, eps = _decode_case("c2", eps=1e6, n=3000, G=2)
    s = gc.compare(w, gpu, heads, unions, eps)
    assert s["fetched"] == 0 and np.all(gpu["k_star"] == 0)


def test_decode_fetch_cap_overflow_reported():
    w = gc.build_case("c2", n=3000, G=1)
    dev = gc.device_inputs(w)
    gc.say("decode fetch_cap overflow")
    gpu = gc.run_library(w, dev, 1e-30, w["delta"], fetch_cap=16)
    assert gpu["rc"] == vk.VKV_EOVERFLOW
    assert gpu["bits"] & vk.STATUS_FETCH_OVERFLOW
    assert int(gpu["host_bytes"][0]) == 16 * 512


def test_decode_not_pinned_rejected():
    gc.say("decode with pageable host_kv")
    w = gc.build_case("c1")
    dev = gc.device_inputs(w)
    step = vk.DecodeStep(1, 1, 1, w["n"], w["s"], w["cap"], w["n"],
                         torch.device("cuda"))
    step.bind(dev["q"], dev["resident_kv"], dev["resident_idx"],
              dev["resident_count"], dev["sketch"], dev["proj"], dev["r"],
              dev["host_kv"], 0.1, 0.05)
    pageable = torch.from_numpy(w["host_kv"].view(np.int16).copy())
    step.args.host_kv = vk._ptr(pageable)
    assert vk.vkv_decode_step(step.args, vk._stream(None)) == vk.VKV_ENOTPINNED
    assert "pinned" in vk.vkv_last_error()


def test_decode_bad_resident_list_reported():
    w = gc.build_case("c1")
    dev = gc.device_inputs(w)
    dev["resident_idx"][0, 0, 5] = dev["resident_idx"][0, 0, 4]  # not ascending
    gpu = gc.run_library(w, dev, 0.1, w["delta"])
    assert gpu["rc"] == vk.VKV_EDATA
    assert gpu["bits"] & vk.STATUS_BAD_RESIDENT


def test_decode_bad_r_reported():
    w = gc.build_case("c1")
    dev = gc.device_inputs(w)
    dev["r"][0, 0, 700] = 0.0  # outside (0, 1]
    gc.say("decode with r = 0 at one token")
    gpu = gc.run_library(w, dev, 0.1, w["delta"])
    assert gpu["rc"] == vk.VKV_EDATA
    assert gpu["bits"] & vk.STATUS_BAD_R


@pytest.mark.parametrize("cfg,kw", [
    ("c2", dict(n=4000, G=2)),
    ("c3", dict(n=6000, G=2, B=4, seed=1, shift_from=2)),
])
@pytest.mark.parametrize("est", [0, 2])
def test_decode_deterministic(cfg, kw, est):
    """Two runs of the same step give bit-identical outputs: every reduction
    runs in a fixed order and no result depends on the scheduling of
    workgroups (no float atomics)."""
    w = gc.build_case(cfg, **kw)
    dev = gc.device_inputs(w)
    gc.say(f"decode determinism {cfg} est={est}")
    a = gc.run_library(w, dev, w["eps"], w["delta"], est)
    b = gc.run_library(w, dev, w["eps"], w["delta"], est)
    assert a["rc"] == b["rc"] == 0
    for key in ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
                "fetch_count", "host_bytes", "row_stats", "row_path"):
        assert a[key].tobytes() == b[key].tobytes(), key
    for bb in range(w["B"]):
        for g in range(w["G"]):
            c = int(a["fetch_count"][bb, g])
            assert np.array_equal(a["fetch_idx"][bb, g, :c],
                                  b["fetch_idx"][bb, g, :c])
    assert int(a["host_bytes"][0]) > 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("eps", [1e-30, 2e-4])
def test_decode_streaming_selection(eps):
    """The streaming selection over every token of L, the fallback taken
    when the gain candidates (at most 8192 per row) cannot decide a row: a
    full-length 32K layer (one KV head, ~30K tokens in L) with eps small
    enough that k* exceeds the candidates, over several rounds of the
    selection. The row_path output shows that the fallback decided every
    row, and every output matches the oracle (the decide kernel's full-row
    re-solve, "Verify Before You Fetch", Appendix A.3)."""
    w, gpu, heads, unions, eps = _decode_case("c2", eps=eps, G=1)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")
    assert np.all(gpu["row_path"] == vk.PATH_STREAMING), gpu["row_path"]
    assert np.all(gpu["k_star"] > 8192), gpu["k_star"]


@pytest.mark.parametrize("est", [0, 2])
def test_decode_certificate_coverage_on_gpu(est):
    """Theorem 2 on the library's own outputs: over 400 fresh Poisson samples
    (Philox seeds) of the tiny layer, planned with exact weights, the
    estimate stays within eps^(L') of the true denominator with frequency
    >= 1 - delta (3 sigma slack)."""
    w = make_decode_workload("c1", seed=0)
    dev = torch.device("cuda")
    kb = w["host_kv"][:, :, :, 0, :]
    vb = w["host_kv"][:, :, :, 1, :]
    t_tau = torch.from_numpy(w["tau"]).to(dev)
    t_k = torch.from_numpy(np.ascontiguousarray(kb).view(np.int16)).to(dev)
    t_v = torch.from_numpy(np.ascontiguousarray(vb).view(np.int16)).to(dev)
    host_kv = torch.from_numpy(w["host_kv"].view(np.int16)).pin_memory()
    q = torch.from_numpy(w["q"].view(np.int16)).to(dev)
    sk = torch.from_numpy(w["sketch"].view(np.int16)).to(dev)
    proj = torch.from_numpy(w["proj"]).to(dev)
    kv = bf16_to_f32(w["host_kv"][0, 0])
    _, logd = od.exact_attention(bf16_to_f32(w["q"][0, 0]), kv[:, 0], kv[:, 1])
    cap = 512
    delta, eps = w["delta"], 0.1
    n_trials, fails = 400, 0
    for s in range(n_trials):
        comp = vk.compress(t_tau, t_k, t_v, w["budget"], w["n_sink"],
                           w["n_local"], 5000 + s, cap)
        out = vk.decode_step(q, comp["resident_kv"], comp["resident_idx"],
                             comp["resident_count"], sk, proj, comp["r"],
                             host_kv, eps, delta, estimator=est, weights=1)
        torch.cuda.synchronize()
        dh = float(out["d_hat"][0, 0]) * math.exp(float(out["log_shift"][0, 0]))
        err = abs(dh / math.exp(logd) - 1.0)
        fails += err > float(out["eps_hat"][0, 0])
    gc.say(f"  coverage failures {fails} of {n_trials} (delta {delta})")
    assert fails <= delta * n_trials + 3 * math.sqrt(delta * n_trials)


@pytest.mark.timeout(600)
def test_decode_all_candidates_tier():
    """k* between the top tier (2048 candidates per row) and all candidates
    (8192): a full-length 32K layer at eps = 0.01 (oracle k* of 2.3K-6K).
    Every row is decided by the larger candidate tier or the streaming
    selection, at least one by the candidates, and every output matches."""
    w, gpu, heads, unions, eps = _decode_case("c2", eps=0.01, G=1)
    s = gc.compare(w, gpu, heads, unions, eps)
    gc.say(f"  {s}")
    paths = gpu["row_path"].ravel()
    assert np.all((paths == vk.PATH_ALL_CANDIDATES) | (paths == vk.PATH_STREAMING))
    assert np.any(paths == vk.PATH_ALL_CANDIDATES)
