"""The read-ahead of likely fetched rows during planning (prefetch_rows):
rows copied from host memory into the workspace on a second stream before
k* is known, taken from there by the gather. A row is the same bytes
wherever it is read from, so every output must be bit-identical to the
step without read-ahead; only host_bytes grows, by the rows read ahead and
not fetched (MI355X only)."""

import numpy as np
import pytest

from oracle import decode as od
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

ROW = 2 * 128 * 2  # bytes of one K/V row
KEYS = ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
        "fetch_count", "row_stats", "row_path")


def _same(a, b):
    for k in KEYS:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8),
                              np.asarray(b[k]).view(np.uint8)), k
    cnt = a["fetch_count"]
    for bg in np.ndindex(cnt.shape):
        c = int(cnt[bg])
        assert np.array_equal(a["fetch_idx"][bg][:c], b["fetch_idx"][bg][:c]), bg


def _run(w, dev, pf, est=0, weights=0):
    return gc.run_library(w, dev, w["eps"], w["delta"], est, weights,
                          prefetch_rows=pf)


def _check(w, dev, pfs, est=0, weights=0):
    plain = _run(w, dev, 0, est, weights)
    assert plain["rc"] == 0, plain["bits"]
    base = int(plain["host_bytes"][0])
    for pf in pfs:
        gc.say(f"  prefetch_rows={pf}")
        spec = _run(w, dev, pf, est, weights)
        assert spec["rc"] == 0, spec["bits"]
        _same(spec, plain)
        if weights == od.W_SKETCH2:
            assert np.array_equal(spec["shortlist"], plain["shortlist"])
        hb = int(spec["host_bytes"][0])
        assert hb % ROW == 0
        # rows read ahead replace gather reads one for one; the rest is extra
        m = w["n"] if pf < 0 else pf
        assert base <= hb <= base + ROW * m * w["B"] * w["G"], (base, hb)
    return plain


@pytest.mark.timeout(600)
def test_full_c2():
    """The batch-1, 32K-token layer at its full size: the library's own
    choice and explicit counts, up to more rows than are fetched."""
    gc.say("prefetch full c2")
    w = gc.build_case("c2")
    dev = gc.device_inputs(w)
    plain = _check(w, dev, [-1, 64, 768, 4096])
    assert int(np.sum(plain["fetch_count"])) > 0  # the gather has work


@pytest.mark.parametrize("cfg,weights,est,kw", [
    ("c3", od.W_SKETCH, 0, dict(n=8192, B=4, shift_from=1)),
    ("c2", od.W_SKETCH2, 0, dict(n=6000, G=4, pair_profile=True)),
    ("c2", od.W_PERFECT, 0, dict(n=5000, G=2)),
    ("c2", od.W_SKETCH, 2, dict(n=6000, G=2)),
    ("c2", od.W_SKETCH, 1, dict(n=4321, G=2, B=2)),
    ("c4", od.W_SKETCH, 0, dict(n=20000, B=1, G=2)),
    ("c2", od.W_SKETCH, 0, dict(n=5000, G=2, grp=8)),
    ("c2", od.W_SKETCH, 0, dict(n=5000, G=4, grp=1)),
    ("c2", od.W_SKETCH, 0, dict(n=300, G=2, budget=160)),
    ("c3", od.W_SKETCH, 0, dict(n=2049, B=3, G=1, shift_from=0)),
])
def test_modes(cfg, weights, est, kw):
    """Every planning-weight mode (the fork follows the pass-0 launch with
    the 2-bit sketch), every estimator, ragged lengths and batches."""
    gc.say(f"prefetch {cfg} weights={weights} est={est} {kw}")
    w = gc.build_case(cfg, **kw)
    dev = gc.device_inputs(w)
    # (8 rows: more tokens pass the threshold than fit, so the area's slots
    # run out and the rest are dropped)
    _check(w, dev, [-1, 200, 8], est, weights)


def test_every_row_read_ahead():
    """With room for every token, every token of L outside S is read ahead
    and the gather reads nothing from host memory: host_bytes is exactly
    one row per such token."""
    gc.say("prefetch all rows")
    w = gc.build_case("c2", n=4096, G=2, B=2)
    dev = gc.device_inputs(w)
    plain = _run(w, dev, 0)
    spec = _run(w, dev, w["n"])
    assert spec["rc"] == 0, spec["bits"]
    _same(spec, plain)
    rows = 0
    for b in range(w["B"]):
        for g in range(w["G"]):
            res = np.zeros(w["n"], dtype=bool)
            res[w["cm"][b][g]["resident_idx"]] = True
            rows += int(np.sum((w["r_all"][b, g] < 1.0) & ~res))
    assert int(spec["host_bytes"][0]) == rows * ROW


def test_steps_alternate_with_and_without():
    """Steps with and without read-ahead, one after the other on the same
    device (the second stream is shared), give the same outputs."""
    w = gc.build_case("c2", n=3000, G=2, B=1)
    dev = gc.device_inputs(w)
    ref = _run(w, dev, 0)
    for pf in (100, 0, -1, 0, 100):
        _same(_run(w, dev, pf), ref)


def test_with_staging():
    """Read-ahead beside rows staged by the previous step (those are not
    read ahead again): a short serving loop, each step against the step
    without either."""
    from tests.test_gpu_maint import Serving
    sv = Serving("c2", od.W_SKETCH, 3, n=3000, G=2, B=2)
    w = sv.w
    sv.step_s = vk.DecodeStep(w["B"], w["Hq"], w["G"], sv.n, w["s"], sv.cap,
                              sv.fetch_cap, gc.torch_mod().device("cuda"),
                              ctx_stride=sv.ns, prefetch_rows=500)
    for t in range(3):
        staged, plain = sv.decode()
        assert staged["rc"] == 0 and plain["rc"] == 0
        _same(staged, plain)
        if t < 2:
            sv.append()


def test_noalloc_reads_nothing_ahead():
    """The no-allocation entry point takes prefetch_rows as 0: asked for the
    library's count, it gives the plain step's outputs and host bytes."""
    w = gc.build_case("c2", n=5000, G=2, seed=5)
    dev = gc.device_inputs(w)
    plain = _run(w, dev, 0)
    step = vk.DecodeStep(w["B"], w["Hq"], w["G"], w["n"], w["s"], w["cap"],
                         w["n"], gc.torch_mod().device("cuda"), prefetch_rows=-1)
    assert vk.vkv_decode_prefetch_rows(step.args) > 0
    step.bind(dev["q"], dev["resident_kv"], dev["resident_idx"],
              dev["resident_count"], dev["sketch"], dev["proj"], dev["r"],
              dev["host_kv"], w["eps"], w["delta"])
    step.args.workspace = None
    step.args.workspace_bytes = 0
    assert vk.vkv_decode_step_noalloc(step.args, vk._stream(None)) == vk.VKV_OK, \
        vk.vkv_last_error()
    rc, bits = step.check_status()
    assert rc == 0, bits
    got = {k: v.cpu().numpy() for k, v in step.out.items()}
    _same(got, plain)
    assert int(got["host_bytes"][0]) == int(plain["host_bytes"][0])
