"""The decode step's timing hook (``phase_events``): with every entry given,
each phase lies between the events recorded around its kernel; with only the
two entries of one phase, that kernel's own dispatch records them. Events
are first recorded long before the step, so an entry the library fails to
record shows up as a phase far longer than the step."""

import time

import numpy as np
import pytest

from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

STALE_S = 0.05  # host sleep between the first records and the step


def _step():
    w = gc.build_case("c1", seed=3)
    dev = gc.device_inputs(w)
    step = vk.DecodeStep(w["B"], w["Hq"], w["G"], w["n"], w["s"], w["cap"],
                         w["n"], torch.device("cuda"))
    step.bind(dev["q"], dev["resident_kv"], dev["resident_idx"],
              dev["resident_count"], dev["sketch"], dev["proj"], dev["r"],
              dev["host_kv"], w["eps"], w["delta"])
    step.launch()
    torch.cuda.synchronize()
    return step


def _stale_events(count):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    time.sleep(STALE_S)
    return evs


def test_every_phase_recorded():
    step = _step()
    P = len(vk.decode_phase_names())
    evs = _stale_events(P + 1)
    step.set_phase_events(evs)
    step.launch()
    torch.cuda.synchronize()
    step.set_phase_events(None)
    ph = np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(P)])
    print("phases ms", ph.round(4).tolist(), flush=True)
    assert np.all(ph >= 0.0)
    assert ph.sum() < 1e3 * STALE_S / 2  # no entry left from before the step
    assert step.check_status()[0] == 0


@pytest.mark.parametrize("name", ["scan", "shortlist", "shrink", "cert", "fetch"])
def test_one_phase_by_its_dispatch(name):
    """One kernel's own dispatch records the pair (phases with no kernel in
    this mode, the shortlist and binary shrinkage here, record plain
    markers)."""
    step = _step()
    names = vk.decode_phase_names()
    P = len(names)
    phase = names.index(name)
    evs = [None] * (P + 1)
    pair = _stale_events(2)
    evs[phase], evs[phase + 1] = pair
    step.set_phase_events(evs)
    step.launch()
    torch.cuda.synchronize()
    step.set_phase_events(None)
    ms = pair[0].elapsed_time(pair[1])
    print("phase", phase, "ms", ms, flush=True)
    assert 0.0 <= ms < 1e3 * STALE_S / 2
    assert step.check_status()[0] == 0
