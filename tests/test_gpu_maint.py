"""GPU parity of decode-time maintenance ("Verify Before You Fetch",
section 3 and Appendix A.3.1-A.3.2): a serving loop of decode steps on a
cache that grows in place (each generated token appended to H), with rows
staged across steps, and a repeated compression from the host cache --
every step against the oracle on the same state (MI355X only)."""

import numpy as np
import pytest

from oracle import compress as oc
from oracle import decode as od
from oracle import maintain as om
from oracle import sketch2 as sk2
from tests import gpu_cases as gc
from workloads import bf16_bits, bf16_to_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verified_sparse_kv_amd import verkv as vk  # noqa: E402

DEV = torch.device("cuda")
OUT_KEYS = ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
            "fetch_count", "row_stats", "row_path")


def _same_outputs(a, b):
    """Bit-identical outputs (the fetch lists up to their counts: entries
    past them are not written)."""
    for k in OUT_KEYS:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8),
                              np.asarray(b[k]).view(np.uint8)), k
    cnt = a["fetch_count"]
    for bg in np.ndindex(cnt.shape):
        c = int(cnt[bg])
        assert np.array_equal(a["fetch_idx"][bg][:c], b["fetch_idx"][bg][:c]), bg


class Serving:
    """Library and oracle state of one serving loop (capacity ns)."""

    def __init__(self, cfg, weights, steps, n_short=128, **kw):
        w = gc.build_case(cfg, pair_profile=weights == od.W_SKETCH2, **kw)
        self.w, self.weights, self.n_short = w, weights, n_short
        B, G, n0, d, s = w["B"], w["G"], w["n"], w["d"], w["s"]
        self.ns = ns = n0 + steps + 3
        self.n = n0
        self.cap = w["cap"] + steps + 3
        self.fetch_cap = n0
        host = np.zeros((B, G, ns, 2, d), dtype=np.uint16)
        host[:, :, :n0] = w["host_kv"]
        r = np.full((B, G, ns), 0.5, dtype=np.float32)
        r[:, :, :n0] = w["r_all"]
        sketch = np.zeros((B, G, ns, s), dtype=np.uint16)
        sketch[:, :, :n0] = w["sketch"]
        self.orc = dict(host_kv=host, r=r, sketch=sketch,
                        res_idx=[[w["cm"][b][g]["resident_idx"].astype(np.int64)
                                  for g in range(G)] for b in range(B)],
                        res_kv=[[host[b, g, w["cm"][b][g]["resident_idx"]]
                                 for g in range(G)] for b in range(B)])
        # library state
        self.host = torch.from_numpy(host.view(np.int16)).pin_memory()
        rkv = np.zeros((B, G, self.cap, 2, d), dtype=np.uint16)
        ridx = np.zeros((B, G, self.cap), dtype=np.int32)
        rcnt = np.zeros((B, G), dtype=np.int32)
        for b in range(B):
            for g in range(G):
                idx = self.orc["res_idx"][b][g]
                rkv[b, g, :idx.size] = host[b, g, idx]
                ridx[b, g, :idx.size] = idx
                rcnt[b, g] = idx.size
        self.rkv = torch.from_numpy(rkv.view(np.int16)).to(DEV)
        self.ridx = torch.from_numpy(ridx).to(DEV)
        self.rcnt = torch.from_numpy(rcnt).to(DEV)
        self.r = torch.from_numpy(r).to(DEV)
        self.sketch = torch.from_numpy(sketch.view(np.int16)).to(DEV)
        self.proj = torch.from_numpy(w["proj"]).to(DEV)
        self.status = torch.zeros((1,), dtype=torch.int32, device=DEV)
        self.sk2 = None
        self.sk2_orc = None
        if weights == od.W_SKETCH2:
            self.build_sketch2()
        self.q = w["q"].copy()
        self.qrng = np.random.default_rng(99)
        Hq = w["Hq"]
        # two steps (staging and none) over the same capacity layout
        self.step_s = vk.DecodeStep(B, Hq, G, n0, s, self.cap, self.fetch_cap,
                                    DEV, n_short=n_short, ctx_stride=ns)
        self.step_n = vk.DecodeStep(B, Hq, G, n0, s, self.cap, self.fetch_cap,
                                    DEV, n_short=n_short, ctx_stride=ns)
        self.maps = [torch.full((B, G, ns), -1, dtype=torch.int32, device=DEV)
                     for _ in range(2)]
        self.stages = [torch.zeros((B, G, self.fetch_cap, 2, d), dtype=torch.int16,
                                   device=DEV) for _ in range(2)]
        self.t = 0
        self.prev_union = None

    def build_sketch2(self):
        B, G = self.w["B"], self.w["G"]
        view = self.host.view(B, G, self.ns, 256)
        self.sk2 = vk.sketch2_build(view, n=self.n)
        torch.cuda.synchronize()
        chan = self.sk2["chan"].cpu().numpy()
        self.sk2_orc = []
        for b in range(B):
            row = []
            for g in range(G):
                keys = bf16_to_f32(self.orc["host_kv"][b, g, :self.n, 0, :])
                sk = sk2.build(keys)
                lp = np.sort(chan[b, g, :16].astype(np.int64))
                if not np.array_equal(lp, sk["pairs"]):
                    sk = sk2.with_pairs(keys, lp)  # (a near tie of energies)
                row.append(sk)
            self.sk2_orc.append(row)

    def oracle_sketch2_append(self, pos):
        for row in self.sk2_orc:
            for sk in row:
                sk["codes"] = np.concatenate([sk["codes"],
                                              np.zeros((1, sk["codes"].shape[1]), np.uint8)])
                if pos // 128 >= sk["zero"].shape[0]:
                    z = np.zeros((1, sk["zero"].shape[1]), np.float32)
                    sk["zero"] = np.concatenate([sk["zero"], z])
                    sk["scale"] = np.concatenate([sk["scale"], z])

    def bind(self, step, q):
        step.set_tokens(self.n)
        step.bind(q, self.rkv, self.ridx, self.rcnt, self.sketch, self.proj,
                  self.r, self.host, self.w["eps"], self.w["delta"], 0,
                  self.weights, self.sk2)

    def decode(self):
        """One step with staging and the same step without; returns both."""
        q_dev = torch.from_numpy(self.q.view(np.int16)).to(DEV)
        res = []
        for step, staged in ((self.step_s, True), (self.step_n, False)):
            self.bind(step, q_dev)
            if staged:
                step.set_staging(prev=(self.maps[(self.t + 1) % 2], self.stages[(self.t + 1) % 2]),
                                 nxt=(self.maps[self.t % 2], self.stages[self.t % 2]))
            out = step.launch()
            rc, bits = step.check_status()
            g = {k: v.cpu().numpy().copy() for k, v in out.items()}
            g["rc"], g["bits"], g["n_short"] = rc, bits, self.n_short
            res.append(g)
        self.t += 1
        return res

    def oracle(self):
        w, n = self.w, self.n
        B, G = w["B"], w["G"]
        wt = dict(w)
        wt.update(n=n, q=self.q, host_kv=self.orc["host_kv"][:, :, :n],
                  r_all=self.orc["r"][:, :, :n], sketch=self.orc["sketch"][:, :, :n],
                  n_short=self.n_short,
                  cm=[[dict(resident_idx=self.orc["res_idx"][b][g],
                            resident_kv=bf16_to_f32(self.orc["res_kv"][b][g]))
                       for g in range(G)] for b in range(B)])
        if self.weights == od.W_SKETCH2:
            wt["sk2_oracle"] = self.sk2_orc
        heads, unions = od.decode_step(
            bf16_to_f32(self.q), [[c["resident_kv"] for c in row] for row in wt["cm"]],
            [[c["resident_idx"] for c in row] for row in wt["cm"]],
            bf16_to_f32(wt["sketch"]), w["proj"], wt["r_all"],
            bf16_to_f32(wt["host_kv"]), w["eps"], w["delta"], 0, self.weights,
            sketch2=self.sk2_orc, n_short=self.n_short)
        return wt, heads, unions

    def append(self):
        """A generated token joins H on both sides; then the library state is
        checked against the oracle's bit for bit."""
        B, G, d = self.w["B"], self.w["G"], self.w["d"]
        pos = self.n
        k_new = bf16_bits(self.qrng.standard_normal((B, G, d)).astype(np.float32) * 2)
        v_new = bf16_bits(self.qrng.standard_normal((B, G, d)).astype(np.float32))
        vk.append_token(torch.from_numpy(k_new.view(np.int16)).to(DEV),
                        torch.from_numpy(v_new.view(np.int16)).to(DEV), pos,
                        self.host, self.rkv, self.ridx, self.rcnt, self.r,
                        self.status, self.sketch, self.proj, self.sk2)
        torch.cuda.synchronize()
        om.append_token(self.orc, pos, k_new, v_new, self.w["proj"])
        if self.sk2_orc is not None:
            self.oracle_sketch2_append(pos)
        self.n += 1
        assert int(self.status.cpu()[0]) == 0
        rcnt = self.rcnt.cpu().numpy()
        ridx = self.ridx.cpu().numpy()
        rkv = self.rkv.cpu().numpy().view(np.uint16)
        for b in range(B):
            for g in range(G):
                idx = self.orc["res_idx"][b][g]
                assert rcnt[b, g] == idx.size
                assert np.array_equal(ridx[b, g, :idx.size], idx)
                assert np.array_equal(rkv[b, g, :idx.size], self.orc["res_kv"][b][g])
        assert np.array_equal(self.r.cpu().numpy()[:, :, :self.n],
                              self.orc["r"][:, :, :self.n])
        assert np.array_equal(self.host.numpy().view(np.uint16)[:, :, pos],
                              self.orc["host_kv"][:, :, pos])
        assert np.array_equal(self.sketch.cpu().numpy().view(np.uint16)[:, :, pos],
                              self.orc["sketch"][:, :, pos])
        if self.sk2 is not None:
            assert np.all(self.sk2["codes"].cpu().numpy()[:, :, pos] == 0)
        # the next query: correlated with this one, as consecutive decode
        # queries are
        qf = bf16_to_f32(self.q) * 0.9 + 0.44 * self.qrng.standard_normal(self.q.shape)
        self.q = bf16_bits(qf.astype(np.float32))

    def recompress(self, seed):
        """PoissonComp again from the host cache with fresh scores; checked
        against the oracle bit for bit. Staging restarts from empty maps."""
        w = self.w
        B, G, n, ns = w["B"], w["G"], self.n, self.ns
        rng = np.random.default_rng(seed)
        tau = rng.beta(0.5, 5, (B, G, ns)).astype(np.float32)
        budget = w["budget"] + 8
        out = dict(r=self.r, resident_idx=self.ridx, resident_count=self.rcnt,
                   resident_kv=self.rkv,
                   water_level=torch.empty((B, G), dtype=torch.float64, device=DEV),
                   status=torch.zeros((1,), dtype=torch.int32, device=DEV))
        vk.recompress(torch.from_numpy(tau).to(DEV), self.host, n, budget,
                      w["n_sink"], w["n_local"], seed, out)
        rc, bits = vk.vkv_check_status(vk._ptr(out["status"]), vk._stream(None))
        assert rc == 0, (rc, bits)
        kf = bf16_to_f32(self.orc["host_kv"][:, :, :n, 0, :])
        vf = bf16_to_f32(self.orc["host_kv"][:, :, :n, 1, :])
        cm = oc.compress(tau[:, :, :n], kf, vf, budget, w["n_sink"], w["n_local"], seed)
        r = self.r.cpu().numpy()
        ridx = self.ridx.cpu().numpy()
        rcnt = self.rcnt.cpu().numpy()
        rkv = self.rkv.cpu().numpy().view(np.uint16)
        for b in range(B):
            for g in range(G):
                sl = cm[b][g]
                assert np.array_equal(r[b, g, :n].view(np.uint32), sl["r"].view(np.uint32))
                idx = sl["resident_idx"]
                assert rcnt[b, g] == idx.size and np.array_equal(ridx[b, g, :idx.size], idx)
                assert np.array_equal(rkv[b, g, :idx.size], self.orc["host_kv"][b, g, idx])
                self.orc["r"][b, g, :n] = sl["r"]
                self.orc["res_idx"][b][g] = idx.astype(np.int64)
                self.orc["res_kv"][b][g] = self.orc["host_kv"][b, g, idx]
        if self.weights == od.W_SKETCH2:
            self.build_sketch2()
        for m in self.maps:
            m.fill_(-1)


def _check_step(sv, staged, plain, heads, unions, wt):
    s = gc.compare(wt, plain, heads, unions, sv.w["eps"], weights=sv.weights)
    # staging changes where rows come from, never the results
    _same_outputs(staged, plain)
    B, G = sv.w["B"], sv.w["G"]
    hits = 0
    union = [[plain["fetch_idx"][b, g, :plain["fetch_count"][b, g]] for g in range(G)]
             for b in range(B)]
    if sv.prev_union is not None:
        for b in range(B):
            for g in range(G):
                hits += om.staged_hits(sv.prev_union[b][g], union[b][g]).size
    saved = int(plain["host_bytes"][0]) - int(staged["host_bytes"][0])
    assert saved == hits * 512, (saved, hits)
    sv.prev_union = union
    return s, hits


@pytest.mark.parametrize("cfg,weights,kw", [
    ("c2", od.W_SKETCH, dict(n=3000, G=2, B=2)),
    ("c3", od.W_SKETCH, dict(n=4000, G=2, B=3, seed=2)),
    ("c2", od.W_SKETCH2, dict(n=3000, G=2, B=2)),
])
def test_serving_loop(cfg, weights, kw):
    """Decode, append, decode ... with staging; a repeated compression in
    the middle; every step against the oracle on the same state."""
    steps = 5
    gc.say(f"serving {cfg} weights={weights} {kw}")
    sv = Serving(cfg, weights, steps, **kw)
    total_hits = 0
    for t in range(steps):
        if t == 3:
            sv.recompress(seed=40 + t)
            sv.prev_union = None
        staged, plain = sv.decode()
        wt, heads, unions = sv.oracle()
        s, hits = _check_step(sv, staged, plain, heads, unions, wt)
        total_hits += hits
        gc.say(f"  step {t} n={sv.n} fetched={s['fetched']} staged hits={hits} "
               f"ties={s['ties']}")
        if t < steps - 1:
            sv.append()
    assert total_hits > 0  # consecutive correlated queries share fetched rows


def test_first_step_staging_is_empty():
    """With empty maps nothing is found in the staging: the host bytes equal
    those of a step without staging."""
    sv = Serving("c2", od.W_SKETCH, 1, n=2500, G=2, B=1)
    staged, plain = sv.decode()
    assert int(staged["host_bytes"][0]) == int(plain["host_bytes"][0])
    _same_outputs(staged, plain)


def test_same_query_twice_reads_nothing_from_host():
    """The same query at the same context twice: the second step finds every
    fetched row in the staging and reads nothing from host memory."""
    sv = Serving("c2", od.W_SKETCH, 2, n=2500, G=2, B=1)
    first, _ = sv.decode()
    second, plain = sv.decode()
    assert int(first["host_bytes"][0]) > 0
    assert int(second["host_bytes"][0]) == 0
    _same_outputs(second, plain)
