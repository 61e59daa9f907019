#!/usr/bin/env python3
"""Benchmark of one verified decode step (KVFetch) on one MI355X.

Default workload (the metric's configuration): a Qwen3-4B-shaped decode layer
with 32 query heads over 8 KV heads, head_dim 128, 32768 tokens of context,
batch 1, 1/16 of the cache resident, a 32-dim bf16 key sketch, eps = 0.1,
delta = 0.05. The cache is compressed once by the library (PoissonComp);
then every timed step runs the whole decode path -- sketch scan, exact
resident logits, shrinkage fixed point, certificate, gain selection, fetch
from pinned host memory and corrected attention -- for a fresh query.

Prints one JSON line. ``value`` is q-head x context tokens per second over
the timed steps (inputs resident in HBM, full cache in pinned host memory).
The ``roofline`` object covers the longest-running HBM-bound kernel, timed
with a pair of HIP events that the kernel's own dispatch records on the
library's stream, over as many steps as the timed region;
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("verified decode steps/sec (q-heads x ctx tokens/s) at 32K; "
          "% HBM peak; fetch %")
HBM_PEAK_GBS = 8000.0
ROW_BYTES = 2 * 128 * 2  # one token's K and V rows in bf16


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--estimator", default="clip",
                    choices=["clip", "unbiased", "binary"],
                    help="clipped shrinkage (Definition 2, the default), the "
                         "unbiased lambda = 1 estimator, or binary shrinkage "
                         "(Appendix A.2)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the Dense (resident) / Dense (offload) baselines")
    ap.add_argument("--no-compress", action="store_true",
                    help="skip the compression pass over the 36-layer, "
                         "128K-token workload")
    ap.add_argument("--also", nargs="*", default=["c3", "c4"],
                    choices=["c2", "c3", "c4"],
                    help="other decode workloads measured after the headline "
                         "one, each reported as its own block (default: c3, "
                         "batch 16 with fetching active, and c4, 128K at batch "
                         "4); none with --also")
    ap.add_argument("--prefetch-rows", type=int, default=-1,
                    help="rows per (request, KV head) read from host memory "
                         "while the planning launches run (-1: the library's "
                         "choice for the shapes, 0: none); each decode block "
                         "also times the same steps without it")
    ap.add_argument("--no-prefetch-compare", action="store_true",
                    help="do not time the decode steps a second time without "
                         "read-ahead (kernel traces then hold one mode only; "
                         "fetch_pct then counts the rows read ahead too)")
    ap.add_argument("--weights", default="sketch", choices=["sketch", "sketch2"],
                    help="planning weights of the main line: the projected "
                         "sketch (default) or the pages' 2-bit sketch with "
                         "a 128-token exact shortlist")
    ap.add_argument("--serving", nargs="*", default=["c3"],
                    choices=["c2", "c3", "c4"],
                    help="serving loops (block '<config>_serving'): each step "
                         "a decode step and the generated token's append, "
                         "the next query correlated with the last, fetched "
                         "rows staged for the next step; none with --serving")
    ap.add_argument("--sketch2", nargs="*", default=["c2", "c3"],
                    choices=["c2", "c3", "c4"],
                    help="workloads measured again planning with the pages' "
                         "2-bit sketch and a 128-token exact shortlist "
                         "(blocks '<config>_sketch2'); none with --sketch2")
    return ap.parse_args()


ESTIMATORS = {"clip": 0, "unbiased": 1, "binary": 2}


def algorithmic_bytes_sketch2(w, counts, fetching_rows, est="clip"):
    """The same with the 2-bit sketch: the scan reads 8 bytes of codes, one
    byte of zero points and scales (128 bytes per 128-token group) and r per
    (request, KV head, token), with the resident K rows, positions and q.
    Intermediates: the fp32 sketch logit of every (query head, token) and
    the shortlist key of every (KV head, token). The pass-0 launch reads the
    planning logits once and r once per KV head (5 B per q-head x token at 4
    query heads per KV head), like the estimator phases."""
    B, Hq, G, n, d = w["B"], w["Hq"], w["G"], w["n"], w["d"]
    grp = Hq // G
    rows = int(counts.sum())
    tok = B * Hq * n * 4 + B * G * n * 4
    ftok = fetching_rows * n * 4 + min(fetching_rows, B * G) * n * 4
    sk = B * G * n * (8 + 1 + 4)
    per = {"scan": sk + rows * (2 * d + 4) + B * Hq * d * 2,
           "pass0": tok, "beta1": tok, "cert": tok, "cand": ftok}
    inter = {"scan": B * Hq * n * 4 + B * G * n * 4 + rows * grp * 4}
    if est == "binary":
        per["shrink"] = 2 * tok
    return dict(step=sk + rows * (4 * d + 4) + B * Hq * d * (2 + 4),
                kernels=per, intermediate=inter)


def algorithmic_bytes(w, counts, fetching_rows, est="clip"):
    """Algorithmic HBM bytes of one step and of each HBM-bound kernel, each
    input counted once; intermediates the design writes and reads back are
    reported apart and are not in the fractions.

    Step (compulsory): sketch + r for every (request, KV head, token), the
    resident K and V rows with their positions, q in and the output out
    (17 + 129 eta bytes per q-head x token at s = 32, d = 128, 4 query heads
    per KV head).
    Per kernel:
      scan   the sketch and r of every token, the resident K rows and their
             positions, q (the a5/a6 inputs). Intermediate: the fp32 sketch
             logit of every (query head, token) and the resident logits.
      beta1, cert   the estimator phases' own figure: the sketch logit of
             every (query head, token) read once and r once per KV head
             (5 B per q-head x token at 4 query heads per KV head).
      cand   the same for the rows that fetch.
      shrink (binary shrinkage) two reads of the same.
    The gather is bound by the host link and reported separately (it runs in
    one launch with the attention over the resident rows, which hides
    behind it); the resolve and walk steps touch only per-row summaries.
    """
    B, Hq, G, n, s, d = w["B"], w["Hq"], w["G"], w["n"], w["s"], w["d"]
    grp = Hq // G
    rows = int(counts.sum())
    tok = B * Hq * n * 4 + B * G * n * 4
    ftok = fetching_rows * n * 4 + min(fetching_rows, B * G) * n * 4
    per = {"scan": B * G * n * (2 * s + 4) + rows * (2 * d + 4)
           + B * Hq * d * 2,
           "beta1": tok, "cert": tok, "cand": ftok}
    inter = {"scan": B * Hq * n * 4 + rows * grp * 4}
    if est == "binary":
        per["shrink"] = 2 * tok
    return dict(step=B * G * n * (2 * s + 4) + rows * (4 * d + 4)
                + B * Hq * d * (2 + 4), kernels=per, intermediate=inter)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_{}_traffic.md")
DECODE_SOURCES = ("verified_sparse_kv_amd/csrc/vkv_decode.hip",
                  "verified_sparse_kv_amd/csrc/vkv_common.h",
                  "verified_sparse_kv_amd/csrc/vkv_internal.h")


def measured_traffic(config, kernel, estimator="clip"):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE /
    WRITE_SIZE counter summary of this workload, or None when there is none
    or the decode sources changed since the counters were taken."""
    import hashlib
    path = TRAFFIC_FILE.format(config)
    if not os.path.exists(path) or estimator != "clip":
        return None
    vals, want = {}, None
    for line in open(path):
        if " = " not in line:
            continue
        k, v = (x.strip() for x in line.split(" = ", 1))
        if k == "source_sha256":
            want = v
        elif k.startswith("traffic."):
            vals[k[len("traffic."):]] = float(v)
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if want != h.hexdigest():
        return None
    return vals.get(kernel)


def cpu_baseline(w, seconds, est=0):
    """The oracle (never tuned) decoding KV-head groups of the same layer until
    `seconds` of CPU work have been spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import compress as oc
    from oracle import decode as od
    from workloads import bf16_to_f32

    B, G, Hq, n = w["B"], w["G"], w["Hq"], w["n"]
    grp = Hq // G
    units = 0
    groups = 0
    spent = 0.0
    prepared = {}
    while spent < seconds and groups < 1000:
        b, g = (groups // G) % B, groups % G
        if (b, g) not in prepared:
            sl = oc.compress_slice(w["tau"][b, g], w["budget"], w["n_sink"],
                                   w["n_local"], w["seed"], b, g)
            kv = bf16_to_f32(w["host_kv"][b, g])
            idx = sl["resident_idx"]
            prepared[(b, g)] = (sl["r"], idx,
                                np.stack([kv[idx, 0], kv[idx, 1]], axis=1), kv,
                                bf16_to_f32(w["sketch"][b, g]))
        r, idx, res_kv, kv, sk = prepared[(b, g)]
        q = bf16_to_f32(w["q_steps"][groups % len(w["q_steps"])]
                        [b, g * grp:(g + 1) * grp])
        t0 = time.perf_counter()
        od.decode_group(q, res_kv, idx, sk, w["proj"][g], r, kv, w["eps"],
                        w["delta"], est)
        spent += time.perf_counter() - t0
        units += grp * n
        groups += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": units / spent, "unit": "q-head*ctx-tokens/s",
            "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{groups} decisions-groups (one KV head, {grp} query "
                      f"heads, {n} tokens, fresh query each) of the same "
                      f"layer, fp64 numpy, {spent:.1f} s; "
                      f"host cores available: {len(os.sched_getaffinity(0))}"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def compress_pass(dev, steps):
    """PoissonComp over a whole model's prefill cache: 36 layers x 8 KV heads
    x 131072 tokens, tau ~ Beta(0.5, 5), 4 sinks + 256 local tokens, at
    eta = 1/8, 1/16, 1/32 (K and V random bf16 on the device). Per eta: the
    GPU span of one call (events on the stream around it), its algorithmic
    HBM bytes (tau read, r written, the resident positions written, each
    resident K/V row read and written) as GB/s, and the time per (layer,
    KV head) slice."""
    import torch

    from verified_sparse_kv_amd import verkv as vk
    from workloads import C5, make_c5_tau, resident_cap
    L, G, n = C5["layers"], C5["G"], C5["n"]
    t_tau = torch.from_numpy(make_c5_tau(seed=0)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    kv = [torch.randn((L, G, n, 128), dtype=torch.bfloat16, device=dev,
                      generator=gen).view(torch.int16) for _ in range(2)]
    out = {"workload": f"{L} layers x {G} KV heads x {n} tokens, tau ~ "
                       f"Beta(0.5, 5), {C5['n_sink']} sinks + "
                       f"{C5['n_local']} local", "per_eta": {}}
    k = max(1, min(steps, 10))
    for eta in C5["etas"]:
        budget = int(round(eta * n))
        cap = resident_cap(budget)
        ws = None
        for _ in range(2):
            res = vk.compress(t_tau, kv[0], kv[1], budget, C5["n_sink"],
                              C5["n_local"], 0, cap, workspace=ws)
            ws = res["workspace"]
        evs = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        torch.cuda.synchronize()
        for i in range(k):
            evs[i][0].record()
            res = vk.compress(t_tau, kv[0], kv[1], budget, C5["n_sink"],
                              C5["n_local"], 0, cap, workspace=ws)
            evs[i][1].record()
        torch.cuda.synchronize()
        rc, bits = vk.vkv_check_status(vk._ptr(res["status"]), vk._stream(None))
        assert rc == 0, (rc, bits, vk.vkv_last_error())
        ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / k
        rows = int(res["resident_count"].sum().item())
        nbytes = 8 * L * G * n + rows * (4 + 2 * ROW_BYTES)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["per_eta"][f"1/{round(1 / eta)}"] = {
            "ms": ms, "algorithmic_bytes": nbytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "us_per_slice": ms * 1e3 / (L * G), "resident_rows": rows,
            "calls": k}
        del res
    del kv, t_tau
    torch.cuda.empty_cache()
    return out


def serving_loop(config, args, dev):
    """A serving loop on one workload: the cache compressed once (from the
    pinned host cache, into a layout with room to grow), then per step a
    decode step for the current query and the append of the generated token
    (a random bf16 K/V row) to every (request, KV head); the next query is
    0.9 q + 0.44 N(0, I) (consecutive decode queries are correlated). Timed
    twice over the same sequence: with the fetched rows staged for the next
    step (hits read from device memory) and without. Reports ms per step
    (decode + append), host bytes per step and the share of fetched rows
    found in the staging."""
    import numpy as np
    import torch

    from verified_sparse_kv_amd import verkv as vk
    from workloads import bf16_bits, make_decode_workload, resident_cap

    w = make_decode_workload(config, seed=args.seed, with_queries=False)
    B, Hq, G, n0, s, d = w["B"], w["Hq"], w["G"], w["n"], w["s"], w["d"]
    K = max(2, min(args.steps, 20))
    W = max(1, min(args.warmup, 5))
    total = W + K
    ns = n0 + 2 * total + 2
    cap = resident_cap(w["budget"]) + 2 * total + 2
    host0 = np.zeros((B, G, ns, 2, d), dtype=np.uint16)
    host0[:, :, :n0] = w["host_kv"]
    tau = np.zeros((B, G, ns), dtype=np.float32)
    tau[:, :, :n0] = w["tau"]
    sketch0 = np.zeros((B, G, ns, s), dtype=np.uint16)
    sketch0[:, :, :n0] = w["sketch"]
    rng = np.random.default_rng([7, args.seed])
    q0 = bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    new_kv = [(bf16_bits(rng.standard_normal((B, G, d), dtype=np.float32)),
               bf16_bits(rng.standard_normal((B, G, d), dtype=np.float32)))
              for _ in range(total)]
    qs = [q0]
    for _ in range(total - 1):
        qf = (qs[-1].astype(np.uint32) << 16).view(np.float32)
        qs.append(bf16_bits((0.9 * qf + 0.44 * rng.standard_normal(qf.shape))
                            .astype(np.float32)))
    t_qs = [torch.from_numpy(q.view(np.int16)).to(dev) for q in qs]
    t_kv = [(torch.from_numpy(a.view(np.int16)).to(dev),
             torch.from_numpy(b.view(np.int16)).to(dev)) for a, b in new_kv]
    proj = torch.from_numpy(w["proj"]).to(dev)
    host = torch.from_numpy(host0.view(np.int16)).pin_memory()
    t_tau = torch.from_numpy(tau).to(dev)

    def run(staged, record=False):
        """Compress, then W + K steps; returns (ms per timed step, host
        bytes per timed step, fetched rows, rows found in the staging)."""
        st = dict(r=torch.zeros((B, G, ns), dtype=torch.float32, device=dev),
                  resident_idx=torch.zeros((B, G, cap), dtype=torch.int32, device=dev),
                  resident_count=torch.zeros((B, G), dtype=torch.int32, device=dev),
                  resident_kv=torch.zeros((B, G, cap, 2, d), dtype=torch.int16, device=dev),
                  water_level=torch.empty((B, G), dtype=torch.float64, device=dev),
                  status=torch.zeros((1,), dtype=torch.int32, device=dev))
        host.copy_(torch.from_numpy(host0.view(np.int16)))
        vk.recompress(t_tau, host, n0, w["budget"], w["n_sink"], w["n_local"],
                      w["seed"], st)
        sketch = torch.from_numpy(sketch0.view(np.int16)).to(dev)
        status = torch.zeros((1,), dtype=torch.int32, device=dev)
        step = vk.DecodeStep(B, Hq, G, n0, s, cap, n0, dev, ctx_stride=ns,
                             prefetch_rows=args.prefetch_rows)
        maps = [torch.full((B, G, ns), -1, dtype=torch.int32, device=dev)
                for _ in range(2)]
        stages = [torch.empty((B, G, n0, 2, d), dtype=torch.int16, device=dev)
                  for _ in range(2)]
        hb, lists = [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(total):
            if i == W:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            n = n0 + i
            step.set_tokens(n)
            step.bind(t_qs[i], st["resident_kv"], st["resident_idx"],
                      st["resident_count"], sketch, proj, st["r"], host,
                      w["eps"], w["delta"], ESTIMATORS[args.estimator])
            if staged:
                step.set_staging(prev=(maps[(i + 1) % 2], stages[(i + 1) % 2]),
                                 nxt=(maps[i % 2], stages[i % 2]))
            step.launch()
            vk.append_token(t_kv[i][0], t_kv[i][1], n, host, st["resident_kv"],
                            st["resident_idx"], st["resident_count"], st["r"],
                            status, sketch, proj)
            if i >= W:
                hb.append(step.out["host_bytes"].clone())
                if record:
                    lists.append((step.out["fetch_idx"].clone(),
                                  step.out["fetch_count"].clone()))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        rc, bits = step.check_status()
        assert rc == 0 and int(status[0]) == 0, (rc, bits)
        fetched = hits = 0
        for j in range(1, len(lists)):
            a1, c1 = (x.cpu().numpy() for x in lists[j])
            a0, c0 = (x.cpu().numpy() for x in lists[j - 1])
            for b in range(B):
                for g in range(G):
                    u1 = a1[b, g, :c1[b, g]]
                    fetched += u1.size
                    hits += np.intersect1d(u1, a0[b, g, :c0[b, g]]).size
        return ((t1 - t0) * 1e3 / K, float(np.mean([int(x[0]) for x in hb])),
                fetched, hits)

    ms_s, hb_s, _, _ = run(True)
    ms_n, hb_n, _, _ = run(False)
    _, _, fetched, hits = run(True, record=True)
    return {
        "workload": WORKLOADS[config] + ", serving loop (decode + append per "
                    "step, correlated queries)",
        "steps": K, "ctx_tokens_start": n0,
        "ms_per_step": ms_s, "ms_per_step_no_staging": ms_n,
        "host_bytes_per_step": hb_s, "host_bytes_per_step_no_staging": hb_n,
        "host_bytes_saved_pct": 100.0 * (1.0 - hb_s / hb_n) if hb_n else 0.0,
        "staged_rows_pct": 100.0 * hits / fetched if fetched else 0.0,
        "value": B * Hq * (n0 + W + K / 2) / (ms_s * 1e-3),
    }


def dense_baselines(w, t_qs, host_kv, dev, steps, verkv_ms):
    """The pages' Dense baselines on this GPU: exact attention over the whole
    cache, held in HBM (resident) or read from pinned host memory at every
    step (offload), for the same queries; with VerKV's speedup over each."""
    import torch

    from verified_sparse_kv_amd import verkv as vk
    B, Hq, G, n = w["B"], w["Hq"], w["G"], w["n"]
    cache = B * G * n * ROW_BYTES
    out = {}
    kv_dev = host_kv.to(dev)
    k = max(1, min(steps, 10))
    for name, kv in (("resident", kv_dev), ("offload", host_kv)):
        run = vk.DenseAttention(B, Hq, G, n, dev).bind(t_qs[0], kv)
        for i in range(2):
            run.launch()
        # each call between two events on the stream: the GPU time of its
        # two kernels (the host-side call costs more than the resident
        # kernels themselves, so wall-clock would time the host)
        evs = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(k):
            run.args.q = vk._ptr(t_qs[i % len(t_qs)])
            evs[i][0].record()
            run.launch()
            evs[i][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / k
        ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / k
        out[name] = {"ms_per_step": ms, "wall_ms_per_step": wall,
                     "value": B * Hq * n / (ms * 1e-3),
                     "cache_read_gbs": cache / (ms * 1e-3) / 1e9, "steps": k}
    del kv_dev
    out["cache_bytes"] = cache
    out["verkv_speedup_vs_offload"] = out["offload"]["ms_per_step"] / verkv_ms
    out["verkv_speedup_vs_resident"] = out["resident"]["ms_per_step"] / verkv_ms
    return out


WORKLOADS = {"c2": "Qwen3-4B-shaped decode layer, 32K context",
             "c3": "Qwen3-4B-shaped decode layer, batch 16, 32K, fetch active",
             "c4": "Ministral-8B-shaped decode layer, 128K context"}


def measure(config, args, dev, headline, weights=0):
    """Compress one workload's cache with the library (and with the 2-bit
    sketch, build the sketch), then time decode steps on it. Returns (the
    measurement dict, the workload)."""
    import numpy as np
    import torch

    from verified_sparse_kv_amd import verkv as vk
    from workloads import (bf16_bits, c3_shift_queries, make_decode_workload,
                           resident_cap)

    sk2 = weights == vk.W_SKETCH2
    w = make_decode_workload(config, seed=args.seed, with_queries=False,
                             pair_profile=sk2)
    B, Hq, G, n, s, d = w["B"], w["Hq"], w["G"], w["n"], w["s"], w["d"]

    # ---- PoissonComp by the library (prefill time, untimed)
    t_tau = torch.from_numpy(w["tau"]).to(dev)
    t_k = torch.from_numpy(np.ascontiguousarray(
        w["host_kv"][:, :, :, 0, :]).view(np.int16)).to(dev)
    t_v = torch.from_numpy(np.ascontiguousarray(
        w["host_kv"][:, :, :, 1, :]).view(np.int16)).to(dev)
    cap = resident_cap(w["budget"])
    comp = vk.compress(t_tau, t_k, t_v, w["budget"], w["n_sink"], w["n_local"],
                       w["seed"], cap)
    rc, bits = vk.vkv_check_status(vk._ptr(comp["status"]), vk._stream(None))
    assert rc == 0, (rc, bits)
    sketch2, build_ms = None, None
    if sk2:  # the 2-bit sketch, built at prefill time (untimed in the step)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sketch2 = vk.sketch2_build(t_k)
        e1.record()
        torch.cuda.synchronize()
        build_ms = e0.elapsed_time(e1)
    del t_k, t_v
    counts = comp["resident_count"].cpu().numpy()

    # ---- queries: a fresh one per step
    nq = max(args.steps, 1)
    rng = np.random.default_rng([2, args.seed, 4242])
    qs = [bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
          for _ in range(nq)]
    if config == "c3":
        r_np = comp["r"].cpu().numpy()
        ridx = comp["resident_idx"].cpu().numpy()
        masks = np.zeros((B, G, n), dtype=bool)
        for b in range(B):
            for g in range(G):
                masks[b, g, ridx[b, g, :counts[b, g]]] = True
        qs = [c3_shift_queries(w, masks, r_np, step=i) for i in range(nq)]
    w["q_steps"] = qs
    t_qs = [torch.from_numpy(q.view(np.int16)).to(dev) for q in qs]
    sketch = torch.from_numpy(w["sketch"].view(np.int16)).to(dev)
    proj = torch.from_numpy(w["proj"]).to(dev)
    host_kv = torch.from_numpy(w["host_kv"].view(np.int16)).pin_memory()

    def make_step(prefetch_rows):
        st = vk.DecodeStep(B, Hq, G, n, s, cap, n, dev, n_short=128,
                           prefetch_rows=prefetch_rows)
        st.bind(t_qs[0], comp["resident_kv"], comp["resident_idx"],
                comp["resident_count"], sketch, proj, comp["r"], host_kv,
                w["eps"], w["delta"], ESTIMATORS[args.estimator], weights,
                sketch2)
        return st

    step = make_step(args.prefetch_rows)
    names = vk.decode_phase_names()
    P = len(names)

    def timed_events(count):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
        for e in evs:
            e.record()
        return evs

    # untimed warmup, then profiling steps with an event after every kernel:
    # the per-kernel breakdown and the dominant HBM-bound kernel
    for i in range(args.warmup):
        step.args.q = vk._ptr(t_qs[i % nq])
        step.set_phase_events(None)
        step.launch()
    nprof = max(3, min(args.steps, 10))
    prof = [timed_events(P + 1) for _ in range(nprof)]
    torch.cuda.synchronize()
    for i in range(nprof):
        step.args.q = vk._ptr(t_qs[i % nq])
        step.set_phase_events(prof[i])
        step.launch()
    torch.cuda.synchronize()
    ph = np.zeros(P)
    for ev in prof:
        for j in range(P):
            ph[j] += ev[j].elapsed_time(ev[j + 1])
    ph_us = ph * 1e3 / nprof
    out = step.out
    ks = out["k_star"].cpu().numpy()
    ab = (algorithmic_bytes_sketch2 if sk2 else algorithmic_bytes)(
        w, counts, int(np.sum(ks > 0)), args.estimator)
    cand = ab["kernels"]

    def solo_us(k, count):
        """Average duration of kernel k over `count` steps, from two events
        recorded by its own dispatch (no other events in those steps)."""
        j = names.index(k)
        pairs = [timed_events(2) for _ in range(count)]
        torch.cuda.synchronize()
        for i in range(count):
            step.args.q = vk._ptr(t_qs[i % nq])
            evl = [None] * (P + 1)
            evl[j], evl[j + 1] = pairs[i]
            step.set_phase_events(evl)
            step.launch()
        torch.cuda.synchronize()
        step.set_phase_events(None)
        return sum(e0.elapsed_time(e1) for e0, e1 in pairs) * 1e3 / count

    # each counted kernel timed alone (events between every kernel add gaps
    # of their own); the roofline object covers the longest-running one
    solo = {k: solo_us(k, nprof) for k in cand}
    dom = max(cand, key=lambda k: solo[k])
    di = names.index(dom)

    # timed steps, no events: the step time
    torch.cuda.synchronize()
    step.set_phase_events(None)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.args.q = vk._ptr(t_qs[i])
        step.launch()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc, bits = step.check_status()
    assert rc == 0, (rc, bits, vk.vkv_last_error())
    ms = (t1 - t0) * 1e3 / max(args.steps, 1)
    # the same steps again with events on the dominant kernel only (recorded
    # by its dispatch): its average duration on the library's stream
    pairs = [timed_events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step.args.q = vk._ptr(t_qs[i])
        evl = [None] * (P + 1)
        evl[di], evl[di + 1] = pairs[i]
        step.set_phase_events(evl)
        step.launch()
    torch.cuda.synchronize()
    t_dom = sum(e0.elapsed_time(e1) for e0, e1 in pairs) * 1e-3 / max(args.steps, 1)
    # (every row read from host memory, the read-ahead included)
    host_bytes = int(out["host_bytes"][0])
    t_gather = ph_us[names.index("fetch")] * 1e-6
    # the same steps without read-ahead: its step time, the bytes the method
    # itself fetches, and the host link's rate on them in the gather
    ra_rows = vk.vkv_decode_prefetch_rows(step.args)
    read_ahead = None
    fetched_bytes, t_gather_f = host_bytes, t_gather
    if ra_rows > 0 and not args.no_prefetch_compare:
        step0 = make_step(0)
        for i in range(max(2, min(args.warmup, 5))):
            step0.args.q = vk._ptr(t_qs[i % nq])
            step0.launch()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step0.args.q = vk._ptr(t_qs[i])
            step0.launch()
        torch.cuda.synchronize()
        ms0 = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
        fetched_bytes = int(step0.out["host_bytes"][0])
        jf = names.index("fetch")
        fp = [timed_events(2) for _ in range(nprof)]
        torch.cuda.synchronize()
        for i in range(nprof):
            step0.args.q = vk._ptr(t_qs[i % nq])
            evl = [None] * (P + 1)
            evl[jf], evl[jf + 1] = fp[i]
            step0.set_phase_events(evl)
            step0.launch()
        torch.cuda.synchronize()
        t_gather_f = sum(e0.elapsed_time(e1) for e0, e1 in fp) * 1e-3 / nprof
        read_ahead = {"rows_per_kv_head": ra_rows,
                      "ms_per_step_without": ms0,
                      "host_bytes_per_step_without": fetched_bytes,
                      "host_bytes_read_ahead_not_fetched": host_bytes - fetched_bytes,
                      "fetch_us_without": t_gather_f * 1e6,
                      "fetch_us": t_gather * 1e6}
        del step0
    ks = out["k_star"].cpu().numpy()
    paths = np.bincount(out["row_path"].cpu().numpy().ravel(), minlength=4)
    fetch_pct = 100.0 * fetched_bytes / (B * G * n * ROW_BYTES)
    units = B * Hq * n
    achieved = cand[dom] / t_dom / 1e9

    def hbm(k, v):
        t = solo[k] * 1e-6
        e = {"us": round(float(t * 1e6), 2), "bytes": int(v),
             "gbs": round(v / t / 1e9, 1),
             "frac": round(v / t / (HBM_PEAK_GBS * 1e9), 4)}
        if k in ab["intermediate"]:
            e["intermediate_bytes"] = int(ab["intermediate"][k])
        return e

    res = {
        "ms_per_step": ms,
        "value": units / (ms * 1e-3),
        "steps_per_s": 1e3 / ms,
        "config": {
            "workload": WORKLOADS[config],
            "batch": B, "q_heads": Hq, "kv_heads": G, "head_dim": d,
            "ctx_tokens": n, "budget": w["budget"], "sketch_dim": s,
            "n_sink": w["n_sink"], "n_local": w["n_local"], "eps": w["eps"],
            "delta": w["delta"], "estimator": args.estimator,
            "planning": ("2-bit RoPE-pair sketch + 128-token exact shortlist "
                         "(keys with uneven pair energy)") if sk2 else
                        "projected bf16 sketch"},
        "step_compulsory_bytes": int(ab["step"]),
        "hbm_peak_pct": 100.0 * ab["step"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "fetch_pct": fetch_pct,
        "host_bytes_per_step": host_bytes,
        "host_bytes_per_request": host_bytes / B,
        # the method's own fetch over the gather's time without read-ahead
        "host_fetch_gbs": fetched_bytes / t_gather_f / 1e9 if t_gather_f > 0 else None,
        "read_ahead": read_ahead,
        "decisions_fetching_pct": 100.0 * float(np.mean(ks > 0)),
        "decision_paths": {"no_fetch": int(paths[0]), "top_candidates": int(paths[1]),
                           "all_candidates": int(paths[2]),
                           "streaming": int(paths[3])},
        "kernel_us_profiled": {k: round(float(v), 2) for k, v in zip(names, ph_us)},
        # every counted kernel: its compulsory bytes over its own duration
        # (timed alone, like the roofline kernel)
        "kernels_hbm": {k: hbm(k, v) for k, v in cand.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "kernel_us": t_dom * 1e6,
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if sk2 else measured_traffic(
                         config, dom, args.estimator),
                     "algorithmic_bytes": cand[dom]},
    }
    if sk2:
        res["sketch_build_ms"] = build_ms
        res["sketch_bytes"] = int(B * G * (n * 8 + (n + 127) // 128 * 128))
        del res["config"]["sketch_dim"]
    res["_t_qs"], res["_host_kv"] = t_qs, host_kv
    return res, w


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the "
              "decode step shards by request and KV head with no exchange, "
              "so per-GPU throughput is the figure to scale.", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    from verified_sparse_kv_amd import verkv as vk
    main_w = vk.W_SKETCH2 if args.weights == "sketch2" else vk.W_SKETCH
    m, w = measure(args.config, args, dev, True, weights=main_w)
    t_qs, host_kv = m.pop("_t_qs"), m.pop("_host_kv")
    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "q-head*ctx-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(m["config"], parallelism="none (1 GPU)"),
    }
    for k, v in m.items():
        if k not in ("value", "ms_per_step", "config"):
            res[k] = v
    if not args.no_dense:
        res["dense_baselines"] = dense_baselines(w, t_qs, host_kv, dev,
                                                 args.steps, m["ms_per_step"])
    del t_qs, host_kv
    for extra in args.also:
        if extra == args.config:
            continue
        e, _ = measure(extra, args, dev, False)
        e.pop("_t_qs")
        e.pop("_host_kv")
        res[extra] = e
        torch.cuda.empty_cache()
    for extra in args.serving:
        res[extra + "_serving"] = serving_loop(extra, args, dev)
        torch.cuda.empty_cache()
    for extra in args.sketch2:
        if extra == args.config and main_w == vk.W_SKETCH2:
            continue
        e, _ = measure(extra, args, dev, False, weights=vk.W_SKETCH2)
        e.pop("_t_qs")
        e.pop("_host_kv")
        res[extra + "_sketch2"] = e
        torch.cuda.empty_cache()
    if not args.no_compress:
        res["compress_c5"] = compress_pass(dev, args.steps)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds,
                                           ESTIMATORS[args.estimator])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
