"""Shared helpers for the GPU parity tests: build one decode case from the
seeded workloads, run the library and the oracle on identical inputs, and
compare them by the parity rules:

* bit-exact: r, the H/L partition, the sample, resident lists and counts,
  the water level;
* exact up to documented ties: k* per query head and the fetch union per KV
  head. A head whose k* differs is tie-accepted when the oracle's own
  certificate is within 1e-5 relative of eps wherever the two stopping
  decisions differ (the stopping test is a near tie: at the library's k* if
  it stops first, else at its k* - 1) or every token between the two cut
  points has a gain within 1e-5 relative of the gain at k*;
* 2-bit sketch: the kept channels, zero points, scales and codes bit for
  bit (pairs whose float64 energies agree to 1e-9 may be chosen either
  way; the oracle then takes the library's); the shortlist exactly, except
  for tokens whose sketch score is within 1e-5 of the score magnitude of
  the oracle's last shortlisted one (fp32 against float64 scores), where the
  oracle is run again with the library's shortlist;
* numeric: eps^(L), eps^(L') and D^ within 1e-4 relative and the output
  within 1e-3 relative L2 (the stated tolerances); beta* within 1e-5
  relative of the oracle. That last bound is derived from the arithmetic:
  the library's logits are fp32 dot products (absolute error up to ~2e-6 at
  |logit| ~ 10), so every planning weight carries ~2e-6 relative error and
  the fixed point inherits it. The solver itself is checked more tightly on
  the library's own numbers: beta(L) recomputed from its lambdas must equal
  its beta* to 1e-6 of D~.
"""

import math
import sys

import numpy as np

from oracle import compress as oc
from oracle import decode as od
from oracle import sketch2 as sk2
from workloads import bf16_to_f32, c3_shift_queries, make_decode_workload

TOL_BETA = 1e-5
TOL_FIXED_POINT = 1e-6
TOL_EPS = 1e-4
TOL_D = 1e-4
TOL_O = 1e-3
TIE = 1e-5


def say(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def torch_mod():
    import torch
    return torch


def build_case(cfg, seed=0, cap_slack=64, shift_from=None, cap=None,
               mutate=None, **kw):
    """Workload + oracle compression (decode inputs shared by both sides).
    The resident capacity is the largest count plus `cap_slack`, or `cap`.
    `mutate(w)` may edit the generated arrays before compression."""
    w = make_decode_workload(cfg, seed=seed, with_queries=True, **kw)
    if mutate is not None:
        mutate(w)
    if shift_from is not None:
        w["shift_from"] = shift_from
    B, G = w["B"], w["G"]
    kf = bf16_to_f32(w["host_kv"][..., 0, :])
    vf = bf16_to_f32(w["host_kv"][..., 1, :])
    cm = oc.compress(w["tau"], kf, vf, w["budget"], w["n_sink"], w["n_local"],
                     w["seed"])
    counts = np.array([[cm[b][g]["resident_idx"].size for g in range(G)]
                       for b in range(B)])
    cap = int(counts.max()) + cap_slack if cap is None else int(cap)
    assert counts.max() <= cap
    w["cm"] = cm
    w["cap"] = cap
    w["r_all"] = np.stack([np.stack([cm[b][g]["r"] for g in range(G)])
                           for b in range(B)])
    if cfg == "c3" and w.get("shift_from", B) < B:
        res = np.zeros((B, G, w["n"]), dtype=bool)
        for b in range(B):
            for g in range(G):
                res[b, g, cm[b][g]["resident_idx"]] = True
        w["q"] = c3_shift_queries(w, res, w["r_all"])
    return w


def device_inputs(w):
    torch = torch_mod()
    B, G, n, cap, d = w["B"], w["G"], w["n"], w["cap"], w["d"]
    ridx = np.zeros((B, G, cap), dtype=np.int32)
    rkv = np.zeros((B, G, cap, 2, d), dtype=np.uint16)
    rcnt = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        for g in range(G):
            idx = w["cm"][b][g]["resident_idx"]
            ridx[b, g, :idx.size] = idx
            rkv[b, g, :idx.size] = w["host_kv"][b, g, idx]
            rcnt[b, g] = idx.size
    dev = torch.device("cuda")

    def t(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to(dev)

    return dict(
        q=t(w["q"], np.int16), resident_kv=t(rkv, np.int16),
        resident_idx=t(ridx, np.int32), resident_count=t(rcnt, np.int32),
        sketch=t(w["sketch"], np.int16), proj=t(w["proj"], np.float32),
        r=t(w["r_all"], np.float32),
        host_kv=torch.from_numpy(w["host_kv"].view(np.int16)).pin_memory())


def library_sketch2(w, dev):
    """The library's 2-bit sketch of every (request, KV head), built from a
    device copy of the cache (K rows interleaved with V rows)."""
    from verified_sparse_kv_amd import verkv as vk
    torch = torch_mod()
    B, G, n, d = w["B"], w["G"], w["n"], w["d"]
    if "sk2" not in dev:
        kv = dev["host_kv"].to("cuda").view(B, G, n, 2 * d)
        dev["sk2"] = vk.sketch2_build(kv)
        torch.cuda.synchronize()
    return dev["sk2"]


def run_library(w, dev, eps, delta, est=0, weights=0, fetch_cap=None,
                n_short=128, prefetch_rows=0):
    from verified_sparse_kv_amd import verkv as vk
    torch = torch_mod()
    step = vk.DecodeStep(w["B"], w["Hq"], w["G"], w["n"], w["s"], w["cap"],
                         fetch_cap or w["n"], torch.device("cuda"),
                         n_short=n_short, prefetch_rows=prefetch_rows)
    skt = library_sketch2(w, dev) if weights == od.W_SKETCH2 else None
    step.bind(dev["q"], dev["resident_kv"], dev["resident_idx"],
              dev["resident_count"], dev["sketch"], dev["proj"], dev["r"],
              dev["host_kv"], eps, delta, est, weights, skt)
    out = step.launch()
    rc, bits = step.check_status()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["rc"] = rc
    res["bits"] = bits
    res["n_short"] = n_short
    if skt is not None:
        res["sk2"] = {k: v.cpu().numpy() for k, v in skt.items() if k != "_ws"}
    return res


PAIR_TIE = 1e-9


def oracle_sketch2(w, b, g, lib_chan=None):
    """The oracle's sketch of (b, g). If the library kept other pairs and
    every pair in the difference has an energy within 1e-9 relative of the
    oracle's 16th largest, both choices are correct and the oracle takes
    the library's. Returns (sketch, 'tie' | 'same' | 'differs')."""
    keys = bf16_to_f32(w["host_kv"][b, g, :, 0, :])
    sk = sk2.build(keys)
    if lib_chan is None:
        return sk, "same"
    lp = np.sort(np.asarray(lib_chan)[:sk2.N_PAIRS].astype(np.int64))
    if np.array_equal(lp, sk["pairs"]):
        return sk, "same"
    e = sk["energy"]
    e16 = np.sort(e)[::-1][sk2.N_PAIRS - 1]
    diff = np.setxor1d(lp, sk["pairs"])
    if np.all(np.abs(e[diff] - e16) <= PAIR_TIE * e16):
        return sk2.with_pairs(keys, lp), "tie"
    return sk, "differs"


def oracle_sketches(w, gpu=None):
    """Oracle sketches of every (b, g) (kept in w for re-runs)."""
    B, G = w["B"], w["G"]
    out, states = [], []
    for b in range(B):
        row = []
        for g in range(G):
            lib = None if gpu is None else gpu["sk2"]["chan"][b, g]
            sk, st = oracle_sketch2(w, b, g, lib)
            row.append(sk)
            states.append(st)
        out.append(row)
    w["sk2_oracle"] = out
    return out, states


def run_oracle(w, eps, delta, est=0, weights=0, n_short=128, gpu=None):
    B, G = w["B"], w["G"]
    res_kv = [[w["cm"][b][g]["resident_kv"] for g in range(G)] for b in range(B)]
    res_idx = [[w["cm"][b][g]["resident_idx"] for g in range(G)] for b in range(B)]
    skt = None
    if weights == od.W_SKETCH2:
        skt, _ = oracle_sketches(w, gpu)
    w["n_short"] = n_short
    return od.decode_step(bf16_to_f32(w["q"]), res_kv, res_idx,
                          bf16_to_f32(w["sketch"]), w["proj"], w["r_all"],
                          bf16_to_f32(w["host_kv"]), eps, delta, est, weights,
                          sketch2=skt, n_short=n_short)


def shortlist_tie(w, b, g, lib, orc):
    """The library's shortlist differs from the oracle's: a tie when both
    have the same size and every token in the difference has an oracle score
    (largest float64 sketch logit over the group's heads) within 1e-5 of
    its score magnitude (sum of |q_c k^_c| / sqrt(d)) from the score of the
    oracle's last shortlisted token."""
    if lib.size != orc.size:
        return False
    grp = w["Hq"] // w["G"]
    sk = w["sk2_oracle"][b][g]
    qs = bf16_to_f32(w["q"][b, g * grp:(g + 1) * grp]).astype(np.float64)
    sc = np.max([sk2.sketch_logits(q, sk) for q in qs], axis=0)
    kh = np.abs(sk2.dequantize(sk).astype(np.float64))
    mag = np.max([kh @ np.abs(q[sk["chan"]]) for q in qs], axis=0) / math.sqrt(w["d"])
    t = sc[orc].min()
    diff = np.setxor1d(lib, orc)
    return bool(np.all(np.abs(sc[diff] - t) <= 1e-5 * np.maximum(mag[diff], 1e-30)))


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def binary_tie(w, b, h, hd, beta_gpu):
    """Binary shrinkage: the library moved a different number of tokens than
    the oracle. Accepted as a tie when every token whose decision differs is
    a near tie of the stopping test in the oracle's own numbers,
    |kappa - 2 beta| <= 1e-5 kappa (the library decides on fp32 weights).
    Returns the library's move count (the prefix of the oracle's order whose
    bias matches the library's), or None when it is not a tie."""
    g = h // (w["Hq"] // w["G"])
    lpos = hd["lpos"]
    r = w["r_all"][b, g][lpos].astype(np.float64)
    wt = hd["wt"]
    kappa = wt * (1.0 - r) / r
    order = np.lexsort((lpos, -kappa))
    pre = np.concatenate([[0.0], np.cumsum((wt * (1.0 - r))[order])])
    ko = int(np.sum(hd["lam"] != 1.0))
    kg = int(np.argmin(np.abs(pre - beta_gpu)))
    if abs(pre[kg] - beta_gpu) > TOL_BETA * max(beta_gpu, 1e-300):
        return None
    ks = np.arange(min(ko, kg), max(ko, kg))
    kap = kappa[order][ks]
    ok = bool(ks.size) and bool(np.all(np.abs(kap - 2.0 * pre[ks]) <= TIE * kap))
    return kg if ok else None


def kstar_tie(hd, kg, eps):
    """The library's k* differs from the oracle's. A tie when the oracle's
    own certificate is within 1e-5 relative of eps wherever the two
    stopping decisions differ (at kg when the library stops first, else at
    kg - 1: the oracle's eps^_k fall with k, so that is the farthest), or
    when every token between the two cut points has a gain within 1e-5 of
    the gain at the oracle's k*. Returns (tie, the tokens whose membership
    in F_h the tie leaves open)."""
    ko = hd["k_star"]
    if hd["order"] is None or kg <= 0 or kg > hd["order"].size:
        return False, None
    suf = hd["suffix"]
    kd = kg if kg < ko else kg - 1
    if kd < suf.size and abs(suf[kd] - eps) <= TIE * eps:
        return True, np.zeros(0, dtype=np.int64)
    lo_k, hi_k = min(kg, ko), max(kg, ko)
    g = hd["gains"][hd["order"]]
    gk = g[max(ko - 1, 0)]
    band = np.abs(g - gk) <= TIE * gk
    if np.all(band[max(lo_k - 1, 0):hi_k]):
        return True, np.sort(hd["lpos"][hd["order"][band]])
    return False, None


def rerun_group(w, b, g, eps, est, weights, binary_moves=None,
                fetch_override=None, shortlist_override=None):
    """The oracle for one (request, KV head) under the given overrides."""
    grp = w["Hq"] // w["G"]
    sl = w["cm"][b][g]
    skt = w["sk2_oracle"][b][g] if weights == od.W_SKETCH2 else None
    return od.decode_group(bf16_to_f32(w["q"][b, g * grp:(g + 1) * grp]),
                           sl["resident_kv"], sl["resident_idx"],
                           bf16_to_f32(w["sketch"][b, g]), w["proj"][g],
                           w["r_all"][b, g], bf16_to_f32(w["host_kv"][b, g]),
                           eps, w["delta"], est, weights,
                           fetch_override=fetch_override,
                           binary_moves=binary_moves, sketch2=skt,
                           n_short=w.get("n_short", 128),
                           shortlist_override=shortlist_override)


def compare(w, gpu, heads, unions, eps, est=0, weights=0, max_tie_frac=0.01):
    """Apply the parity rules; returns a summary dict. Every violation is
    collected and reported together.

    A tie-accepted row is not skipped: the oracle is run again for its KV
    head under the library's decision (binary shrinkage: the library's move
    count; k*: the oracle's own gain order cut at the library's k*), and
    eps^(L), eps^(L'), D^, the output and the fetch union are checked
    against that run at the same tolerances. At most floor(1% of the rows)
    may be tie-accepted."""
    B, Hq, G = w["B"], w["Hq"], w["G"]
    grp = Hq // G
    bad = []
    if gpu["rc"] != 0:
        bad.append(f"status rc={gpu['rc']} bits={gpu['bits']:#x}")
    ties = 0
    tie_rows = []
    worst = dict(beta=0.0, fixed_point=0.0, eps0=0.0, eps1=0.0, dhat=0.0, o=0.0)

    def check(name, err, tol, where):
        worst[name] = max(worst[name], err)
        if not err <= tol:
            bad.append(f"{name} {where}: {err:.3e} > {tol:.0e}")

    fetched = 0
    short_keys = 0
    short_ties = []
    for b in range(B):
        for g in range(G):
            hs = [heads[b][g * grp + j] for j in range(grp)]
            union = unions[b][g]
            sl_over = None
            if weights == od.W_SKETCH2:
                lib = gpu["shortlist"][b, g][:gpu["n_short"]]
                if np.any(lib[np.cumsum(lib < 0) > 0] >= 0):
                    bad.append(f"shortlist (b={b},g={g}): -1 before a position")
                lib = lib[lib >= 0].astype(np.int64)
                short_keys += lib.size
                orc = hs[0]["shortlist"]
                if not np.all(np.diff(lib) > 0):
                    bad.append(f"shortlist (b={b},g={g}) not ascending")
                if not np.array_equal(lib, orc):
                    if shortlist_tie(w, b, g, lib, orc):
                        sl_over = lib
                        short_ties.append((b, g))
                        hs, union = rerun_group(w, b, g, eps, est, weights,
                                                shortlist_override=sl_over)
                    else:
                        bad.append(f"shortlist (b={b},g={g}): library "
                                   f"{lib.size} oracle {orc.size}, sym diff "
                                   f"{np.setxor1d(lib, orc).size} (not a tie)")
            # binary shrinkage: beta (the moved tokens' bias) and ties of
            # the move count
            moves = [None] * grp
            for j in range(grp):
                h = g * grp + j
                hd, st, where = hs[j], gpu["row_stats"][b, h], f"(b={b},h={h})"
                if est == od.EST_CLIP and hd["beta_star"] > 0:
                    check("beta", _rel(st[2], hd["beta_star"]), TOL_BETA, where)
                    check("fixed_point", abs(st[3] - st[2]) / st[1],
                          TOL_FIXED_POINT, where)
                if est == od.EST_BINARY:
                    # beta(L) from the certificate pass must be the same sum
                    # (both passes apply one rule)
                    check("fixed_point", abs(st[3] - st[2]) / st[1],
                          TOL_FIXED_POINT, where)
                    bo = hd["beta_star"]
                    eb = 0.0 if bo == st[2] == 0.0 else _rel(st[2], bo)
                    if not eb <= TOL_BETA:
                        kg = binary_tie(w, b, h, hd, float(st[2]))
                        if kg is None:
                            check("beta", eb, TOL_BETA, where)
                        else:
                            moves[j] = kg
                            tie_rows.append((b, h, "binary"))
            if any(m is not None for m in moves):
                hs, union = rerun_group(w, b, g, eps, est, weights,
                                        binary_moves=moves,
                                        shortlist_override=sl_over)
            # k*: exact, or a tie scored under the library's k*
            over = [None] * grp
            open_tokens = []
            for j in range(grp):
                h = g * grp + j
                kg, ko = int(gpu["k_star"][b, h]), hs[j]["k_star"]
                if kg == ko:
                    continue
                tie, toks = kstar_tie(hs[j], kg, eps)
                if not tie:
                    bad.append(f"k* (b={b},h={h}): gpu {kg} oracle {ko} "
                               f"(not a tie)")
                    continue
                over[j] = hs[j]["lpos"][hs[j]["order"][:kg]]
                open_tokens.append(toks)
                tie_rows.append((b, h, "k*"))
            kset = [None] * grp
            if any(o is not None for o in over):
                kset = [hs[j]["suffix"][int(gpu["k_star"][b, g * grp + j])]
                        if over[j] is not None else None for j in range(grp)]
                hs, union = rerun_group(w, b, g, eps, est, weights,
                                        binary_moves=moves,
                                        fetch_override=over,
                                        shortlist_override=sl_over)
            for j in range(grp):
                h = g * grp + j
                hd, where = hs[j], f"(b={b},h={h})"
                check("eps0", _rel(float(gpu["eps_hat0"][b, h]), hd["eps_hat0"]),
                      TOL_EPS, where)
                e1 = hd["eps_hat"] if kset[j] is None else kset[j]
                check("eps1", _rel(float(gpu["eps_hat"][b, h]), e1), TOL_EPS,
                      where)
                logd_g = math.log(max(float(gpu["d_hat"][b, h]), 1e-300)) + \
                    float(gpu["log_shift"][b, h])
                logd_o = math.log(hd["d_hat"]) + hd["m"]
                check("dhat", abs(math.expm1(logd_g - logd_o)), TOL_D, where)
                o_g = gpu["out"][b, h].astype(np.float64)
                check("o", float(np.linalg.norm(o_g - hd["o"]) /
                                 np.linalg.norm(hd["o"])), TOL_O, where)
            cnt = int(gpu["fetch_count"][b, g])
            got = gpu["fetch_idx"][b, g, :cnt]
            if not np.all(np.diff(got) > 0):
                bad.append(f"fetch list (b={b},g={g}) not ascending")
            fetched += cnt
            diff = set(got.tolist()) ^ set(union.tolist())
            allowed = set(np.concatenate(open_tokens).tolist()) \
                if open_tokens else set()
            if diff - allowed:
                bad.append(f"fetch union (b={b},g={g}): gpu {cnt} oracle "
                           f"{union.size}, sym diff {len(diff)} "
                           f"({len(diff - allowed)} outside gain ties)")
    n_rows = B * Hq
    ties = len(tie_rows)
    if ties > int(max_tie_frac * n_rows):
        bad.append(f"{ties} tie-accepted rows of {n_rows}: {tie_rows}")
    want_bytes = fetched * 512 + short_keys * 256
    if int(gpu["host_bytes"][0]) != want_bytes:
        bad.append(f"host_bytes {int(gpu['host_bytes'][0])} != {want_bytes}")
    summary = dict(ties=ties, tie_rows=tie_rows, rows=n_rows, fetched=fetched,
                   worst=worst, fetch_frac=fetched / (B * G * w["n"]),
                   kstar_mean=float(np.mean(gpu["k_star"])))
    if weights == od.W_SKETCH2:
        summary.update(short_keys=short_keys, short_ties=short_ties)
    if "row_path" in gpu:
        summary["paths"] = np.bincount(gpu["row_path"].ravel(),
                                       minlength=4).tolist()
    assert not bad, "\n".join(bad[:40] + [f"... {len(bad)} problems", str(summary)])
    return summary
