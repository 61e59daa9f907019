"""Synthetic workloads shaped like the paper's decode layers.

The paper measures on RULER/LOFT with real 4B-9B GQA models; neither the
datasets nor the weights are used here. Instead, seeded inputs take the
paper's shapes (32K/128K context, GQA 4:1, head_dim 128, resident fraction
1/8..1/32, sink/local windows) with these value distributions:

* c1  tiny single head: n=1024, K/V ~ N(0,1) with 8 planted keys scaled x4,
      tau = mean attention of 4 observation queries, normalised by its max,
      4 sinks + 32 local tokens, budget n/8, sketch dim 16 (Gaussian JL,
      entries N(0, 1/16)), eps=0.1, delta=0.05.
* c2  Qwen3-4B-shaped layer: Hq=32, G=8, d=128, n=32768, B=1; keys
      k_i = sigma_i N(0, I) with sigma_i = 1 + 7 rho_i^-1.1 (rho a random
      rank permutation per KV head: heavy-tailed key norms), V ~ N(0, I);
      tau = mean attention of an 8-query window per q-head averaged over
      the group, normalised by its max; budget n/16 with 64 sinks + 64
      local; sketch dim 32 (entries N(0, 1/32)); eps=0.1, delta=0.05.
* c3  as c2 with B=16 independent caches, budget n/8, eps=0.05; requests
      8..15 get queries shifted toward 8 random non-sampled keys.
* c4  Ministral-8B-shaped: n=131072, B=4, budget n/32, 4 sinks + 128 local,
      tau_i = rho_i^-1.1 over a random permutation; keys as c2.
* c5  compression only: 36 layers x 8 KV heads x n=131072,
      tau ~ Beta(0.5, 5), 4 sinks + 256 local, eta in {1/8, 1/16, 1/32}.

With ``pair_profile`` (the workloads of the 2-bit sketch), key energy is
spread unevenly over the RoPE channel pairs (j, j + 64), as the pages'
sketch assumes: per KV head a random ranking of the 64 pairs, and pair j
scaled by (1 + rank_j)^-1/2 (normalised to unit mean square), so the 16
strongest pairs hold about 71% of the key energy.

Every array is drawn from numpy PCG64 ``default_rng([config, seed, ...])``;
K, V, sketches and queries are rounded to bfloat16 (round to nearest even)
and handed to both the library and the oracle as the same bf16 values.
"""

import math

import numpy as np

CONFIGS = {
    "c1": dict(B=1, Hq=1, G=1, d=128, n=1024, s=16, budget=128, n_sink=4,
               n_local=32, eps=0.1, delta=0.05, keys="planted", tau="obs4"),
    "c2": dict(B=1, Hq=32, G=8, d=128, n=32768, s=32, budget=2048, n_sink=64,
               n_local=64, eps=0.1, delta=0.05, keys="zipf", tau="obs8"),
    "c3": dict(B=16, Hq=32, G=8, d=128, n=32768, s=32, budget=4096,
               n_sink=64, n_local=64, eps=0.05, delta=0.05, keys="zipf",
               tau="obs8", shift_from=8, alpha=0.5),
    "c4": dict(B=4, Hq=32, G=8, d=128, n=131072, s=32, budget=4096, n_sink=4,
               n_local=128, eps=0.1, delta=0.05, keys="zipf", tau="zipf"),
}

C5 = dict(layers=36, G=8, n=131072, n_sink=4, n_local=256,
          etas=(1.0 / 8, 1.0 / 16, 1.0 / 32))

_CFG_ID = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits):
    """bfloat16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _softmax_rows(x):
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def _zipf_sigma(rng, n):
    rho = rng.permutation(n).astype(np.float64) + 1.0
    return (1.0 + 7.0 * rho ** -1.1).astype(np.float32)


def _obs_tau(rng, k, n_q):
    """Mean attention of n_q observation queries ~ N(0, I), then / max."""
    d = k.shape[-1]
    qo = rng.standard_normal((n_q, d), dtype=np.float32)
    att = _softmax_rows((qo @ k.T) / np.float32(math.sqrt(d)))
    tau = att.mean(axis=0)
    return (tau / tau.max()).astype(np.float32)


def _pair_scales(rng, d):
    """Per-channel scales with uneven RoPE-pair energy (see the module
    notes): pair j -> channels j and j + d/2."""
    h = d // 2
    rank = rng.permutation(h).astype(np.float64)
    sc = (1.0 + rank) ** -0.5
    sc /= math.sqrt(np.mean(sc ** 2))
    return np.concatenate([sc, sc]).astype(np.float32)


def make_decode_workload(cfg, seed=0, n=None, B=None, G=None, budget=None,
                         alpha=None, with_queries=True, grp=None, s=None,
                         pair_profile=False):
    """Draw one decode workload; optional overrides shrink or reshape it for
    tests (``grp`` query heads per KV head, ``s`` sketch dimension).

    Returns a dict of numpy arrays: tau [B][G][n] f32, host_kv [B][G][n][2][d]
    bf16 bits, sketch [B][G][n][s] bf16 bits, proj [G][d][s] f32,
    q [B][Hq][d] bf16 bits (None if ``with_queries`` is False), plus the scalar
    parameters. For c3 the shifted queries need the sample; call
    ``c3_shift_queries`` once the resident sets are known.
    """
    p = dict(CONFIGS[cfg])
    if n is not None:
        scale = n / p["n"]
        p["n"] = n
        p["budget"] = max(int(round(p["budget"] * scale)),
                          p["n_sink"] + p["n_local"] + 1) if budget is None \
            else budget
    if budget is not None:
        p["budget"] = budget
    if B is not None:
        p["B"] = B
    if G is not None:
        p["Hq"] = p["Hq"] // p["G"] * G
        p["G"] = G
    if alpha is not None:
        p["alpha"] = alpha
    if grp is not None:  # query heads per KV head
        p["Hq"] = p["G"] * grp
    if s is not None:  # sketch dimension
        p["s"] = s
    Bn, Hq, Gn, d, nn, s = p["B"], p["Hq"], p["G"], p["d"], p["n"], p["s"]
    grp = Hq // Gn
    cid = _CFG_ID[cfg]
    host_kv = np.empty((Bn, Gn, nn, 2, d), dtype=np.uint16)
    tau = np.empty((Bn, Gn, nn), dtype=np.float32)
    sketch = np.empty((Bn, Gn, nn, s), dtype=np.uint16)
    prng = np.random.default_rng([cid, seed, 999])
    proj = (prng.standard_normal((Gn, d, s), dtype=np.float32)
            / np.float32(math.sqrt(s))).astype(np.float32)
    for b in range(Bn):
        rng = np.random.default_rng([cid, seed, b])
        for g in range(Gn):
            if p["keys"] == "planted":
                k = rng.standard_normal((nn, d), dtype=np.float32)
                lo, hi = min(4, nn), max(min(4, nn) + 8, nn - 32)
                planted = rng.choice(np.arange(lo, hi), size=min(8, hi - lo),
                                     replace=False)
                k[planted] *= 4.0
            else:
                sig = _zipf_sigma(rng, nn)
                k = rng.standard_normal((nn, d), dtype=np.float32) * sig[:, None]
            if pair_profile:
                k = k * _pair_scales(np.random.default_rng([cid, seed, b, g, 555]), d)
            v = rng.standard_normal((nn, d), dtype=np.float32)
            kb = bf16_bits(k)
            host_kv[b, g, :, 0, :] = kb
            host_kv[b, g, :, 1, :] = bf16_bits(v)
            kf = bf16_to_f32(kb)
            if p["tau"] == "obs4":
                tau[b, g] = _obs_tau(rng, kf, 4)
            elif p["tau"] == "obs8":
                tau[b, g] = _obs_tau(rng, kf, 8 * grp)
            else:
                rho = rng.permutation(nn).astype(np.float64) + 1.0
                tau[b, g] = (rho ** -1.1).astype(np.float32)
            sketch[b, g] = bf16_bits(kf @ proj[g])
    q = None
    if with_queries:
        qrng = np.random.default_rng([cid, seed, 777])
        q = bf16_bits(qrng.standard_normal((Bn, Hq, d), dtype=np.float32))
    p.update(tau=tau, host_kv=host_kv, sketch=sketch, proj=proj, q=q,
             seed=seed, cfg=cfg, pair_profile=pair_profile)
    return p


def c3_shift_queries(w, resident_masks, r, step=0):
    """Queries for the fetch-active workload: requests >= shift_from get
    q = z + alpha sqrt(d) mean_j khat_j over 8 keys drawn from L minus S of
    the same KV head (khat = unit key); earlier requests keep q ~ N(0, I).

    ``resident_masks``: bool [B][G][n]; ``r``: float32 [B][G][n].
    """
    Bn, Hq, Gn, d = w["B"], w["Hq"], w["G"], w["d"]
    grp = Hq // Gn
    alpha = w.get("alpha", 0.5)
    first = w.get("shift_from", Bn)
    rng = np.random.default_rng([_CFG_ID[w["cfg"]], w["seed"], 555, step])
    z = rng.standard_normal((Bn, Hq, d), dtype=np.float32)
    for b in range(first, Bn):
        for h in range(Hq):
            g = h // grp
            cand = np.nonzero((r[b, g] < 1.0) & ~resident_masks[b, g])[0]
            pick = rng.choice(cand, size=min(8, cand.size), replace=False)
            kk = bf16_to_f32(w["host_kv"][b, g, pick, 0, :]).astype(np.float64)
            kh = kk / np.linalg.norm(kk, axis=1, keepdims=True)
            z[b, h] += np.float32(alpha * math.sqrt(d)) * \
                kh.mean(axis=0).astype(np.float32)
    return bf16_bits(z)


def resident_cap(budget):
    """Resident-row capacity for a budget: the budget plus eight standard
    deviations of a Poisson sample's size, plus 64."""
    return int(budget + 8 * math.sqrt(budget) + 64)


def make_c5_tau(seed=0, layers=None, G=None, n=None):
    """Beta(0.5, 5) scores for the compression pass: [layers][G][n] f32."""
    L = C5["layers"] if layers is None else layers
    Gn = C5["G"] if G is None else G
    nn = C5["n"] if n is None else n
    rng = np.random.default_rng([5, seed])
    return rng.beta(0.5, 5.0, size=(L, Gn, nn)).astype(np.float32)
